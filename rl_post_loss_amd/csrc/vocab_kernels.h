// Internal interface between the C ABI layer (abi.cpp) and the full-vocab
// reverse-KL kernels (vocab_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "loss_kernels.h"

namespace rlpl {

struct VocabArgs {
    const void* student;   // (rows, vocab) logits
    const void* teacher;   // (rows, vocab) logits
    const uint8_t* mask;   // (rows,)
    void* grad;            // (rows, vocab) d loss / d student logits (fwd+bwd only)
    float* loss;
    uint32_t* n_out;       // valid-row count or NULL
    Workspace* ws;
    int64_t rows;          // < 2^31
    int64_t vocab;         // rows * vocab < 2^62
    uint32_t chunks;       // workgroups per row (gridDim.x is a multiple of it)
    uint64_t chunk_blocks; // 32-byte blocks per piece of a row
};

constexpr int kVocabMaxChunks = 256;      // pieces per row
constexpr int kVocabMinPieceBlocks = 1024; // a piece is at least 1024 blocks (4 per lane)

// How a (rows, vocab) problem is spread over `cap` co-resident workgroups.
// Forward only (one read of each row): one workgroup per row when there are at
// least as many rows as workgroups, else rows split into pieces of at least
// kVocabMinPieceBlocks blocks, as many as fill the device.  Fused: always
// pieces of about kVocabMinPieceBlocks blocks (64 KB of both slabs at 16-bit),
// which a workgroup keeps in registers between its two passes (a longer piece,
// when a row needs more than kVocabMaxChunks pieces, is read a second time).
// The forward-only kernel keeps its own split (pieces cost it 155 -> 219 us at
// 1024 x 248320 bf16), so the two losses agree to float32 summation rounding
// rather than bit for bit when the splits differ.  Every row, wherever it
// starts, spans at most floor(vocab / per_block) + 2 blocks of per_block
// elements.
struct VocabSplit {
    int64_t chunks, chunk_blocks, groups;
};
inline VocabSplit vocab_split(int64_t rows, int64_t vocab, int elem, int64_t cap, bool fused) {
    const int64_t per_block = 32 / elem;
    const int64_t blocks = vocab % per_block == 0 ? vocab / per_block : vocab / per_block + 2;
    int64_t c = rows >= cap ? 1 : cap / rows;
    const int64_t most = (blocks + kVocabMinPieceBlocks - 1) / kVocabMinPieceBlocks;
    if (c > most || fused) c = most;
    if (c > kVocabMaxChunks) c = kVocabMaxChunks;
    if (c < 1) c = 1;
    const int64_t chunk_blocks = (blocks + c - 1) / c;
    const int64_t groups = cap / c < rows ? cap / c : rows;
    return VocabSplit{c, chunk_blocks, groups};
}

// Kernel variants: forward only; fwd+bwd with each piece kept in registers
// between its two passes (pieces of at most kVocabResidentBlocks blocks, four
// per lane); fwd+bwd reading its piece a second time (longer pieces).
enum { kVocabFwd = 0, kVocabResident = 1, kVocabStream = 2 };
constexpr int64_t kVocabResidentBlocks = 1024;

inline int vocab_mode(bool write_grad, int64_t chunk_blocks) {
    return !write_grad ? kVocabFwd : chunk_blocks <= kVocabResidentBlocks ? kVocabResident : kVocabStream;
}

// Kernel for <dtype, mode>, or nullptr.
const void* pick_vocab_kernel(int dtype, int mode);

}  // namespace rlpl
