// Internal interface between the C ABI layer (abi.cpp) and the selective
// log-probability kernels (logprob_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rlpl {

// Tiles of the MFMA contraction: 256 x 256 outputs per workgroup (eight
// wavefronts of 128 x 64), K in 64-deep stages through a 128 KB LDS ring
// (two stages); one workgroup per compute unit.
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;               // stage depth (also the split-K granule)
constexpr int kGemmWavesM = 2;            // wavefronts along M
constexpr int kGemmWavesN = 4;            // and along N
constexpr int kGemmThreads = 64 * kGemmWavesM * kGemmWavesN;
constexpr int kGemmDynLds = 128 * 1024;   // dynamic LDS bytes per workgroup (the ring)
constexpr int kLogprobChunk = 1024;       // rows of logits gradient formed at a time (backward)
constexpr int kSplitK = 4;                // K splits of the hidden-gradient contraction

enum { kEpiLse = 0, kEpiDlogits = 1, kEpiSplit = 2, kEpiAccum = 3 };

// C = A . B with A (M x K) and B (K x N), bf16/fp16 operands, fp32 accumulation.
// A_KCONTIG: element (m, k) of A at a[m * lda + k], else at a[k * lda + m];
// B_KCONTIG: element (k, n) of B at b[n * ldb + k], else at b[k * ldb + n].
struct GemmArgs {
    const void* a;
    const void* b;
    int64_t lda, ldb;
    int32_t M, N, K;
    int32_t k_split;           // K range per blockIdx.z (kEpiSplit), else K
    uint32_t tiles_m, tiles_n;
    // epilogue operands
    void* c;                   // dlogits (dtype), split partials (fp32, z-major) or the fp32 accumulator
    int64_t ldc;
    int32_t accumulate;        // kEpiAccum: add to c (1) or overwrite it (0)
    const void* bias;          // (N) in the operand dtype, or NULL (kEpiLse, kEpiDlogits)
    const int64_t* targets;    // (M) (kEpiLse, kEpiDlogits)
    const float* lse;          // (M) (kEpiDlogits)
    const float* grad;         // (M) (kEpiDlogits)
    float* part;               // (M, tiles_n, 2) per-tile (max, sum exp) (kEpiLse)
    float* target_logit;       // (M) (kEpiLse)
    float* col_part;           // (tiles_m, N) per-tile column sums of the logits gradient, or NULL (kEpiDlogits)
};

const void* pick_gemm_kernel(int dtype, int epi, bool a_kcontig, bool b_kcontig);

// Per-row log-sum-exp from the per-tile partials, and the target log-probability.
struct LseArgs {
    const float* part;         // (rows, tiles, 2)
    const float* target_logit; // (rows); read only where the target is in [0, vocab)
    const int64_t* targets;    // (rows)
    float* logp;               // (rows): NaN where the target is outside [0, vocab)
    float* lse;                // (rows) or NULL
    int64_t vocab;
    int32_t rows, tiles;
};
const void* lse_combine_kernel();

// Sum of kSplitK fp32 partial planes (rows, cols) in split order, written in the dtype.
struct SplitSumArgs {
    const float* part;
    void* out;
    int64_t plane;             // rows * cols
    int32_t splits;
};
const void* pick_split_sum_kernel(int dtype);

// Sums of `rows` per-tile column partials (rows, cols) fp32 into an fp32 vector (add or overwrite), in row order.
struct ColSumArgs {
    const float* x;
    float* out;
    int32_t rows, cols, accumulate;
};
const void* col_sum_kernel();

}  // namespace rlpl
