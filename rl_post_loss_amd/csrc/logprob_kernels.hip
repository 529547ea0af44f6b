// Selective log-probabilities on gfx950 (MI355X) matrix cores: the step
// upstream of the policy losses (page "Add SM100 CuTe DSL GRPO fast path",
// section "Summary": one large matrix multiplication per group of up to 1024
// tokens, the cross-entropy done in place, full logits never kept, FP32
// weight-gradient accumulation across chunks).
//
// Forward: logits tiles z = hidden . weight^T (+ bias) come out of the MFMA
// contraction and never leave the chip: each 256 x 256 tile's epilogue
// reduces its rows to (max, sum exp(z - max)) partials and picks out the
// target's logit; a small kernel combines a row's partials into its
// log-sum-exp and log-probability.
// Backward (per chunk of up to 1024 tokens): the same contraction recomputes
// the logits and its epilogue writes dz = g (onehot - exp(z - lse)) in the
// operand dtype to a workspace; d hidden = dz . weight (split-K, fp32
// partials summed in split order) and d weight (+)= dz^T . hidden (fp32,
// one owner per element) are two more contractions of the same kernel with
// transposed operand layouts; d bias is a column sum of dz.
//
// The contraction: 512 threads (2 x 4 wavefronts), a 256 x 256 output tile,
// each wavefront a 128 x 64 block of eight v_mfma_f32_32x32x16 accumulators
// held in VGPRs; one workgroup per compute unit.  K advances through a 128 KB
// ring of two 64-deep LDS stages filled by buffer-to-LDS copies (one in
// flight while the other is consumed; copies past the operand's end read as
// zeros).  K-contiguous operands are read from LDS as
// one 16-byte fragment per lane; MN-contiguous ones with transposing 8-byte
// LDS reads.  Blocks are mapped so that each XCD works on a contiguous run of
// tiles (shared weight panels stay in its L2).  The tile and wave grid are
// the constants of logprob_kernels.h; the code holds for other grids whose
// wavefront blocks are multiples of 32 x 32.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "device_common.h"
#include "logprob_kernels.h"
#include "loss_kernels.h"

namespace rlpl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// One v_mfma_f32_32x32x16 of the operand type (tag argument selects bf16 or fp16).
template <typename U> struct Mfma {
    static __device__ __forceinline__ floatx16 run(uint4 a, uint4 b, floatx16 c, __bf16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx16 run(uint4 a, uint4 b, floatx16 c, _Float16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

template <typename T> __device__ __forceinline__ float to_f(T x) { return float(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return T(x); }

constexpr int kGemmWaves = kGemmWavesM * kGemmWavesN;
constexpr int kWaveM = kGemmBM / kGemmWavesM;   // rows of C per wavefront
constexpr int kWaveN = kGemmBN / kGemmWavesN;   // columns of C per wavefront
constexpr int kFragM = kWaveM / 32;      // 32 x 32 MFMA tiles per wavefront, rows
constexpr int kFragN = kWaveN / 32;      // and columns
constexpr float kLog2eG = 1.4426950408889634f;

static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "32 x 32 matrix tiles");
static_assert(kGemmBN == 256 && kGemmBM <= kGemmThreads && kGemmBN <= kGemmThreads,
              "the epilogues use one thread per tile column / row");
static_assert(kWaveM == 64 || kWaveM == 128, "log-sum-exp partial layout");

// LDS layout of one R x BK operand tile (R = kGemmBM or kGemmBN rows, BK the stage depth),
// filled by 16-byte global->LDS copies (each wavefront copy writes 1 KB
// contiguously: lane l's 16 bytes at +16*l), with an XOR swizzle of 16-byte
// chunks that keeps the matrix-core fragment reads free of bank conflicts.
// A 16-byte read serves 16 lanes per pass over all 64 banks (256 bytes), so
// the 16 rows a pass reads must spread over distinct 16-byte bank groups.
//
// K-contiguous operand (element (r, k) at x[r*ld + k]): row r is 2 BK bytes,
// kC = BK / 8 chunks; chunk c (elements 8c..8c+7) sits in slot
// c ^ swizzle(r).  64-byte rows (BK = 32): rows four apart share banks,
// swizzle (r >> 2) & 3 (measured free of bank conflicts on gfx950; (r >> 1) & 3
// had 2-way conflicts).  128-byte rows (BK = 64): rows two apart share
// banks, swizzle (r >> 1) & 7.  Fragment reads are one 16-byte read per lane;
// a copy covers 1024 / (2 BK) whole rows, so it reads full 64- or 128-byte
// row segments (the 128-byte ones copy about 1.5x faster from cache,
// measured).
//
// MN-contiguous operand (element (r, k) at x[k*ld + r]): blocks of 64 r by
// BK K rows; in a block, K row k is 128 bytes and its chunk c (r = 8c..8c+7 of
// the block) sits in slot c ^ (4 ((k >> 1) & 1)), so that a copy brings 8 K
// rows of 128 bytes.  Fragment reads are two transposing 8-byte reads per
// lane (ds_read_b64_tr_b16); a pass of 32 lanes reads 4 K rows of 32 r, and
// the swizzle puts K rows two apart on the other half of the banks.
// The stages of depth BK: sizes, copy counts and LDS layouts.
template <int BK>
struct Stage {
    static constexpr int kBytesA = kGemmBM * BK * 2;   // A tile of one stage
    static constexpr int kBytesB = kGemmBN * BK * 2;   // B tile of one stage
    static constexpr int kBytes = kBytesA + kBytesB;
    static constexpr int kCount = kGemmDynLds / kBytes;   // ring slots
    static constexpr int kDmaA = kBytesA / 1024 / kGemmWaves;   // 1 KB copies per wavefront for the A tile
    static constexpr int kDmaB = kBytesB / 1024 / kGemmWaves;   // and for the B tile
    static constexpr int kC = BK / 8;                 // 16-byte chunks per K-contiguous row
    static constexpr int kRowsPerCopy = 1024 / (2 * BK);
    static_assert(kC == 4 || kC == 8, "32- or 64-deep stages");
    static_assert(kCount >= 2 && kCount * kBytes == kGemmDynLds, "LDS ring");
    static_assert(kDmaA * kGemmWaves * 1024 == kBytesA && kDmaB * kGemmWaves * 1024 == kBytesB, "whole copies");
    static __device__ __forceinline__ int kc_swizzle(int r) { return kC == 4 ? (r >> 2) & 3 : (r >> 1) & 7; }
    static __device__ __forceinline__ int kc_offset(int r, int c) { return r * (2 * BK) + 16 * (c ^ kc_swizzle(r)); }
    static __device__ __forceinline__ int mn_swizzle(int k) { return ((k >> 1) & 1) << 2; }
    static __device__ __forceinline__ int mn_offset(int k, int r) {
        return (r >> 6) * (128 * BK) + k * 128 + 16 * (((r & 63) >> 3) ^ mn_swizzle(k)) + 2 * (r & 7);
    }
};

// Per-lane source of the wavefront's 1 KB copies of one operand tile: copy q
// (0 .. R * BK / 512 - 1; each wavefront issues 1/kGemmWaves of them) of
// the tile whose first element is (r0, k0).  Returns the byte offset of the
// lane's 16 bytes from that element (the copy goes through a buffer descriptor
// based there), or kOutOfRange for a chunk of rows past R or of K at or past
// ke, which the buffer unit reads as zeros.  A chunk that starts before ke is
// read whole: the caller guarantees that the elements past ke in it are zeros
// or that ke is a multiple of 8.  Offsets stay below 2 * (BK + 256 * ld)
// bytes.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
constexpr int kBufferRecords = 0x7FFFFFF0;

template <bool KCONTIG, int BK>
__device__ __forceinline__ uint32_t dma_source(int q, int lane, uint32_t ld, int R, int ke, int r0, int k0) {
    using St = Stage<BK>;
    if constexpr (KCONTIG) {
        const int r = St::kRowsPerCopy * q + lane / St::kC;
        const int c = (lane % St::kC) ^ St::kc_swizzle(r);
        const bool ok = r0 + r < R && k0 + 8 * c < ke;
        return ok ? 2u * (uint32_t(r) * ld + uint32_t(8 * c)) : kOutOfRange;
    } else {
        const int cb = q / (BK / 8), k = 8 * (q % (BK / 8)) + (lane >> 3);
        const int c = (lane & 7) ^ St::mn_swizzle(k);
        const int rr = 64 * cb + 8 * c;
        const bool ok = r0 + rr < R && k0 + k < ke;
        return ok ? 2u * (uint32_t(k) * ld + uint32_t(rr)) : kOutOfRange;
    }
}

// One 16-byte copy per lane from a buffer (offset `off`) into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t src, uint32_t off, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, int(off), 0, 0, 0);
}

// Raw buffer descriptor over the memory from p on (gfx9 raw-buffer flags).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, kBufferRecords, 0x00020000);
}

// s_waitcnt immediate that waits for vmcnt <= v (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int v) { return 0x0F70 | (v & 15) | ((v >> 4) << 14); }

// Wait until at most `pending` (compile-time) stages of this wavefront's copies
// (kDmaA + kDmaB of Stage<BK> per stage) are in flight, then meet the other
// wavefronts.
template <int PENDING, int BK>
__device__ __forceinline__ void wait_stages() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PENDING * (Stage<BK>::kDmaA + Stage<BK>::kDmaB)));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Matrix-core fragments of stage tile t for wavefront row/column block wb (of
// WT rows), 32-row tile f, K step kk (16 K): the eight K values lane l needs
// for row/column wb*WT + f*32 + l%32, K 8*(l/32) .. +8.
template <bool KCONTIG, int WT, int BK>
__device__ __forceinline__ uint4 fragment(const uint16_t* __restrict__ t, int wb, int f, int kk, int lane) {
    if constexpr (KCONTIG) {
        const int r = wb * WT + f * 32 + (lane & 31);
        return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(t) + Stage<BK>::kc_offset(r, kk * 2 + (lane >> 5)));
    } else {
        // 16-lane group G: columns 16*(G%2) .. +16 of the 32-wide tile, K base 8*(G/2).
        // Input lane q = 4j + t of the group points at K row kbase + j, columns 4t .. 4t+3;
        // output lane i then holds K rows kbase .. kbase+3 of column i.
        const int G = lane >> 4, q = lane & 15;
        const int r = wb * WT + f * 32 + 16 * (G & 1) + 4 * (q & 3);
        const int k = kk * 16 + 8 * (G >> 1) + (q >> 2);
        typedef short v4s __attribute__((ext_vector_type(4)));
        const char* base = reinterpret_cast<const char*>(t);
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(base + Stage<BK>::mn_offset(k, r)));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(base + Stage<BK>::mn_offset(k + 4, r)));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
}

// Column of partial p's row in the log-sum-exp partial layout: rows XOR p % 32
// (32 writing lanes, one row: distinct banks), and the four 32-partial shares
// of a row, read at once by the row's four merging threads, moved apart by
// 4 (p / 32) (16 lanes of four rows: distinct banks).
__device__ __forceinline__ int part_swizzle(int p) { return (p & 31) ^ ((p >> 5) << 2); }

// The value of the neighbouring lane (lane ^ 1), by a DPP quad permute [1, 0, 3, 2].
__device__ __forceinline__ float swap_pair(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// The value of lane ^ X within a quad (X = 1: permute [1, 0, 3, 2]; X = 2: [2, 3, 0, 1]).
template <int X>
__device__ __forceinline__ float quad_xor(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), X == 1 ? 0xB1 : 0x4E, 0xF, 0xF, false));
}

// XCD-aware tile order: consecutive block indices go to different XCDs, so
// XCD x (block % 8) takes a contiguous run of the (split, tile) pairs, split
// slowest (a split-K product gives each split's tiles to whole XCDs).
// Within the run, tiles come in groups of kTileGroupM M tiles by all N
// tiles, M varying fastest inside a group: the 32 tiles an XCD runs at once
// form a 4 x 8 block that shares 4 A panels and 8 B panels in its L2 (M
// fastest over the whole range would, for a tall product, put 32 A panels
// beside one B panel).  b is the linear block index over splits blocks of
// tiles_m * tiles_n.
constexpr uint32_t kTileGroupM = 4;
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t tiles_m, uint32_t tiles_n, uint32_t splits, uint32_t& tm,
                                        uint32_t& tn, uint32_t& split) {
    const uint32_t T = tiles_m * tiles_n, all = T * splits;
    const uint32_t x = b & 7u, idx = b >> 3;
    const uint32_t q = all >> 3, r = all & 7u;
    const uint32_t v = (x < r ? x * (q + 1u) : r * (q + 1u) + (x - r) * q) + idx;
    split = v / T;
    const uint32_t t = v % T;
    const uint32_t group = t / (kTileGroupM * tiles_n), in = t % (kTileGroupM * tiles_n);
    const uint32_t m_first = group * kTileGroupM;
    const uint32_t rows = tiles_m - m_first < kTileGroupM ? tiles_m - m_first : kTileGroupM;
    tm = m_first + in % rows;
    tn = in / rows;
}

}  // namespace

template <typename T, int EPI, bool A_KCONTIG, bool B_KCONTIG>
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_kernel(const GemmArgs g) {
    extern __shared__ __attribute__((aligned(1024))) uint16_t ring[];   // St::kCount x (A tile, B tile)
    constexpr int BK = kGemmBK;   // stage depth
    using St = Stage<BK>;
    __shared__ float red_a[kGemmWavesM][kGemmBN];
    __shared__ int tgt_col[kGemmBM];

    uint32_t tm, tn, split;
    tile_of(blockIdx.x + gridDim.x * blockIdx.z, g.tiles_m, g.tiles_n, gridDim.z, tm, tn, split);
    const int m0 = int(tm) * kGemmBM, n0 = int(tn) * kGemmBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / kGemmWavesN, wn = wave % kGemmWavesN;
    const int kb = EPI == kEpiSplit ? int(split) * g.k_split : 0;
    const int ke = EPI == kEpiSplit ? min(g.K, kb + g.k_split) : g.K;
    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.a);
    const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.b);

    // Accumulator element e of tile (i, j) is tile row wm*kWaveM + i*32 + 8*(e/4) +
    // 4*(lane/32) + e%4 and column wn*kWaveN + j*32 + lane%32.
    auto row_of_e = [&](int i, int e) { return wm * kWaveM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); };
    auto col_of_j = [&](int j) { return wn * kWaveN + j * 32 + (lane & 31); };

    floatx16 acc[kFragM][kFragN];
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nst = kb < ke ? (ke - kb + BK - 1) / BK : 0;
    // This wavefront's copies of stage s (St::kDmaA of the A tile, St::kDmaB of the B tile,
    // 1 KB each) into ring slot s % stages.  Copies of a stage past the last are all
    // out of range (zeros).
    auto issue = [&](int s) {
        const int k0 = kb + s * BK;
        char* slot = reinterpret_cast<char*>(ring) + (s % St::kCount) * St::kBytes;
        // first element (tile row 0, K k0) of each operand's tile
        const __amdgpu_buffer_rsrc_t a0 =
            buffer_at(A + (A_KCONTIG ? int64_t(m0) * g.lda + k0 : int64_t(k0) * g.lda + m0));
        const __amdgpu_buffer_rsrc_t b0 =
            buffer_at(B + (B_KCONTIG ? int64_t(n0) * g.ldb + k0 : int64_t(k0) * g.ldb + n0));
#pragma unroll
        for (int u = 0; u < St::kDmaA; ++u) {
            const int q = wave * St::kDmaA + u;
            dma16(a0, dma_source<A_KCONTIG, BK>(q, lane, uint32_t(g.lda), g.M, ke, m0, k0), slot + q * 1024);
        }
#pragma unroll
        for (int u = 0; u < St::kDmaB; ++u) {
            const int q = wave * St::kDmaB + u;
            dma16(b0, dma_source<B_KCONTIG, BK>(q, lane, uint32_t(g.ldb), g.N, ke, n0, k0),
                  slot + St::kBytesA + q * 1024);
        }
    };
    // Step s: wait for stage s's copies (later stages may stay in flight), meet the
    // other wavefronts (so every one is done with stage s-1), refill stage s-1's
    // slot with stage s + kCount - 1, then the matrix instructions of stage s, one
    // 16-deep K step at a time.
    if (nst > 0) {
        for (int s = 0; s < St::kCount - 1; ++s) issue(s);
        for (int s = 0; s < nst; ++s) {
            wait_stages<St::kCount - 2, BK>();
            issue(s + St::kCount - 1);
            const uint16_t* at = ring + (s % St::kCount) * (St::kBytes / 2);
            const uint16_t* bt = at + St::kBytesA / 2;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                uint4 af[kFragM], bf[kFragN];
#pragma unroll
                for (int i = 0; i < kFragM; ++i) af[i] = fragment<A_KCONTIG, kWaveM, BK>(at, wm, i, kk, lane);
#pragma unroll
                for (int j = 0; j < kFragN; ++j) bf[j] = fragment<B_KCONTIG, kWaveN, BK>(bt, wn, j, kk, lane);
#pragma unroll
                for (int i = 0; i < kFragM; ++i)
#pragma unroll
                    for (int j = 0; j < kFragN; ++j) acc[i][j] = Mfma<uint16_t>::run(af[i], bf[j], acc[i][j], T());
            }
        }
    }
    __syncthreads();

    if constexpr (EPI == kEpiSplit || EPI == kEpiAccum) {
        float* __restrict__ C = static_cast<float*>(g.c);
        if constexpr (EPI == kEpiSplit) C += int64_t(split) * g.M * g.ldc;
        if (EPI == kEpiAccum && g.accumulate) {
            // C += acc, one 32-row tile at a time: its 64 reads are issued together.
            if (m0 + wm * kWaveM + kWaveM <= g.M && n0 + wn * kWaveN + kWaveN <= g.N) {
                // the wavefront's kWaveM x kWaveN block lies inside C
#pragma unroll
                for (int i = 0; i < kFragM; ++i) {
                    float* base = C + int64_t(m0 + row_of_e(i, 0)) * g.ldc + n0 + col_of_j(0);
                    float old[16][kFragN];
#pragma unroll
                    for (int e = 0; e < 16; ++e)
#pragma unroll
                        for (int j = 0; j < kFragN; ++j) old[e][j] = base[int64_t(8 * (e >> 2) + (e & 3)) * g.ldc + 32 * j];
#pragma unroll
                    for (int e = 0; e < 16; ++e)
#pragma unroll
                        for (int j = 0; j < kFragN; ++j)
                            base[int64_t(8 * (e >> 2) + (e & 3)) * g.ldc + 32 * j] = old[e][j] + acc[i][j][e];
                }
                return;
            }
            // edge blocks: reads clamped to a valid element outside M x N, where nothing is stored
#pragma unroll
            for (int i = 0; i < kFragM; ++i) {
                float old[16][kFragN];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = min(m0 + row_of_e(i, e), g.M - 1);
#pragma unroll
                    for (int j = 0; j < kFragN; ++j)
                        old[e][j] = C[int64_t(row) * g.ldc + min(n0 + col_of_j(j), g.N - 1)];
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + row_of_e(i, e);
                    if (row >= g.M) continue;
#pragma unroll
                    for (int j = 0; j < kFragN; ++j) {
                        const int col = n0 + col_of_j(j);
                        if (col < g.N) C[int64_t(row) * g.ldc + col] = old[e][j] + acc[i][j][e];
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + row_of_e(i, e);
                if (row >= g.M) continue;
#pragma unroll
                for (int j = 0; j < kFragN; ++j) {
                    const int col = n0 + col_of_j(j);
                    if (col < g.N) C[int64_t(row) * g.ldc + col] = acc[i][j][e];
                }
            }
        return;
    }

    // Logits epilogues: z = acc + bias; columns past N are -inf.
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    float bcol[kFragN];
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
        const int col = n0 + col_of_j(j);
        bcol[j] = col < g.N ? (bias ? to_f<T>(bias[col]) : 0.0f) : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] += bcol[j];

    if constexpr (EPI == kEpiDlogits) {
        // dz = g (onehot - exp(z - lse)), exact zeros outside the M x N range, one
        // 32-row tile at a time, with the rows' lse, g and target column staged in
        // LDS.  Stores: lanes 2c and 2c+1 (columns c, c+1 of a 32-column group)
        // swap one value (DPP quad permute) so that each writes two adjacent
        // columns of one row (rows r and r+1 of elements e, e+1) as a 32-bit word.
        float* row_lse = reinterpret_cast<float*>(ring);
        float* row_g = row_lse + kGemmBM;
        int* row_tc = reinterpret_cast<int*>(row_g + kGemmBM);
        if (threadIdx.x < kGemmBM) {
            const int row = m0 + int(threadIdx.x);
            const bool in = row < g.M;
            const int64_t t = in ? g.targets[row] : -1;
            row_lse[threadIdx.x] = in ? g.lse[row] : 0.0f;
            row_g[threadIdx.x] = in ? g.grad[row] : 0.0f;
            row_tc[threadIdx.x] = (t >= n0 && t < n0 + kGemmBN && t < g.N) ? int(t - n0) : -1;
        }
        __syncthreads();
        T* __restrict__ D = static_cast<T*>(g.c);
        const bool odd = lane & 1;
        float csum[kFragN] = {};
#pragma unroll
        for (int i = 0; i < kFragM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                float dz[2][kFragN];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = row_of_e(i, e + h);
                    const bool in = m0 + r < g.M;
                    const float l = row_lse[r], gr = row_g[r];
                    const int tc = row_tc[r];
#pragma unroll
                    for (int j = 0; j < kFragN; ++j) {
                        const int c = col_of_j(j);
                        const float p = __builtin_amdgcn_exp2f((acc[i][j][e + h] - l) * kLog2eG);
                        dz[h][j] = (in && n0 + c < g.N) ? gr * ((c == tc ? 1.0f : 0.0f) - p) : 0.0f;
                        csum[j] += dz[h][j];
                    }
                }
                const int row = m0 + row_of_e(i, e) + (odd ? 1 : 0);
#pragma unroll
                for (int j = 0; j < kFragN; ++j) {
                    const float got = swap_pair(odd ? dz[0][j] : dz[1][j]);
                    const float lo = odd ? got : dz[0][j];
                    const float hi = odd ? dz[1][j] : got;
                    const int col = n0 + col_of_j(j) - (odd ? 1 : 0);   // even column of the pair
                    // pairs up to the row pitch (a multiple of 8): the padding columns past N
                    // get zeros, which the hidden-gradient contraction reads as a K tail
                    if (row < g.M && col < g.ldc)
                        *reinterpret_cast<uint32_t*>(D + int64_t(row) * g.ldc + col) = Elem<T>::pack(lo, hi);
                }
            }
        }
        if (g.col_part) {
            // Column sums of dz over the tile's rows (fixed order: the lane's rows,
            // the two lane halves, the row wavefronts in order).
#pragma unroll
            for (int j = 0; j < kFragN; ++j) {
                const float s = csum[j] + __shfl_xor(csum[j], 32, 64);
                if (lane < 32) red_a[wm][col_of_j(j)] = s;
            }
            __syncthreads();
            const int col = n0 + int(threadIdx.x);
            if (threadIdx.x < kGemmBN && col < g.N) {
                float t = red_a[0][threadIdx.x];
#pragma unroll
                for (int w = 1; w < kGemmWavesM; ++w) t += red_a[w][threadIdx.x];
                g.col_part[int64_t(tm) * g.N + col] = t;
            }
        }
        return;
    }

    // kEpiLse: per row of the tile, (max, sum exp(z - max)) over its 256 columns, and
    // the target logit.  Each lane reduces its own kFragN columns of a row; the
    // kGemmWavesN * 32 partials of a row (column wavefronts x 32 lanes) meet in LDS,
    // laid out [partial p][row ^ part_swizzle(p)] so that both the writes (32
    // lanes, one row) and the reads (four threads per row) are free of bank
    // conflicts; the row's threads then merge them in a fixed order.  When the
    // partials of all rows do not fit in the ring, the row wavefronts take turns.
    constexpr int kParts = kGemmWavesN * 32;
    constexpr int kRounds = kParts * kGemmBM * 8 <= kGemmDynLds ? 1 : kGemmWavesM;
    constexpr int kRoundRows = kGemmBM / kRounds;
    constexpr int kQ = kGemmThreads / kRoundRows;       // threads merging one row's partials
    constexpr int kShare = kParts / kQ;
    static_assert((kQ == 2 || kQ == 4) && kShare * kQ == kParts, "row merge split");
    float2* parts = reinterpret_cast<float2*>(ring);   // kParts x kRoundRows float2, inside the ring
    static_assert(kParts * kRoundRows * 8 <= kGemmDynLds && kRoundRows % 32 == 0 && kParts <= 256,
                  "partials fit; part_swizzle stays below 32");
    if (threadIdx.x < kGemmBM) {
        const int row = m0 + int(threadIdx.x);
        const int64_t t = row < g.M ? g.targets[row] : -1;
        tgt_col[threadIdx.x] = (t >= n0 && t < n0 + kGemmBN && t < g.N) ? int(t - n0) : -1;
    }
    const int pidx = wn * 32 + (lane & 31);
    const int my_round = wm * kRounds / kGemmWavesM;
#pragma unroll
    for (int w = 0; w < kRounds; ++w) {
        __syncthreads();                                // tgt_col written; parts free
        if (my_round == w) {
#pragma unroll
            for (int i = 0; i < kFragM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = row_of_e(i, e);
                    float m = acc[i][0][e];
#pragma unroll
                    for (int j = 1; j < kFragN; ++j) m = fmaxf(m, acc[i][j][e]);
                    float sum = 0.0f;
                    if (m != -__builtin_inff()) {
#pragma unroll
                        for (int j = 0; j < kFragN; ++j) sum += __builtin_amdgcn_exp2f((acc[i][j][e] - m) * kLog2eG);
                    }
                    const int rr = r - w * kRoundRows;
                    parts[pidx * kRoundRows + (rr ^ part_swizzle(pidx))] = make_float2(m, sum);
                    const int tc = tgt_col[r];
#pragma unroll
                    for (int j = 0; j < kFragN; ++j)
                        if (col_of_j(j) == tc && m0 + r < g.M) g.target_logit[m0 + r] = acc[i][j][e];
                }
        }
        __syncthreads();
        {
            // kQ neighbouring threads per row, each over a 1/kQ share of the partials;
            // the row maximum is their common maximum, the sum adds the shares in pairs
            // ((0 + 1) + (2 + 3)), so the order is fixed.
            const int rr = threadIdx.x / kQ, qq = threadIdx.x % kQ, row = m0 + w * kRoundRows + rr;
            float M = -__builtin_inff();
            for (int q = qq * kShare; q < (qq + 1) * kShare; ++q)
                M = fmaxf(M, parts[q * kRoundRows + (rr ^ part_swizzle(q))].x);
            M = fmaxf(M, quad_xor<1>(M));
            if constexpr (kQ == 4) M = fmaxf(M, quad_xor<2>(M));
            float S = 0.0f;
            for (int q = qq * kShare; q < (qq + 1) * kShare; ++q) {
                const float2 v = parts[q * kRoundRows + (rr ^ part_swizzle(q))];
                S += v.y * __builtin_amdgcn_exp2f((v.x - M) * kLog2eG);
            }
            S += quad_xor<1>(S);
            if constexpr (kQ == 4) S += quad_xor<2>(S);
            if (qq == 0 && row < g.M)
                reinterpret_cast<float2*>(g.part)[int64_t(row) * g.tiles_n + tn] = make_float2(M, S);
        }
    }
}

// One workgroup per row: the row's log-sum-exp from its per-tile partials
// (fixed order: strided per thread, then the workgroup tree), and the
// target's log-probability.
__global__ void __launch_bounds__(kThreads) lse_combine(const LseArgs a) {
    __shared__ float red[kWaves];
    const int row = blockIdx.x;
    const float2* p = reinterpret_cast<const float2*>(a.part) + int64_t(row) * a.tiles;
    float m = -__builtin_inff();
    for (int t = threadIdx.x; t < a.tiles; t += kThreads) m = fmaxf(m, p[t].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, red[i]);
    float s = 0.0f;
    for (int t = threadIdx.x; t < a.tiles; t += kThreads)
        s += p[t].y * __builtin_amdgcn_exp2f((p[t].x - M) * kLog2eG);
    s = block_sum(s, red);
    if (threadIdx.x == 0) {
        const float lse = M + __builtin_amdgcn_logf(s) * 0.6931471805599453f;
        const int64_t t = a.targets[row];
        a.logp[row] = (t >= 0 && t < a.vocab) ? a.target_logit[row] - lse : __builtin_nanf("");
        if (a.lse) a.lse[row] = lse;
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads) split_sum(const SplitSumArgs a) {
    for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < a.plane; i += int64_t(gridDim.x) * kThreads) {
        float s = 0.0f;
        for (int z = 0; z < a.splits; ++z) s += a.part[int64_t(z) * a.plane + i];
        static_cast<T*>(a.out)[i] = from_f<T>(s);
    }
}

__global__ void __launch_bounds__(kThreads) col_sum(const ColSumArgs a) {
    const int col = blockIdx.x * kThreads + threadIdx.x;
    if (col >= a.cols) return;
    float s = 0.0f;
    for (int r = 0; r < a.rows; ++r) s += a.x[int64_t(r) * a.cols + col];
    a.out[col] = a.accumulate ? a.out[col] + s : s;
}

// ----------------------------------------------------------------------------- host-side table

template <typename T>
static const void* gemm_for(int epi, bool ak, bool bk) {
    switch (epi) {
    case kEpiLse: return (ak && bk) ? reinterpret_cast<const void*>(&gemm_kernel<T, kEpiLse, true, true>) : nullptr;
    case kEpiDlogits:
        return (ak && bk) ? reinterpret_cast<const void*>(&gemm_kernel<T, kEpiDlogits, true, true>) : nullptr;
    case kEpiSplit:
        return (ak && !bk) ? reinterpret_cast<const void*>(&gemm_kernel<T, kEpiSplit, true, false>) : nullptr;
    case kEpiAccum:
        return (!ak && !bk) ? reinterpret_cast<const void*>(&gemm_kernel<T, kEpiAccum, false, false>) : nullptr;
    }
    return nullptr;
}

const void* pick_gemm_kernel(int dtype, int epi, bool a_kcontig, bool b_kcontig) {
    switch (dtype) {
    case kF16: return gemm_for<_Float16>(epi, a_kcontig, b_kcontig);
    case kBF16: return gemm_for<__bf16>(epi, a_kcontig, b_kcontig);
    }
    return nullptr;
}

const void* lse_combine_kernel() { return reinterpret_cast<const void*>(&lse_combine); }

const void* pick_split_sum_kernel(int dtype) {
    switch (dtype) {
    case kF16: return reinterpret_cast<const void*>(&split_sum<_Float16>);
    case kBF16: return reinterpret_cast<const void*>(&split_sum<__bf16>);
    }
    return nullptr;
}

const void* col_sum_kernel() { return reinterpret_cast<const void*>(&col_sum); }

}  // namespace rlpl
