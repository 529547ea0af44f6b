// Selective log-probabilities on gfx950 (MI355X) matrix cores: the step
// upstream of the policy losses (page "Add SM100 CuTe DSL GRPO fast path",
// section "Summary": one large matrix multiplication per group of up to 1024
// tokens, the cross-entropy done in place, full logits never kept, FP32
// weight-gradient accumulation across chunks).
//
// Forward: logits tiles z = hidden . weight^T (+ bias) come out of the MFMA
// contraction and never leave the chip: each 128 x 128 tile's epilogue
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
// The contraction: 256 threads (2 x 2 wavefronts), a 128 x 128 output tile,
// K in steps of 32 staged through LDS (double-buffered, the next step's
// global loads in flight during the current step's MFMAs), each wavefront a
// 64 x 64 block of four v_mfma_f32_32x32x16 accumulators.  Operands whose K
// is contiguous in memory move to LDS with 128-bit stores; the others are
// transposed on the way in.  Blocks are mapped so that each XCD works on a
// contiguous run of tiles (shared weight panels stay in its L2).
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

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    static __device__ __forceinline__ floatx16 run(uint4 a, uint4 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    static __device__ __forceinline__ floatx16 run(uint4 a, uint4 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

template <typename T> __device__ __forceinline__ float to_f(T x) { return float(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return T(x); }

constexpr int kLdsK = kGemmBK + 8;        // LDS row: 32 K elements + 8 of padding (80 bytes)
constexpr int kTileElems = kGemmBM * kLdsK;
constexpr float kLog2eG = 1.4426950408889634f;

// One 128 x 32 operand tile in flight: eight 32-bit words per thread.
struct Stage {
    uint32_t w[8];
};

// Global -> registers for the 128-row (M or N) by 32-deep tile at (r0, k0) of
// an operand with R rows and K depth; out-of-range elements read as 0.
// KCONTIG (element (r, k) at x[r*ld + k]): two 16-byte pieces, piece c is
// row c/4, K elements 8*(c%4) .. +8.
// Otherwise (element (r, k) at x[k*ld + r]): the thread takes the row pair
// 2*(tid%64), +1 at the eight K rows 8*(tid/64) .. +8, one 32-bit word per
// K row (a wavefront's load covers 128 contiguous elements of one K row).
template <typename T, bool KCONTIG>
__device__ __forceinline__ void load_stage(const T* __restrict__ x, int64_t ld, int R, int K, int r0, int k0,
                                           Stage& st) {
    const uint16_t* __restrict__ h = reinterpret_cast<const uint16_t*>(x);
    if constexpr (KCONTIG) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = threadIdx.x + q * kGemmThreads;
            const int r = r0 + (c >> 2), k = k0 + 8 * (c & 3);
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r < R) {
                const uint16_t* p = h + int64_t(r) * ld + k;
                if (k + 8 <= K) {
                    v = *reinterpret_cast<const uint4*>(p);
                } else {
                    uint32_t e[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (k + j < K) e[j] = p[j];
                    v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                   e[6] | (e[7] << 16));
                }
            }
            st.w[4 * q + 0] = v.x;
            st.w[4 * q + 1] = v.y;
            st.w[4 * q + 2] = v.z;
            st.w[4 * q + 3] = v.w;
        }
    } else {
        const int r = r0 + 2 * (threadIdx.x & 63), kg = k0 + 8 * (threadIdx.x >> 6);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t w = 0u;
            if (kg + j < K) {
                const uint16_t* p = h + int64_t(kg + j) * ld + r;
                if (r + 1 < R) w = *reinterpret_cast<const uint32_t*>(p);
                else if (r < R) w = p[0];
            }
            st.w[j] = w;
        }
    }
}

// Registers -> LDS tile laid out [row][k] (K contiguous, kLdsK per row),
// 16-byte stores only (the transposed operand is repacked in registers).
template <bool KCONTIG>
__device__ __forceinline__ void store_stage(uint16_t* __restrict__ lds, const Stage& st) {
    if constexpr (KCONTIG) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = threadIdx.x + q * kGemmThreads;
            *reinterpret_cast<uint4*>(lds + (c >> 2) * kLdsK + 8 * (c & 3)) =
                make_uint4(st.w[4 * q], st.w[4 * q + 1], st.w[4 * q + 2], st.w[4 * q + 3]);
        }
    } else {
        const int r = 2 * (threadIdx.x & 63), k = 8 * (threadIdx.x >> 6);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = st.w[2 * j], b = st.w[2 * j + 1];
            lo[j] = (a & 0xffffu) | (b << 16);           // row r: K elements 2j, 2j+1
            hi[j] = (a >> 16) | (b & 0xffff0000u);       // row r+1
        }
        *reinterpret_cast<uint4*>(lds + r * kLdsK + k) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4*>(lds + (r + 1) * kLdsK + k) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
}

// XCD-aware tile order: consecutive block indices go to different XCDs, so
// XCD x (block % 8) takes a contiguous run of tiles; within the run the M
// tile varies fastest, so that neighbours share the N operand's panel.
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t tiles_m, uint32_t tiles_n, uint32_t& tm, uint32_t& tn) {
    const uint32_t T = tiles_m * tiles_n;
    const uint32_t x = b & 7u, idx = b >> 3;
    const uint32_t q = T >> 3, r = T & 7u;
    const uint32_t t = (x < r ? x * (q + 1u) : r * (q + 1u) + (x - r) * q) + idx;
    tm = t % tiles_m;
    tn = t / tiles_m;
}

}  // namespace

template <typename T, int EPI, bool A_KCONTIG, bool B_KCONTIG>
__global__ void __launch_bounds__(kGemmThreads) gemm_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTileElems];
    __shared__ float red_max[2][kGemmBM];
    __shared__ float red_sum[2][kGemmBM];

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int m0 = int(tm) * kGemmBM, n0 = int(tn) * kGemmBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int kb = EPI == kEpiSplit ? int(blockIdx.z) * g.k_split : 0;
    const int ke = EPI == kEpiSplit ? min(g.K, kb + g.k_split) : g.K;
    const T* __restrict__ A = static_cast<const T*>(g.a);
    const T* __restrict__ B = static_cast<const T*>(g.b);

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (kb < ke) {
        Stage sa, sb;
        load_stage<T, A_KCONTIG>(A, g.lda, g.M, ke, m0, kb, sa);
        load_stage<T, B_KCONTIG>(B, g.ldb, g.N, ke, n0, kb, sb);
        store_stage<A_KCONTIG>(As[0], sa);
        store_stage<B_KCONTIG>(Bs[0], sb);
        __syncthreads();
        int cur = 0;
        for (int k0 = kb; k0 < ke; k0 += kGemmBK) {
            const bool more = k0 + kGemmBK < ke;
            if (more) {
                load_stage<T, A_KCONTIG>(A, g.lda, g.M, ke, m0, k0 + kGemmBK, sa);
                load_stage<T, B_KCONTIG>(B, g.ldb, g.N, ke, n0, k0 + kGemmBK, sb);
            }
#pragma unroll
            for (int kk = 0; kk < kGemmBK / 16; ++kk) {
                uint4 af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wm * 64 + i * 32 + (lane & 31);
                    af[i] = *reinterpret_cast<const uint4*>(&As[cur][row * kLdsK + kk * 16 + (lane >> 5) * 8]);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = wn * 64 + j * 32 + (lane & 31);
                    bf[j] = *reinterpret_cast<const uint4*>(&Bs[cur][col * kLdsK + kk * 16 + (lane >> 5) * 8]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<T>::run(af[i], bf[j], acc[i][j]);
            }
            if (more) {
                store_stage<A_KCONTIG>(As[cur ^ 1], sa);
                store_stage<B_KCONTIG>(Bs[cur ^ 1], sb);
            }
            __syncthreads();
            cur ^= 1;
        }
    }

    // Epilogue.  Accumulator element e of tile (i, j) is output row
    // wm*64 + i*32 + 8*(e/4) + 4*(lane/32) + e%4 and column wn*64 + j*32 + lane%32.
    auto row_of_e = [&](int i, int e) { return wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); };
    const int col_l[2] = {wn * 64 + (lane & 31), wn * 64 + 32 + (lane & 31)};

    if constexpr (EPI == kEpiSplit || EPI == kEpiAccum) {
        float* __restrict__ C = static_cast<float*>(g.c);
        if constexpr (EPI == kEpiSplit) C += int64_t(blockIdx.z) * g.M * g.ldc;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + row_of_e(i, e), col = n0 + col_l[j];
                    if (row < g.M && col < g.N) {
                        float* p = C + int64_t(row) * g.ldc + col;
                        *p = (EPI == kEpiAccum && g.accumulate) ? *p + acc[i][j][e] : acc[i][j][e];
                    }
                }
        return;
    }

    // Logits epilogues: z = acc + bias; columns past N are -inf.
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    float bcol[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + col_l[j];
        bcol[j] = col < g.N ? (bias ? to_f<T>(bias[col]) : 0.0f) : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] += bcol[j];

    if constexpr (EPI == kEpiDlogits) {
        T* __restrict__ D = static_cast<T*>(g.c);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + row_of_e(i, e);
                if (row >= g.M) continue;
                const float l = g.lse[row], gr = g.grad[row];
                const int64_t tgt = g.targets[row];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + col_l[j];
                    if (col >= g.N) continue;
                    const float p = __builtin_amdgcn_exp2f((acc[i][j][e] - l) * kLog2eG);
                    const float dz = gr * ((col == tgt ? 1.0f : 0.0f) - p);
                    D[int64_t(row) * g.ldc + col] = from_f<T>(dz);
                }
            }
        return;
    }

    // kEpiLse: per row of the tile, (max, sum exp(z - max)) over its columns, and the target logit.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float m = fmaxf(acc[i][0][e], acc[i][1][e]);
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
            if ((lane & 31) == 0) red_max[wn][row_of_e(i, e)] = m;
            const int row = m0 + row_of_e(i, e);
            if (row < g.M) {
                const int64_t tgt = g.targets[row];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (int64_t(n0 + col_l[j]) == tgt) g.target_logit[row] = acc[i][j][e];
            }
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = row_of_e(i, e);
            const float M = fmaxf(red_max[0][r], red_max[1][r]);
            float s = __builtin_amdgcn_exp2f((acc[i][0][e] - M) * kLog2eG) +
                      __builtin_amdgcn_exp2f((acc[i][1][e] - M) * kLog2eG);
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) s += __shfl_xor(s, off, 64);
            if ((lane & 31) == 0) red_sum[wn][r] = s;
        }
    __syncthreads();
    if (threadIdx.x < kGemmBM) {
        const int r = threadIdx.x, row = m0 + r;
        if (row < g.M) {
            float2* p = reinterpret_cast<float2*>(g.part) + int64_t(row) * g.tiles_n + tn;
            *p = make_float2(fmaxf(red_max[0][r], red_max[1][r]), red_sum[0][r] + red_sum[1][r]);
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

template <typename T>
__global__ void __launch_bounds__(kThreads) col_sum(const ColSumArgs a) {
    const int col = blockIdx.x * kThreads + threadIdx.x;
    if (col >= a.cols) return;
    const T* x = static_cast<const T*>(a.x);
    float s = 0.0f;
    for (int r = 0; r < a.rows; ++r) s += to_f<T>(x[int64_t(r) * a.ldx + col]);
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

const void* pick_col_sum_kernel(int dtype) {
    switch (dtype) {
    case kF16: return reinterpret_cast<const void*>(&col_sum<_Float16>);
    case kBF16: return reinterpret_cast<const void*>(&col_sum<__bf16>);
    }
    return nullptr;
}

}  // namespace rlpl
