// Full-vocab reverse KL between the softmaxes of two (rows, vocab) logit slabs
// for gfx950 (MI355X).
//
// Operation (model card "Geometric-AI Kernels", section "Reverse KL"): for
// each row r, p = softmax(student[r]), q = softmax(teacher[r]),
//   kl_r = sum_v p_v (log p_v - log q_v),
//   loss = sum_r mask_r kl_r / N,  N = number of rows with a nonzero mask byte
//   (unclamped: 0/0 = NaN when no row is valid),
//   grad_v = mask_r / N * p_v (log p_v - log q_v - kl_r).
// Since log p_v - log q_v = (s_v - t_v) - (lse_s - lse_t), the last factor is
// d_v - E_p[d] with d = s - t, and kl_r = E_p[d] - lse_s + lse_t, formed as
// (E_p[d] - (m_s - m_t)) - (ln z_s - ln z_t) with m the row maxima and z the
// sums of exp(x - m): each bracket is of the size of the logits' spread, not
// of lse, and both are exactly 0 when the rows are equal or vocab is 1.
//
// Design (HBM-bound streaming; no contraction, so no MFMA):
//  * A persistent grid sized to be co-resident, each workgroup taking one piece of a
//    row per round (the whole row when rows are plentiful and the kernel is
//    forward only).  Rows whose mask byte is zero are never read (the fwd+bwd
//    kernel writes their gradient as +0).
//  * Pass 1 reads a row once.  Each lane takes its blocks in groups of four
//    (loaded together), and keeps for its elements the running maximum of s
//    and of t and the sums sum e^(s-m_s), sum e^(t-m_t) and
//    sum e^(s-m_s) (s - t), rescaled when a group raises a maximum (the
//    online normaliser of Milakov and Gimelshein, 2018).  Four interleaved
//    accumulators per lane (sharing the maxima) keep the dependency chains
//    short and each float32 sum to a quarter of a lane's terms.  A wavefront
//    merges its lanes: the maxima first (a butterfly), then each lane's sums
//    rescaled once and added in a butterfly; the four waves are merged alike
//    through LDS.  The pieces of a split row are merged the same way, one
//    piece per lane.
//  * The forward-only kernel stops there.  The fwd+bwd kernel then writes
//    grad_v = p_v (d_v - E_p[d]) / N: from the registers that still hold its
//    piece of the row (one group per lane), or, for rows too long for that,
//    by reading the piece a second time.  p_v / N is one exponential of one
//    fma, 2^(s_v log2 e - (lse_s log2 e + log2 N)).
//  * N needs no exchange: every workgroup counts the (rows-byte) mask itself.
//    The loss is the fixed-order sum of per-workgroup partials that
//    workgroup 0 gathers from the workspace (the protocol of the policy-loss
//    kernels), so the fused and forward-only losses are bit-identical when
//    both split the rows alike.
//  * Rows need not start on a block boundary: a row covers the 32-byte
//    blocks (counted from the slab's start) it touches, all read with 128-bit
//    buffer loads (positions of neighbouring rows are masked in registers; a
//    read past the slab's end returns zeros); the one or two partial blocks
//    are written element by element.
//  * At most 168 VGPRs per lane (three wavefronts per SIMD), so that three
//    workgroups share a compute unit.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "device_common.h"
#include "loss_kernels.h"
#include "vocab_kernels.h"

// No implicit a*b+c contraction in this file: the forward-only and fwd+bwd
// kernels must round pass 1 identically (their losses are bit-identical), and
// the compiler contracts differently in the two instantiations.  The fmaf
// calls below are the intended fused operations.
#pragma clang fp contract(off)

namespace rlpl {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNone = -FLT_MAX;   // logit of a position outside the row: never the maximum, weight 0

// Online sums of one lane (or, after merging, of a wavefront, a workgroup or a
// row).
struct Stats {
    float ms, mt;       // running maxima of s and t
    float zs, zt;       // sum exp(s - ms), sum exp(t - mt)
    float as;           // sum exp(s - ms) * (s - t)
};

// exp(x) for x <= 0 on the hardware base-2 unit; exp(0) is exactly 1.
__device__ __forceinline__ float exp_le0(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Symmetric in a and b (so both lanes of a butterfly get the same bits).
__device__ __forceinline__ Stats merge(const Stats& a, const Stats& b) {
    Stats r;
    r.ms = fmaxf(a.ms, b.ms);
    r.mt = fmaxf(a.mt, b.mt);
    const float fa = exp_le0(a.ms - r.ms), fb = exp_le0(b.ms - r.ms);
    const float ga = exp_le0(a.mt - r.mt), gb = exp_le0(b.mt - r.mt);
    r.zs = a.zs * fa + b.zs * fb;
    r.as = a.as * fa + b.as * fb;
    r.zt = a.zt * ga + b.zt * gb;
    return r;
}

// Merge over the 64 lanes of a wavefront: the maxima first, then each lane's
// sums rescaled once and added in an xor butterfly.  Every lane gets the same
// bits (each addition has the same two operands in both lanes).
__device__ __forceinline__ Stats wave_merge(const Stats& v) {
    float ms = v.ms, mt = v.mt;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        ms = fmaxf(ms, __shfl_xor(ms, off, 64));
        mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    }
    const float f = exp_le0(v.ms - ms), g = exp_le0(v.mt - mt);
    float zs = v.zs * f, as = v.as * f, zt = v.zt * g;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        zs += __shfl_xor(zs, off, 64);
        as += __shfl_xor(as, off, 64);
        zt += __shfl_xor(zt, off, 64);
    }
    return Stats{ms, mt, zs, zt, as};
}

// Merge over the workgroup in a fixed order; the result is valid in every thread.
__device__ __forceinline__ Stats block_merge(const Stats& v, Stats* red) {
    const Stats w = wave_merge(v);
    __syncthreads();                        // red[] may still be read by the previous row
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    float ms = red[0].ms, mt = red[0].mt;
#pragma unroll
    for (int i = 1; i < kWaves; ++i) { ms = fmaxf(ms, red[i].ms); mt = fmaxf(mt, red[i].mt); }
    float zs = 0.0f, zt = 0.0f, as = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const float f = exp_le0(red[i].ms - ms), g = exp_le0(red[i].mt - mt);
        zs += red[i].zs * f;
        as += red[i].as * f;
        zt += red[i].zt * g;
    }
    return Stats{ms, mt, zs, zt, as};
}

// Valid rows: the number of nonzero bytes of mask[0, rows), summed by the whole workgroup.
__device__ __forceinline__ uint32_t count_rows(const uint8_t* __restrict__ mask, uint32_t rows, uint32_t* red) {
    uint32_t n = 0;
    for (uint32_t i = threadIdx.x * 16u; i < rows; i += kThreads * 16u) {
        Dwords<4> d;
        if (i + 16u <= rows) {
            d.load(mask + i);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) d.w[q] = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (i + k < rows) d.w[k >> 2] |= uint32_t(mask[i + k]) << (8 * (k & 3));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = ((d.w[q] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | d.w[q];
            n += __builtin_popcount(x & 0x80808080u);
        }
    }
    return block_sum(n, red);
}

constexpr int kAcc = 4;   // interleaved accumulators per lane

// Positions of block b (elements b*VEC .. b*VEC+VEC-1) inside [lo, hi), as a
// bitmask (bit k = position k); all VEC bits for a block inside the row.
template <int VEC>
__device__ __forceinline__ uint32_t block_bits(uint64_t b, uint64_t lo, uint64_t hi) {
    const uint64_t e0 = b * VEC;
    const uint32_t first = lo > e0 ? uint32_t(lo - e0) : 0u;                 // < VEC for a block of the row
    const uint32_t end = hi < e0 + VEC ? uint32_t(hi - e0) : uint32_t(VEC);  // > first
    return ((1u << end) - 1u) & ~((1u << first) - 1u);
}

constexpr uint32_t all_bits(int vec) { return (1u << vec) - 1u; }

// One 32-byte block of a plane as floats; positions whose bit is clear read as kNone.
template <typename T, int VEC>
__device__ __forceinline__ void block_values(const Plane<T, VEC>& p, uint32_t bits, float (&x)[VEC]) {
#pragma unroll
    for (int k = 0; k < VEC; ++k) x[k] = p.get(k);
    if (bits != all_bits(VEC)) {
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            if (!((bits >> k) & 1u)) x[k] = kNone;
    }
}

// Stores VEC gradient values of block b, only the positions whose bit is set.
template <typename T, int VEC>
__device__ __forceinline__ void store_bits(T* __restrict__ base, uint64_t b, uint32_t bits, const float (&v)[VEC]) {
    T* __restrict__ q = base + b * VEC;
    Dwords<VEC * int(sizeof(T)) / 4> out;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) out.w[k] = __float_as_uint(v[k]);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; k += 2) out.w[k >> 1] = Elem<T>::pack(v[k], v[k + 1]);
    }
    if (bits == all_bits(VEC)) {
        out.store(q);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            if ((bits >> k) & 1u) {
                if constexpr (sizeof(T) == 4) reinterpret_cast<uint32_t*>(q)[k] = out.w[k];
                else reinterpret_cast<uint16_t*>(q)[k] = uint16_t(out.w[k >> 1] >> (16 * (k & 1)));
            }
        }
    }
}

// Running sums of one lane: one maximum per plane, kAcc interleaved sums.
struct LaneSums {
    float ms, mt;
    float zs[kAcc], zt[kAcc], as[kAcc];
};

__device__ __forceinline__ void lane_init(LaneSums& L) {
    L.ms = L.mt = kNone;
#pragma unroll
    for (int q = 0; q < kAcc; ++q) L.zs[q] = L.zt[q] = L.as[q] = 0.0f;
}

constexpr int kGroup = 4;   // blocks a lane loads at once (kThreads apart)

// kGroup blocks of both planes held by one lane: blocks b0 + j * kThreads,
// j < kGroup; bits[j] == 0 marks a block past the piece's end (not loaded).
template <typename T, int VEC>
struct Group {
    Plane<T, VEC> s[kGroup], t[kGroup];
    uint32_t bits[kGroup];
};

// Buffer view of a slab from byte `first` on, `bytes` long (at most 1 GiB):
// reads at or past its end return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_view(const void* base, uint64_t first, uint64_t bytes) {
    const uint32_t n = bytes < (uint64_t(1) << 30) ? uint32_t(bytes) : (1u << 30);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(base) + first), 0, int(n), 0x00020000);
}

constexpr uint32_t kOffView = 0x80000000u;   // a view offset past every view's end

template <typename T, int VEC>
__device__ __forceinline__ void set_plane(Plane<T, VEC>& p, const __attribute__((ext_vector_type(4))) uint32_t& h0,
                                          const __attribute__((ext_vector_type(4))) uint32_t& h1) {
    static_assert(Plane<T, VEC>::kWords == 8, "a block is 32 bytes");
#pragma unroll
    for (int i = 0; i < 4; ++i) { p.d.w[i] = h0[i]; p.d.w[4 + i] = h1[i]; }
}

// The group of blocks g0 + tid + j * kThreads.  g0 is the same in the whole
// workgroup; `end16` is the slab's size in bytes rounded up to 16, so a read
// that starts before the slab's end stays in its last (mapped) page, and one
// that starts after it returns zeros.  Positions outside the row are masked
// later, by block_values; blocks past the piece are not read (zeros).
template <typename T, int VEC>
__device__ __forceinline__ void load_group(Group<T, VEC>& G, const T* __restrict__ S, const T* __restrict__ Tt,
                                           uint64_t g0, uint64_t cb1, uint64_t lo, uint64_t hi, uint64_t end16) {
    const uint64_t first = g0 * 32u;
    const __amdgpu_buffer_rsrc_t rs = slab_view(S, first, end16 - first);
    const __amdgpu_buffer_rsrc_t rt = slab_view(Tt, first, end16 - first);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        const uint64_t b = g0 + threadIdx.x + uint64_t(j) * kThreads;
        G.bits[j] = b < cb1 ? block_bits<VEC>(b, lo, hi) : 0u;
        // view offsets of the two halves (< 32 KB), or past the view's end
        const uint32_t off = G.bits[j] ? (threadIdx.x + uint32_t(j) * kThreads) * 32u : kOffView;
        const auto s0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        const auto s1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0);
        const auto t0 = __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0);
        const auto t1 = __builtin_amdgcn_raw_buffer_load_b128(rt, off + 16u, 0, 0);
        set_plane(G.s[j], s0, s1);
        set_plane(G.t[j], t0, t1);
    }
}

// The held words are declared rewritten, so later uses convert them again
// instead of keeping float copies (twice the registers) alive.
template <typename T, int VEC>
__device__ __forceinline__ void opaque(Group<T, VEC>& G) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
#pragma unroll
        for (int i = 0; i < Plane<T, VEC>::kWords; ++i) asm volatile("" : "+v"(G.s[j].d.w[i]), "+v"(G.t[j].d.w[i]));
}

// Adds a group: the maxima take the whole group first, so the sums are
// rescaled at most once per group.
template <typename T, int VEC>
__device__ __forceinline__ void lane_add(LaneSums& L, Group<T, VEC>& G) {
    float bs = kNone, bt = kNone;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        if (G.bits[j]) {
            float s[VEC], t[VEC];
            block_values<T, VEC>(G.s[j], G.bits[j], s);
            block_values<T, VEC>(G.t[j], G.bits[j], t);
#pragma unroll
            for (int k = 0; k < VEC; ++k) { bs = fmaxf(bs, s[k]); bt = fmaxf(bt, t[k]); }
        }
    }
    opaque(G);
    const float ns = fmaxf(L.ms, bs), nt = fmaxf(L.mt, bt);
    if (ns > L.ms || nt > L.mt) {
        const float fs = exp_le0(L.ms - ns), ft = exp_le0(L.mt - nt);
#pragma unroll
        for (int q = 0; q < kAcc; ++q) { L.zs[q] *= fs; L.as[q] *= fs; L.zt[q] *= ft; }
        L.ms = ns;
        L.mt = nt;
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        if (G.bits[j]) {
            float s[VEC], t[VEC];
            block_values<T, VEC>(G.s[j], G.bits[j], s);
            block_values<T, VEC>(G.t[j], G.bits[j], t);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float es = exp_le0(s[k] - L.ms);
                const float et = exp_le0(t[k] - L.mt);
                L.zs[k % kAcc] += es;
                L.zt[k % kAcc] += et;
                L.as[k % kAcc] = fmaf(es, s[k] - t[k], L.as[k % kAcc]);
            }
        }
        // one block's floats at a time: the scheduler may not hoist the next block's work
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ Stats lane_total(const LaneSums& L) {
    Stats st{L.ms, L.mt, L.zs[0], L.zt[0], L.as[0]};
#pragma unroll
    for (int q = 1; q < kAcc; ++q) { st.zs += L.zs[q]; st.zt += L.zt[q]; st.as += L.as[q]; }
    return st;
}

// grad_v = p_v (d_v - E_p[d]) / N for the positions of one block (others unused):
// p_v / N = 2^(s_v log2 e - c) with c = lse_s log2 e + log2 N, the exponent one fma.
template <typename T, int VEC>
__device__ __forceinline__ void grad_block(const Plane<T, VEC>& ps, const Plane<T, VEC>& pt, uint32_t bits,
                                           float c, float ed, float (&g)[VEC]) {
    float s[VEC], t[VEC];
    block_values<T, VEC>(ps, bits, s);
    block_values<T, VEC>(pt, bits, t);
#pragma unroll
    for (int k = 0; k < VEC; ++k) g[k] = __builtin_amdgcn_exp2f(fmaf(s[k], kLog2e, -c)) * ((s[k] - t[k]) - ed);
}

// The gradient of a group's blocks (g0 as in load_group).
template <typename T, int VEC>
__device__ __forceinline__ void grad_group(const Group<T, VEC>& G, T* __restrict__ grad, uint64_t g0, float c,
                                           float ed) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        if (G.bits[j]) {
            float g[VEC];
            grad_block<T, VEC>(G.s[j], G.t[j], G.bits[j], c, ed, g);
            store_bits<T, VEC>(grad, g0 + threadIdx.x + uint64_t(j) * kThreads, G.bits[j], g);
        }
    }
}

}  // namespace

// Rows are split into `chunks` pieces of `chunk_blocks` 32-byte blocks (one
// piece, the whole row, when there are enough rows to fill the device);
// workgroup w owns piece w % chunks of rows w / chunks, w / chunks + R, ...
// (R = gridDim.x / chunks), one row per round.  With several pieces, their
// online sums go to the workspace and are merged in one fixed order (so every
// workgroup of the row, and the forward-only kernel, gets the same bits).  The
// fwd+bwd kernel then writes the gradient of its piece: from the registers
// that still hold it (kVocabResident, pieces of at most kVocabResidentBlocks
// blocks), or by reading it again (kVocabStream, longer pieces).  A piece's
// sums that have not arrived within the steal limit are computed by the waiting
// workgroup itself, so the only unbounded wait is workgroup 0's for the row
// partials, which every other workgroup publishes without waiting on anything
// unbounded: it ends once they have all run, which needs one free workgroup
// slot on the device besides workgroup 0.  Past the give-up limit that wait
// stops, writes a NaN loss and sets the workspace's sticky flag.
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) vocab_kernel(const VocabArgs a) {
    constexpr int VEC = 32 / int(sizeof(T));   // elements per 32-byte block
    constexpr bool WRITE_GRAD = MODE != kVocabFwd;
    static_assert(VEC % kAcc == 0, "accumulators split a block's elements");
    static_assert(kGroup * kThreads == kVocabResidentBlocks, "a resident piece is one group per lane");
    const uint64_t chunk_blocks = a.chunk_blocks;
    __shared__ float red_f[kWaves];
    __shared__ uint32_t red_u[kWaves];
    __shared__ uint32_t word[1];
    __shared__ Stats red_s[kWaves];
    __shared__ float peer[kVocabMaxChunks * 5];
    __shared__ uint32_t missing[kVocabMaxChunks / 32];

    Workspace* ws = a.ws;
    uint32_t gen = 0;
    if (threadIdx.x == 0) gen = load_relaxed(&ws->generation);
    const Limits lim = read_limits(ws);

    const uint32_t C = a.chunks;
    const uint32_t R = gridDim.x / C;
    const uint32_t grp = blockIdx.x / C, c = blockIdx.x % C;
    const uint32_t rows = uint32_t(a.rows);
    const uint64_t V = uint64_t(a.vocab);
    const uint64_t end16 = (uint64_t(rows) * V * sizeof(T) + 15u) & ~uint64_t(15);   // slab bytes, rounded up
    const T* __restrict__ S = static_cast<const T*>(a.student);
    const T* __restrict__ Tt = static_cast<const T*>(a.teacher);
    const uint32_t N = count_rows(a.mask, rows, red_u);
    gen = share_generation(gen, word);
    const float log2_n = __builtin_amdgcn_logf(float(N));   // -inf when N == 0, used by no row then
    float part = 0.0f;                        // sum of kl_r over the rows whose chunk 0 this is
    const uint32_t rounds = (rows + R - 1) / R;
    // Exchanges so far: the stats buffer alternates per exchange (not per round:
    // masked rows exchange nothing), so a workgroup writes a buffer only after
    // every peer has finished reading it (each peer published the exchange in
    // between only after it had read the one before).
    uint32_t exch = 0;

    for (uint32_t round = 0, r = grp; r < rows; ++round, r += R) {
        const uint64_t lo = uint64_t(r) * V, hi = lo + V;
        const uint64_t rb1 = (hi + VEC - 1) / VEC;
        const uint64_t cb0 = lo / VEC + c * chunk_blocks;
        const uint64_t cb1 = cb0 + chunk_blocks < rb1 ? cb0 + chunk_blocks : rb1;
        if (a.mask[r] == 0) {
            if constexpr (WRITE_GRAD) {
                float z[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) z[k] = 0.0f;
                for (uint64_t b = cb0 + threadIdx.x; b < cb1; b += kThreads)
                    store_bits<T, VEC>(static_cast<T*>(a.grad), b, block_bits<VEC>(b, lo, hi), z);
            }
            continue;
        }
        // Online sums of the chunk: blocks cb0 + tid, cb0 + tid + kThreads, ...,
        // a group of kGroup at a time, in the same order in every variant.
        LaneSums acc;
        lane_init(acc);
        Group<T, VEC> G;
        if constexpr (MODE == kVocabResident) {
            // The piece is one group (at most kGroup * kThreads blocks); it stays
            // in registers for the gradient.
            load_group<T, VEC>(G, S, Tt, cb0, cb1, lo, hi, end16);
            lane_add<T, VEC>(acc, G);
            opaque(G);
        } else {
            for (uint64_t g0 = cb0; g0 < cb1; g0 += kGroup * kThreads) {
                load_group<T, VEC>(G, S, Tt, g0, cb1, lo, hi, end16);
                lane_add<T, VEC>(acc, G);
            }
        }
        Stats st = block_merge(lane_total(acc), red_s);
        Stats row = st;
        if (C > 1) {
            // Publish the chunk's sums, read every chunk's of this row, merge them in a
            // fixed order: lane q of each wavefront takes chunks q, q + 64, ... in turn,
            // then the wavefront merges its lanes.  A chunk whose sums have not come
            // within the steal limit is summed here from the slabs, by the same code
            // as its own workgroup's (the same bits), so no workgroup depends on
            // another being resident.
            const uint32_t tag = gen + 1u + round;
            const uint32_t buf = exch++ & 1u;
            uint64_t* mine = &ws->slot[blockIdx.x].stats[buf][0];
            const float own[5] = {st.ms, st.mt, st.zs, st.zt, st.as};
            if (threadIdx.x < 5) store_relaxed(mine + threadIdx.x, tagged(tag, __float_as_uint(own[threadIdx.x])));
            if (threadIdx.x < kVocabMaxChunks / 32) missing[threadIdx.x] = 0;
            __syncthreads();
            for (uint32_t i = threadIdx.x; i < 5 * C; i += kThreads) {
                const uint32_t q = i / 5;
                if (q == c) {
                    peer[i] = own[i % 5];
                    continue;
                }
                const uint64_t* w = &ws->slot[grp * C + q].stats[buf][i % 5];
                uint64_t x = load_relaxed(w);
                if (uint32_t(x >> 32) != tag && !wait_tagged(w, tag, lim.steal_now(), x))
                    atomicOr(&missing[q >> 5], 1u << (q & 31u));
                else
                    peer[i] = __uint_as_float(uint32_t(x));
            }
            __syncthreads();
            uint32_t any = 0;
#pragma unroll
            for (int k = 0; k < kVocabMaxChunks / 32; ++k) any |= missing[k];
            if (any) {
                for (uint32_t q = 0; q < C; ++q) {
                    if (!((missing[q >> 5] >> (q & 31u)) & 1u)) continue;
                    const uint64_t qb0 = lo / VEC + q * chunk_blocks;
                    const uint64_t qb1 = qb0 + chunk_blocks < rb1 ? qb0 + chunk_blocks : rb1;
                    LaneSums qa;
                    lane_init(qa);
                    Group<T, VEC> Q;
                    for (uint64_t g0 = qb0; g0 < qb1; g0 += kGroup * kThreads) {
                        load_group<T, VEC>(Q, S, Tt, g0, qb1, lo, hi, end16);
                        lane_add<T, VEC>(qa, Q);
                    }
                    const Stats qs = block_merge(lane_total(qa), red_s);
                    if (threadIdx.x < 5) {
                        const float v[5] = {qs.ms, qs.mt, qs.zs, qs.zt, qs.as};
                        peer[5 * q + threadIdx.x] = v[threadIdx.x];
                    }
                }
                __syncthreads();
                if constexpr (MODE == kVocabResident) {
                    // The held piece was given up for the registers of the sums above:
                    // read it again for the gradient.
                    load_group<T, VEC>(G, S, Tt, cb0, cb1, lo, hi, end16);
                    opaque(G);
                }
            }
            Stats mine_q{kNone, kNone, 0.0f, 0.0f, 0.0f};
            for (uint32_t q = threadIdx.x & 63u; q < C; q += 64u)
                mine_q = merge(mine_q, Stats{peer[5 * q], peer[5 * q + 1], peer[5 * q + 2], peer[5 * q + 3],
                                             peer[5 * q + 4]});
            row = wave_merge(mine_q);
            __syncthreads();                    // peer[] and missing[] are rewritten next round
        }
        // log2 z (v_log_f32 is base 2); z >= 1.
        const float l2zs = __builtin_amdgcn_logf(row.zs);
        const float l2zt = __builtin_amdgcn_logf(row.zt);
        const float ed = row.as / row.zs;                       // E_p[s - t]
        if (c == 0) part += (ed - (row.ms - row.mt)) - (l2zs * kLn2 - l2zt * kLn2);   // kl_r
        if constexpr (WRITE_GRAD) {
            // grad_v = p_v (d_v - E_p[d]) / N = 2^(s_v log2 e - c) (d_v - E_p[d]),
            // c = lse_s log2 e + log2 N = m_s log2 e + log2 z_s + log2 N.
            const float cg = fmaf(row.ms, kLog2e, l2zs + log2_n);
            if constexpr (MODE == kVocabResident) {
                grad_group<T, VEC>(G, static_cast<T*>(a.grad), cb0, cg, ed);
            } else {
                for (uint64_t g0 = cb0; g0 < cb1; g0 += kGroup * kThreads) {
                    load_group<T, VEC>(G, S, Tt, g0, cb1, lo, hi, end16);
                    grad_group<T, VEC>(G, static_cast<T*>(a.grad), g0, cg, ed);
                }
            }
        }
    }

    if (threadIdx.x == 0) publish_partial(ws, blockIdx.x, gen, part);
    if (blockIdx.x == 0) {
        const float total = gather_partials(ws, gridDim.x, gen, lim.giveup, red_f);
        // This launch used tags gen + 1 .. gen + rounds; the next starts above them.
        advance_generation(ws, gen, rounds + 1u);
        if (threadIdx.x == 0) {
            *a.loss = total / float(N);                         // 0/0 = NaN when no row is valid
            if (a.n_out) a.n_out[0] = N;
        }
    }
}

// ----------------------------------------------------------------------------- host-side table

template <typename T>
const void* vocab_kernel_of(int mode) {
    switch (mode) {
    case kVocabFwd: return reinterpret_cast<const void*>(&vocab_kernel<T, kVocabFwd>);
    case kVocabResident: return reinterpret_cast<const void*>(&vocab_kernel<T, kVocabResident>);
    case kVocabStream: return reinterpret_cast<const void*>(&vocab_kernel<T, kVocabStream>);
    }
    return nullptr;
}

const void* pick_vocab_kernel(int dtype, int mode) {
    switch (dtype) {
    case kF32: return vocab_kernel_of<float>(mode);
    case kF16: return vocab_kernel_of<_Float16>(mode);
    case kBF16: return vocab_kernel_of<__bf16>(mode);
    }
    return nullptr;
}

}  // namespace rlpl
