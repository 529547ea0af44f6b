// Fused forward+backward PPO-family policy losses for gfx950 (MI355X): the
// kernels, included by one source file per input dtype
// (loss_kernels_{f32,f16,bf16}.hip, compiled in parallel), each of which
// instantiates its dtype's table of kernels.
//
// Operations (model card "Geometric-AI Kernels", sections "BNPO Loss",
// "GRPO Loss", "Reverse KL"):
//   BNPO  loss = sum((per_token + beta*kl)*mask) / max(sum(mask), 1)
//   GRPO  loss = mean_r( sum_t((per_token + beta*kl)*mask) / max(sum_t(mask), 1) )
//   RKL   loss = sum(mask * kl(student, teacher)) / sum(mask)      (unclamped)
// with ratio = exp(lp - old), per_token = -A_r * min(ratio, clip(ratio, 1-eps, 1+eps_high)),
// kl = exp(x) - x - 1, x = ref - lp (teacher - student for RKL).
//
// Design (one launch per call; the path is elementwise + reductions and
// HBM-bound, so there is no MFMA here):
//  * The (bs, seq_len) planes are treated as one flat run of `slots`.  A tile
//    is kThreads lanes x VEC consecutive slots.  Each lane moves its VEC mask
//    bytes and its VEC log-probs per plane with 32/64/128-bit loads.  VEC is
//    16 for large problems and 4 for small ones, so that a small problem
//    still spreads over every compute unit.
//  * A grid of G workgroups (at most what the device holds at once): with
//    one tile per worker, workgroup 0 coordinates and worker w takes tile w;
//    with more, each workgroup is a worker over its share of the tiles
//    (groups of eight consecutive tiles, the workers side by side, for BNPO
//    and reverse-KL; one contiguous run for GRPO; non-temporal accesses) and
//    workgroup 0 also coordinates.  Per-token
//    math is fp32 in registers and branch-free: every slot of a lane is
//    computed and masked slots are selected away (their values never reach
//    a result).
//  * Reductions: per-lane sums -> wavefront tree on DPP lane moves -> LDS
//    across the 4 waves -> one partial per worker in the workspace.  The
//    coordinator sums the partials in worker order, so the loss is
//    deterministic and identical between the fwd+bwd and forward-only
//    kernels.
//  * BNPO / RKL fwd+bwd need the global valid count N before any gradient is
//    scaled: each worker publishes its count as an entry of the workspace;
//    the coordinator gathers them and publishes N (the release) that the
//    workers read once their own tile is computed.  Entries carry the
//    launch's tags (its dispatch id on its queue), so nothing carries over
//    from one launch to the next; all cross-workgroup traffic is
//    device-coherent 16-byte loads and stores: no read-modify-write atomics,
//    never an L2-wide writeback or invalidate.
//  * No workgroup depends on another being resident: a value not published
//    within a time limit is computed by the waiting workgroup itself (the
//    coordinator a worker's count or partial, a worker the global count),
//    by the same code, so the results are bit-identical however the launch
//    is scheduled (beside other kernels, on several streams).
//    When a workgroup owns a single tile, its count is published as soon as
//    its mask has arrived (the exchange then overlaps the plane loads and the
//    per-token math) and the tile never leaves registers; with more tiles it
//    counts its masks first (eight loads in flight) and streams after.
//  * GRPO needs each row's own count; a row may span several workers' runs.
//    Its kernel (grpo_kernel below) exchanges only the counts and sums of the
//    rows that cross a run's ends, and reads each mask byte once.
//  * Plane loads wait for the mask and are skipped for lanes whose mask
//    bytes are all zero; when streaming several tiles per workgroup, the next
//    tile's mask is fetched while the current tile is computed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "loss_kernels.h"

// No implicit a*b+c contraction: a value the coordinator computes in place of
// a worker must round exactly as the worker's own (the fmaf calls below are
// the intended fused operations).
#pragma clang fp contract(off)

namespace rlpl {

// VEC mask bytes of one lane (in E-slot chunks, as the planes: byte k is the
// lane's element k).
template <int VEC>
struct Mask {
    Dwords<VEC / 4> d;
    template <bool NT = false, bool CHECK = true, int E = VEC>
    __device__ __forceinline__ void load(const uint8_t* __restrict__ mask, uint32_t s, uint32_t slots) {
#pragma unroll
        for (int c = 0; c < VEC / E; ++c) {
            const uint32_t sc = chunk_slot<VEC, E>(s, c);
            if (!CHECK || sc + E <= slots) {
                Dwords<E / 4> v;
                v.template load<NT>(mask + sc);
#pragma unroll
                for (int i = 0; i < E / 4; ++i) d.w[c * (E / 4) + i] = v.w[i];
            } else {
#pragma unroll
                for (int i = 0; i < E / 4; ++i) d.w[c * (E / 4) + i] = 0;
#pragma unroll
                for (int k = 0; k < E; ++k)
                    if (sc + k < slots) d.w[c * (E / 4) + (k >> 2)] |= uint32_t(mask[sc + k]) << (8 * (k & 3));
            }
        }
    }
    __device__ __forceinline__ bool any() const {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) o |= d.w[i];
        return o != 0;
    }
    // Whether chunk c (E slots) has a valid slot.
    template <int E>
    __device__ __forceinline__ bool any_in(int c) const {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < E / 4; ++i) o |= d.w[c * (E / 4) + i];
        return o != 0;
    }
    __device__ __forceinline__ bool valid(int k) const { return ((d.w[k >> 2] >> (8 * (k & 3))) & 0xFFu) != 0; }
    // Moves every byte down one position (byte k+1 becomes k; the last becomes 0).
    __device__ __forceinline__ void rotate() {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i)
            d.w[i] = __builtin_amdgcn_alignbit(i + 1 < VEC / 4 ? d.w[i + 1] : 0u, d.w[i], 8);
    }
    // Number of nonzero bytes: for each byte, (b & 0x7F) + 0x7F sets bit 7 iff the low 7 bits
    // are nonzero; OR-ing b itself covers bit 7.
    __device__ __forceinline__ uint32_t count() const {
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            const uint32_t x = ((d.w[i] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | d.w[i];
            n += __builtin_popcount(x & 0x80808080u);
        }
        return n;
    }
    // One bit per slot (bit k = slot k valid).  Per dword, the nonzero-byte
    // flags (bits 7, 15, 23, 31) are shifted to bits 0, 8, 16, 24 and gathered
    // into bits 21..24 by one multiply by 1 + 2^7 + 2^14 + 2^21 (the sixteen
    // partial products land on distinct bits, so nothing carries).
    __device__ __forceinline__ uint32_t bits() const {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            const uint32_t f = ((((d.w[i] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | d.w[i]) & 0x80808080u) >> 7;
            b |= ((f * 0x00204081u) >> 21 & 0xFu) << (4 * i);
        }
        return b;
    }
    // The inverse, with valid slots as byte 1: the same multiply spreads four
    // bits to bits 0, 8, 16, 24 (again on distinct bits).
    __device__ __forceinline__ void from_bits(uint32_t b) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) d.w[i] = ((b >> (4 * i)) & 0xFu) * 0x00204081u & 0x01010101u;
    }
};

// ----------------------------------------------------------------------------- per-token math

// exp on the hardware base-2 exponential unit.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Per-row coefficients of the per-token terms: c = ac*med3(ratio, L, H) + bc*kl
// and g = [unclipped]*ag*ratio - bg*(exp(ref - lp) - 1), where ac = -A and
// bc = beta, and ag, bg are the same times the gradient's scale wherever that
// is known before the tile is computed.  GRPO's per-row scale (an LDS value)
// multiplies c and g afterwards: folded into the coefficients it made every
// product wait for the LDS read and cost 17 VGPRs (one fewer wave per SIMD).
struct Coef {
    float ac, ag, bc, bg;
    float L, H;   // clip bounds of the row: (-inf, 1+eps_high), or (1-eps, +inf) where the
                  // sign-aware form meets A < 0
};

// Per-token contribution c = per_token + beta*kl and its derivative g in lp.
// The literal per_token -A*min(ratio, clip(ratio, lo, hi)) is -A*min(ratio, hi)
// for every ratio (the lower bound never enters); the sign-aware
// -min(A*ratio, A*clip(ratio, lo, hi)) is the same where A >= 0 and
// -A*max(ratio, lo) where A < 0.  Both are ac*med3(ratio, L, H) with the row's
// bounds, and the unclipped branch (ties included) is exactly chosen == ratio.
template <int MODE, bool HAS_KL>
__device__ __forceinline__ void token_terms(float lp, float old, float ref, const Coef& k,
                                            float& c, float& g) {
    if constexpr (MODE == kModeRKL) {
        const float x = ref - lp;                 // teacher - student
        const float em1 = fast_exp(x) - 1.0f;
        c = em1 - x;                              // exp(x) - x - 1
        g = em1 * k.ag;                           // ag = -scale: d/dstudent = 1 - exp(x)
    } else {
        const float ratio = fast_exp(lp - old);
        const float chosen = __builtin_amdgcn_fmed3f(ratio, k.L, k.H);
        c = k.ac * chosen;
        g = (chosen == ratio) ? k.ag * ratio : 0.0f;
        if constexpr (HAS_KL) {
            const float x = ref - lp;
            const float em1 = fast_exp(x) - 1.0f;
            c = fmaf(k.bc, em1 - x, c);
            g = fmaf(-k.bg, em1, g);
        }
    }
}

// ----------------------------------------------------------------------------- rows

// Row of slot s: s / seq_len by multiply-shift with the host's exact magic
// constant (valid for every s < 2^31).
__device__ __forceinline__ uint32_t row_of(const Args& a, uint32_t s) {
    return uint32_t((uint64_t(s) * a.row_magic) >> a.row_shift);
}

// The row and position that a lane chunk starting at slot sc takes its row's
// coefficients from: a chunk that starts past the last slot (the last tile's
// tail, all of it masked) takes those of the last slot, so that no row index
// reaches bs (no read past the advantages, no scale of a row outside the tile).
__device__ __forceinline__ uint32_t chunk_row_slot(const Args& a, uint32_t sc) {
    const uint32_t last = uint32_t(a.slots) - 1u;
    return sc < last ? sc : last;
}

template <typename T>
__device__ __forceinline__ float load_adv(const void* adv, uint32_t r) {
    if constexpr (sizeof(T) == 4) return static_cast<const float*>(adv)[r];
    else {
        const uint32_t w = static_cast<const uint16_t*>(adv)[r];
        return Elem<T>::get(&w, 0);
    }
}

// ----------------------------------------------------------------------------- one tile of one lane

template <typename T, int VEC>
struct Lane {
    Mask<VEC> m;
    Plane<T, VEC> lp, old, ref;
};

// Issues one lane's mask and plane loads (mask first) and returns its valid
// count.  SPEC: the plane loads go out together with the mask (one memory
// latency instead of two, at the price of plane bytes for masked slots);
// otherwise they wait for the mask and are skipped when all of its bytes are
// zero.  Interleaved A/B on one-tile launches: speculative loads are faster
// for the narrow-lane forward-only and GRPO kernels, which serve the
// smallest, latency-bound problems (bf16 64x4096 forward-only BNPO -3 to
// -9 %, GRPO 128x2048 -1 to -5 %); slower for the wide-lane ones, where the
// extra bytes start to count (forward-only BNPO 1024x4096 +13 %, GRPO +9 %);
// and no faster for BNPO and reverse-KL fwd+bwd, whose count exchange takes
// longer than the second latency.  A lane entirely in range
// takes straight-line code; the lane that runs past `slots` (one per launch
// at most) loads element by element.  No workgroup barrier inside, so the
// divergent branch is safe.
template <typename T, int MODE, bool HAS_KL, int VEC, bool SPEC, bool CHECK = true, int E = VEC>
__device__ __forceinline__ uint32_t load_lane_count(const Args& a, uint32_t s, Lane<T, VEC>& L) {
    const uint32_t slots = uint32_t(a.slots);
    if constexpr (E != VEC) {
        // Chunked lanes: each chunk checks its own range, and loads its planes
        // only where it has a valid slot.
        L.m.template load<false, CHECK, E>(a.mask, s, slots);
#pragma unroll
        for (int c = 0; c < VEC / E; ++c) {
            if (SPEC || L.m.template any_in<E>(c)) {
                L.lp.template load_chunk<false, CHECK, E>(static_cast<const T*>(a.lp), s, slots, c);
                if constexpr (MODE != kModeRKL)
                    L.old.template load_chunk<false, CHECK, E>(static_cast<const T*>(a.old), s, slots, c);
                if constexpr (HAS_KL) L.ref.template load_chunk<false, CHECK, E>(static_cast<const T*>(a.ref), s, slots, c);
            }
        }
        return L.m.count();
    }
    if (!CHECK || s + VEC <= slots) {
        L.m.d.load(a.mask + s);
        if constexpr (SPEC) {
            L.lp.d.load(static_cast<const T*>(a.lp) + s);
            if constexpr (MODE != kModeRKL) L.old.d.load(static_cast<const T*>(a.old) + s);
            if constexpr (HAS_KL) L.ref.d.load(static_cast<const T*>(a.ref) + s);
            return L.m.count();
        } else {
            const uint32_t n = L.m.count();
            if (n) {
                L.lp.d.load(static_cast<const T*>(a.lp) + s);
                if constexpr (MODE != kModeRKL) L.old.d.load(static_cast<const T*>(a.old) + s);
                if constexpr (HAS_KL) L.ref.d.load(static_cast<const T*>(a.ref) + s);
            }
            return n;
        }
    }
    L.m.load(a.mask, s, slots);
    L.lp.load(static_cast<const T*>(a.lp), s, slots);
    if constexpr (MODE != kModeRKL) L.old.load(static_cast<const T*>(a.old), s, slots);
    if constexpr (HAS_KL) L.ref.load(static_cast<const T*>(a.ref), s, slots);
    return L.m.count();
}

// Loads one lane's planes once its mask has arrived, chunk by chunk; a chunk
// whose mask bytes are all zero loads nothing (its registers are never used
// for a valid slot).
template <typename T, int MODE, bool HAS_KL, int VEC, bool NT = false, bool CHECK = true, int E = VEC>
__device__ __forceinline__ void load_planes(const Args& a, uint32_t s, Lane<T, VEC>& L) {
#pragma unroll
    for (int c = 0; c < VEC / E; ++c) {
        // Per chunk (a lane's chunks are a wavefront access apart): the row end
        // of a prefix mask leaves one chunk of a lane valid and the other not.
        if (L.m.template any_in<E>(c)) {
            L.lp.template load_chunk<NT, CHECK, E>(static_cast<const T*>(a.lp), s, a.slots, c);
            if constexpr (MODE != kModeRKL)
                L.old.template load_chunk<NT, CHECK, E>(static_cast<const T*>(a.old), s, a.slots, c);
            if constexpr (HAS_KL) L.ref.template load_chunk<NT, CHECK, E>(static_cast<const T*>(a.ref), s, a.slots, c);
        }
    }
}

// Per-slot terms of one lane (slots s .. s+VEC-1): returns the lane's sum of c
// over valid slots and leaves the derivative of every slot, times gscale, in g
// (the store selects masked slots to +0).  GRPO multiplies c and g by each
// row's 1/(max(n_r,1)*bs) (row_scale[r - row_base], LDS).
template <int MODE>
__device__ __forceinline__ Coef row_coef(const Args& a, float A, float row_scale, float gscale) {
    Coef k;
    const bool low_clip = a.sign_aware != 0u && A < 0.0f;
    k.L = low_clip ? a.lo : -__builtin_inff();
    k.H = low_clip ? __builtin_inff() : a.hi;
    if constexpr (MODE == kModeRKL) {
        k.ac = k.bc = 0.0f;
        k.ag = -gscale;
        k.bg = 0.0f;
    } else if constexpr (MODE == kModeGRPO) {
        k.ac = k.ag = -A;                 // the row scale multiplies c and g afterwards
        k.bc = k.bg = a.beta;
    } else {
        k.ac = -A;
        k.bc = a.beta;
        k.ag = -A * gscale;
        k.bg = a.beta * gscale;
    }
    return k;
}

template <typename T, int MODE, bool HAS_KL, int VEC, int E = VEC>
__device__ __forceinline__ float lane_terms(const Args& a, uint32_t s, const Lane<T, VEC>& L,
                                            const float* row_scale, uint32_t row_base, float gscale,
                                            float (&g)[VEC]) {
    constexpr int C = VEC / E;   // chunks of E consecutive slots
    float part = 0.0f;
    if (!L.m.any()) return part;
    const uint32_t T_len = uint32_t(a.seq_len);
    uint32_t r[C], t[C];
    bool one_row = true;         // every chunk within one row
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint32_t sc = chunk_row_slot(a, chunk_slot<VEC, E>(s, c));
        r[c] = row_of(a, sc);
        t[c] = sc - r[c] * T_len;
        one_row = one_row && t[c] + E <= T_len;
    }
    if (MODE == kModeRKL || one_row) {
        // Each chunk in one row (always, when seq_len is a multiple of E; the
        // reverse-KL terms do not depend on the row at all): branch-free.
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float A = 0.0f, rs = 1.0f;
            if constexpr (MODE != kModeRKL) A = load_adv<T>(a.adv, r[c]);
            if constexpr (MODE == kModeGRPO) rs = row_scale[r[c] - row_base];
            const Coef k = row_coef<MODE>(a, A, rs, gscale);
#pragma unroll
            for (int i = c * E; i < c * E + E; ++i) {
                float cv, gi;
                token_terms<MODE, HAS_KL>(L.lp.get(i), MODE == kModeRKL ? 0.0f : L.old.get(i),
                                          HAS_KL ? L.ref.get(i) : 0.0f, k, cv, gi);
                if constexpr (MODE == kModeGRPO) { cv *= rs; gi *= rs; }
                part += L.m.valid(i) ? cv : 0.0f;
                g[i] = gi;
            }
        }
    } else {
        // A chunk crosses a row boundary: slot by slot, tracking the row.  A rolled
        // loop keeps one slot's terms live (this path is rare: only lanes that
        // straddle a row end); it always works on slot 0 of a copy of the lane
        // that rotates down one slot per step, and the derivatives rotate in at
        // the top, so that every register index stays static.  The row is found
        // afresh at each chunk's first slot.
        Lane<T, VEC> R = L;
        float out[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) out[i] = 0.0f;
        uint32_t rr = 0, tt = 0;
        float A = 0.0f, rs = 1.0f;
        Coef k{};
#pragma unroll 1
        for (int i = 0; i < VEC; ++i) {
            if ((i & (E - 1)) == 0) {
                const uint32_t sc = chunk_row_slot(a, chunk_slot<VEC, E>(s, i / E));
                rr = row_of(a, sc);
                tt = sc - rr * T_len;
                if constexpr (MODE != kModeRKL) A = load_adv<T>(a.adv, rr);
                if constexpr (MODE == kModeGRPO) rs = row_scale[rr - row_base];
                k = row_coef<MODE>(a, A, rs, gscale);
            }
            float cv, gi;
            token_terms<MODE, HAS_KL>(R.lp.get(0), MODE == kModeRKL ? 0.0f : R.old.get(0),
                                      HAS_KL ? R.ref.get(0) : 0.0f, k, cv, gi);
            if constexpr (MODE == kModeGRPO) { cv *= rs; gi *= rs; }
            part += R.m.valid(0) ? cv : 0.0f;
#pragma unroll
            for (int j = 0; j + 1 < VEC; ++j) out[j] = out[j + 1];
            out[VEC - 1] = gi;
            R.m.rotate();
            R.lp.rotate();
            if constexpr (MODE != kModeRKL) R.old.rotate();
            if constexpr (HAS_KL) R.ref.rotate();
            if (++tt == T_len) {
                tt = 0;
                ++rr;
                if (rr < uint32_t(a.bs)) {
                    if constexpr (MODE != kModeRKL) A = load_adv<T>(a.adv, rr);
                    if constexpr (MODE == kModeGRPO) rs = row_scale[rr - row_base];
                    k = row_coef<MODE>(a, A, rs, gscale);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) g[i] = out[i];
    }
    return part;
}

// Stores one lane's gradient, masked slots as +0; SCALE multiplies by `scale`
// first (the one-tile fwd+bwd path, whose N arrives after the terms are formed).
template <typename T, int VEC, bool SCALE, bool NT = false, bool CHECK = true, int E = VEC>
__device__ __forceinline__ void store_grad(const Args& a, uint32_t s, const Mask<VEC>& m,
                                           const float (&g)[VEC], float scale) {
    float v[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) v[k] = m.valid(k) ? (SCALE ? g[k] * scale : g[k]) : 0.0f;
    store_values<T, VEC, NT, CHECK, E>(static_cast<T*>(a.grad), s, a.slots, v);
}


// ----------------------------------------------------------------------------- the kernel

template <int MODE>
__device__ __forceinline__ float inv_count(uint32_t N) {
    // BNPO: 1 / max(N, 1); reverse-KL: 1 / N unclamped (inf when N == 0, used by no slot).
    if constexpr (MODE == kModeRKL) return 1.0f / float(N);
    else return 1.0f / float(N > 0 ? N : 1u);
}

template <int MODE>
__device__ __forceinline__ float final_loss(float total, uint32_t N) {
    if constexpr (MODE == kModeRKL) return total / float(N);          // 0/0 = NaN when N == 0
    else return total / float(N > 0 ? N : 1u);
}

// Thread 0 of the coordinating workgroup: the loss (and for the global-count
// losses, the valid-token count N).
template <int MODE>
__device__ __forceinline__ void write_results(const Args& a, float total, uint32_t N) {
    if constexpr (MODE == kModeGRPO) {
        *a.loss = total;
    } else {
        *a.loss = final_loss<MODE>(total, N);
        if (a.n_out) a.n_out[0] = N;
    }
}

// The mask bits of this lane's chunks (bit k = the lane's element k), from
// per-thread mask bits in the one-chunk layout (grp[t] = bits of slots
// t*VEC .. t*VEC+VEC-1 of the tile, in LDS): each chunk lies inside one
// thread's VEC slots, of a thread of the same wavefront.
template <int VEC, int E>
__device__ __forceinline__ uint32_t chunk_bits(const uint16_t* grp) {
    if constexpr (E == VEC) return grp[threadIdx.x];
    const uint32_t w = threadIdx.x >> 6, l = threadIdx.x & 63u;
    uint32_t b = 0;
#pragma unroll
    for (int c = 0; c < VEC / E; ++c) {
        const uint32_t rel = (uint32_t(c) * 64u + l) * uint32_t(E);   // the chunk's slot in the wavefront's span
        const uint32_t g = 64u * w + rel / uint32_t(VEC), off = rel % uint32_t(VEC);
        b |= ((uint32_t(grp[g]) >> off) & ((1u << E) - 1u)) << (c * E);
    }
    return b;
}

// Streams a worker's tiles (`sw`): per tile, the lane's terms,
// its count and (WRITE_GRAD) the scaled gradient.  Masks and planes are read
// with non-temporal loads (they stream through once); the gradient is stored
// through the caches, or non-temporally with NT_GRAD (the host's choice from
// kNtGradBytes of inputs and gradient on: below, cached stores measured 6-20 %
// faster, above, non-temporal ones 1-8 %; a wavefront's store covers 1 KB
// without a gap, so either way whole lines are written).  The
// plane loads wait for the mask, and the next tile's mask is fetched during
// the current tile.  (Measured A/B: leaving out the per-lane range test on
// tiles known to be in range, or keeping a second tile's planes in flight,
// made this loop 4-18 % slower at 2^26 and 2^28 slots.)
// The counting pass reads the mask in the one-chunk layout (16 bytes per lane;
// 8-byte accesses per chunk made that pass slower) and keeps per-thread bits,
// which reach the lanes' chunks through chunk_bits(); tiles past the kept
// bits read their mask bytes again, per chunk.
// The tiles of one worker of a striding kernel: in rounds, worker w of W
// takes the group of kSweepGroup consecutive tiles k * W + w of round k; the
// tiles left after the full rounds are split into W contiguous pieces of at
// most q tiles (so no worker has more than one tile above the mean).  At any
// moment the workers stream a window of about W groups instead of W runs
// spread over the whole slab.  Measured against one contiguous run per worker
// (interleaved A/B, bf16): fused BNPO 2^28 slots 354.4 -> 347.7 us, 2^26
// 80.9 -> 78.3, reverse KL 2^28 290.6 -> 275.1; groups of 16 or 32 tiles
// were slower, and tiles strided one by one over the grid markedly slower.
constexpr uint32_t kSweepGroup = 8;
struct Sweep {
    uint32_t w, W, full, base, q;   // full: tiles per worker in the full rounds
    __device__ __forceinline__ Sweep(uint32_t w_, uint32_t W_, uint32_t tiles) : w(w_), W(W_) {
        const uint32_t rounds = tiles / (W * kSweepGroup);
        full = rounds * kSweepGroup;
        base = rounds * W * kSweepGroup;
        q = (tiles - base + W - 1u) / W;
        const uint32_t end = base + q * (w + 1u);
        const uint32_t lo = base + q * w;
        extra = lo < tiles ? (end < tiles ? q : tiles - lo) : 0u;
    }
    uint32_t extra;                  // tiles of w's piece of the remainder
    __device__ __forceinline__ uint32_t count() const { return full + extra; }
    // Worker w's j-th tile (j < count()).  kSweepGroup consecutive j from a
    // multiple of kSweepGroup are consecutive tiles.
    __device__ __forceinline__ uint32_t tile(uint32_t j) const {
        return j < full ? ((j / kSweepGroup) * W + w) * kSweepGroup + j % kSweepGroup : base + q * w + (j - full);
    }
};

template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD, int VEC, bool NT_GRAD = false>
__device__ __forceinline__ void stream_tiles(const Args& a, const Sweep& sw, float& part, uint32_t& n_lane,
                                             float scale, const uint16_t* bits = nullptr, uint32_t n_bits = 0) {
    constexpr uint32_t kTileV = kThreads * VEC;
    constexpr int E = chunk_slots<T, VEC>();
    const uint32_t lane_off = threadIdx.x * VEC;
    const uint32_t slots = uint32_t(a.slots);
    const uint32_t nt = sw.count();
    // The worker's first n_bits tiles take their masks from `bits` (each
    // thread's entry of each, in LDS); later ones read the mask bytes again.
    Mask<VEC> next;
    if (nt > 0 && n_bits == 0) next.template load<true, true, E>(a.mask, sw.tile(0) * kTileV + lane_off, slots);
    for (uint32_t j = 0; j < nt; ++j) {
        const uint32_t s = sw.tile(j) * kTileV + lane_off;
        Lane<T, VEC> L;
        if (j < n_bits) L.m.from_bits(chunk_bits<VEC, E>(bits + j * kThreads));
        else L.m = next;
        if (j + 1 < nt && j + 1 >= n_bits)
            next.template load<true, true, E>(a.mask, sw.tile(j + 1) * kTileV + lane_off, slots);
        load_planes<T, MODE, HAS_KL, VEC, true, true, E>(a, s, L);
        n_lane += L.m.count();
        float g[VEC];
        part += lane_terms<T, MODE, HAS_KL, VEC, E>(a, s, L, nullptr, 0, scale, g);
        if constexpr (WRITE_GRAD) store_grad<T, VEC, false, NT_GRAD, true, E>(a, s, L.m, g, 1.0f);
    }
}

// Workgroup 0 coordinates: it gathers the workers' counts, releases N (fwd+bwd
// BNPO / reverse-KL), gathers their partials in worker order and writes the
// loss.  ONE_TILE kernels are launched with exactly one tile per worker and a
// coordinator that owns no tile (G = tiles + 1), and keep the tile in registers
// in straight-line code.  The others (G at most the co-resident capacity,
// G <= tiles) stride over any number of tiles per worker, which costs
// registers, and workgroup 0 is a worker as well.
//
// No wait depends on another workgroup being resident: a count or partial the
// coordinator has not seen within the steal limit is computed by the
// coordinator itself from the inputs (the worker, whenever it runs, computes
// and stores the same values), and a worker that has not seen N within the
// release limit gathers it itself.  Every such value is computed by the same
// code as the worker's own, so the results are bit-identical either way.
template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD, int VEC, bool ONE_TILE, bool NT_GRAD = false>
__global__ void __launch_bounds__(kThreads) loss_kernel(const Args a) {
    constexpr uint32_t kTileV = kThreads * VEC;
    constexpr int E = chunk_slots<T, VEC>();   // slots per chunk of a lane
    __shared__ float red_f[kWaves];
    __shared__ uint32_t red_u[kWaves];
    __shared__ uint32_t word[2];
    __shared__ uint32_t list[kThreads + 1];
    // Striding fwd+bwd kernels: the counting pass keeps each lane's mask bits
    // of the worker's first kBitTiles tiles, so that the streaming pass does
    // not read those mask bytes again.
    constexpr bool kKeepBits = !ONE_TILE && WRITE_GRAD;
    constexpr int kBitTiles = kKeepBits ? (MODE == kModeRKL ? kBitTilesRkl : kBitTilesPolicy) : 1;
    __shared__ uint16_t mask_bits[kBitTiles * kThreads];

    static_assert(MODE != kModeGRPO, "GRPO has a kernel of its own (grpo_kernel)");
    constexpr bool kExchange = WRITE_GRAD;
    const Workspace* ws = a.ws;
    const __amdgpu_buffer_rsrc_t view = entry_view(ws);
    const Tag tg = launch_tag();
    const Limits lim = read_limits(ws);
    const uint32_t slots = uint32_t(a.slots);
    const uint32_t W = ONE_TILE ? gridDim.x - 1 : gridDim.x;   // workers
    const uint32_t lane_off = threadIdx.x * VEC;

    // Worker w's valid count and partial loss, computed by the calling workgroup
    // (uniform), exactly as worker w forms its own (the one-tile kernels' worker
    // w owns tile w; the striding kernels' workers sweep the tiles of Sweep).
    auto count_of = [&](uint32_t w) -> uint32_t {
        uint32_t n = 0;
        if constexpr (ONE_TILE) {
            Mask<VEC> m;
            m.load(a.mask, w * kTileV + lane_off, slots);
            n = m.count();
        } else {
            const Sweep sw(w, W, a.tiles);
            for (uint32_t j = 0; j < sw.count(); ++j) {
                Mask<VEC> m;
                m.load(a.mask, sw.tile(j) * kTileV + lane_off, slots);
                n += m.count();
            }
        }
        return block_sum(n, red_u);
    };
    auto partial_of = [&](uint32_t w) -> float {
        float part = 0.0f;
        if constexpr (ONE_TILE) {
            const uint32_t s = w * kTileV + lane_off;
            Lane<T, VEC> L;
            (void)load_lane_count<T, MODE, HAS_KL, VEC, false, true, E>(a, s, L);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC, E>(a, s, L, nullptr, 0, 1.0f, g);
        } else {
            uint32_t n_unused = 0;
            stream_tiles<T, MODE, HAS_KL, false, VEC>(a, Sweep(w, W, a.tiles), part, n_unused, 1.0f);
        }
        return block_sum(part, red_f);
    };
    auto nothing = [] {};
    auto gather_counts = [&]() -> uint32_t {
        return gather<uint32_t>(view, cnt_off, W, tg, lim.steal_now(), list, red_u, count_of, nothing);
    };
    // The partials' first reads go out before the release (when there is one) is stored.
    auto gather_partials = [&](auto&& between) -> float {
        return gather<float>(view, par_off, W, tg, lim.steal_now(), list, red_f, partial_of, between);
    };

    float part = 0.0f;
    uint32_t n_lane = 0;

    if constexpr (ONE_TILE) {
        // Workgroup 0 coordinates only; workgroup w > 0 is worker w - 1 and owns tile w - 1.
        if (blockIdx.x == 0) {
            const uint32_t N = gather_counts();
            const float total = gather_partials([&] {
                if (kExchange && threadIdx.x == 0) publish(view, kReleaseOff, tg, N);
            });
            if (threadIdx.x == 0) write_results<MODE>(a, total, N);
            return;
        }
        const uint32_t worker = blockIdx.x - 1;
        const uint32_t s = worker * kTileV + lane_off;
        Lane<T, VEC> L;
        if constexpr (kExchange) {
            // The tile stays in registers across the count exchange.  The count is
            // published as soon as the mask (loaded first) has arrived, so the exchange
            // runs while the planes are still arriving and being computed on; the
            // partial loss follows.
            const uint32_t n_wg = block_sum(load_lane_count<T, MODE, HAS_KL, VEC, false, true, E>(a, s, L), red_u);
            if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC, E>(a, s, L, nullptr, 0, 1.0f, g);
            const float part_wg = block_sum(part, red_f);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
            const uint32_t N = await_release(view, lim.release_now(), tg, word, gather_counts);
            store_grad<T, VEC, true, false, true, E>(a, s, L.m, g, inv_count<MODE>(N));
        } else {
            // Forward only.
            n_lane = load_lane_count<T, MODE, HAS_KL, VEC, VEC == kVecSmall, true, E>(a, s, L);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC, E>(a, s, L, nullptr, 0, 1.0f, g);
            const float part_wg = block_sum(part, red_f);
            const uint32_t n_wg = block_sum(n_lane, red_u);
            if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
        }
    } else {
        // Every workgroup is a worker over its tiles (Sweep: groups of consecutive
        // tiles stream markedly faster than tiles strided one by one across the
        // grid); workgroup 0 also coordinates (a dedicated coordinator would take
        // one of the co-resident slots, and with it a whole extra tile from some
        // worker's share).
        const uint32_t worker = blockIdx.x;
        const Sweep sw(worker, W, a.tiles);
        const uint32_t nt = sw.count();
        uint32_t N = 0;
        if constexpr (kExchange) {
            // Count every owned mask (eight loads in flight per lane, eight
            // consecutive tiles) and keep the bits of the first kBitTiles tiles,
            // exchange, then stream.
            static_assert(kSweepGroup % 8 == 0, "eight consecutive tiles per batch");
            uint32_t j = 0;
            for (; j + 7 < nt; j += 8) {
                const uint32_t tile = sw.tile(j);
                Mask<VEC> m[8];
                if ((tile + 8) * kTileV <= slots) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        m[u].template load<true, false>(a.mask, (tile + u) * kTileV + lane_off, slots);
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u) m[u].template load<true>(a.mask, (tile + u) * kTileV + lane_off, slots);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t b = m[u].bits();
                    n_lane += __builtin_popcount(b);
                    if (j + u < uint32_t(kBitTiles)) mask_bits[(j + u) * kThreads + threadIdx.x] = uint16_t(b);
                }
            }
            for (; j < nt; ++j) {
                Mask<VEC> m;
                m.template load<true>(a.mask, sw.tile(j) * kTileV + lane_off, slots);
                const uint32_t b = m.bits();
                n_lane += __builtin_popcount(b);
                if (j < uint32_t(kBitTiles)) mask_bits[j * kThreads + threadIdx.x] = uint16_t(b);
            }
            const uint32_t n_bits = j < uint32_t(kBitTiles) ? j : uint32_t(kBitTiles);
            const uint32_t n_wg = block_sum(n_lane, red_u);
            if (blockIdx.x == 0) {
                // The coordinator's own count goes out once its reads of the others' are issued.
                N = gather<uint32_t>(view, cnt_off, W, tg, lim.steal_now(), list, red_u, count_of, [&] {
                    if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
                });
                if (threadIdx.x == kCountThread) publish(view, kReleaseOff, tg, N);
            } else {
                if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
                N = await_release(view, lim.release_now(), tg, word, gather_counts);
            }
            uint32_t unused_n = 0;
            stream_tiles<T, MODE, HAS_KL, true, VEC, NT_GRAD>(a, sw, part, unused_n, inv_count<MODE>(N), mask_bits,
                                                          n_bits);
            const float part_wg = block_sum(part, red_f);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
        } else {
            // Forward only: one streaming pass, no exchange.
            stream_tiles<T, MODE, HAS_KL, false, VEC>(a, sw, part, n_lane, 1.0f);
            const float part_wg = block_sum(part, red_f);
            const uint32_t n_wg = block_sum(n_lane, red_u);
            if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
            if (blockIdx.x == 0) N = gather_counts();
        }
        if (blockIdx.x == 0) {
            const float total = gather_partials(nothing);
            if (threadIdx.x == 0) write_results<MODE>(a, total, N);
        }
    }
}

// ----------------------------------------------------------------------------- GRPO
//
// GRPO scales row r's terms by 1 / (max(n_r, 1) * bs), n_r the row's own
// valid count (the card's per-row denominator).  Worker w owns the contiguous
// tiles [w * per, min((w + 1) * per, tiles)), slots [lo_w, hi_w) (its run;
// per = 1 in the one-tile kernels), and reads each of its mask bytes once.
//  * A row inside the run other than its first and last is counted and
//    scaled by the worker alone.
//  * Of the run's first and last row the worker publishes the valid count as
//    soon as its masks are in (cnt and, when the run ends in another row,
//    tail entries), and, once the terms are formed, the count with the
//    unscaled sum of terms inside the run (hpair / tpair entries) and the sum
//    over its other rows (par).
//  * Workgroup 0 reads every worker's pairs (computing those not published
//    within the steal limit itself, with the worker's code) and closes the
//    rows that cross runs: each thread takes consecutive workers and adds up
//    the pieces of the rows they share, a segmented scan over the threads
//    carries the rows that run on (the counts exactly, the sums in one fixed
//    tree), and each row's term sum / (max(n, 1) * bs) is taken where the row
//    ends.  The loss thus needs one cross-workgroup hop after the terms.
//  * A fwd+bwd worker needs the whole count of its run's first and last row
//    for the gradient's scale when they extend beyond the run: it gathers the
//    other workers' counts of the row (cnt / tail entries), counting from the
//    mask any not published within the steal limit.  Where seq_len divides
//    the tile no row crosses a tile boundary, and no count is exchanged.

// Threads that publish a worker's entries: the counts from wavefronts 2 and 3
// (a gather of up to 128 entries reads from wavefronts 0 and 1 only, and a
// poll must not wait for the write-through of an earlier store of its own
// wavefront), the pairs and the inner sum from wavefront 1, which then only
// stores.
constexpr uint32_t kHeadThread = 128;
constexpr uint32_t kTailThread = 192;

struct Run {
    uint32_t lo, hi;   // slots of a worker's run
};
__device__ __forceinline__ Run run_of(const Args& a, uint32_t v, uint32_t tile_v) {
    const uint32_t lo = v * a.per * tile_v;    // < slots for every worker v < grid
    const uint32_t hi = lo + a.per * tile_v;   // per * tile_v <= 2^22, so no wrap
    return Run{lo, hi < uint32_t(a.slots) ? hi : uint32_t(a.slots)};
}

__device__ __forceinline__ float row_scale(const Args& a, uint32_t n) {
    return 1.0f / (float(n > 0 ? n : 1u) * float(a.bs));
}

// What a worker contributes: the valid counts and unscaled sums of terms of
// its run's first and last row inside the run (the last equal to the first
// when the run lies in one row), and the sum over its other rows, each
// scaled by its row's count.
struct GrpoPart {
    uint32_t n_first, n_last;
    float s_first, s_last, inner;
};

// Valid slots of the mask in [b0, b1), in every thread (uniform arguments).
__device__ __forceinline__ uint32_t count_mask(const Args& a, uint32_t b0, uint32_t b1, uint32_t* red) {
    uint32_t n = 0;
    for (uint32_t c = (b0 & ~15u) + threadIdx.x * 16u; c < b1; c += kThreads * 16u) {
        Mask<16> m;
        m.load(a.mask, c, uint32_t(a.slots));
        const uint32_t cut_lo = b0 > c ? b0 - c : 0u;             // < 16
        const uint32_t cut_hi = b1 - c < 16u ? b1 - c : 16u;      // >= 1
        n += __builtin_popcount(m.bits() & ((1u << cut_hi) - 1u) & ~((1u << cut_lo) - 1u));
    }
    return block_sum(n, red);
}

// One lane's valid slots (mask bits `bits`, slots s .. s+VEC-1) in row rf (low
// 16 bits) and, when rl != rf, in row rl (high 16 bits): rf and rl are the
// first and last row of the lane's tile, so the workgroup sum holds the tile's
// counts of both (at most kThreads * VEC = 4096 each, no carry).
template <int VEC>
__device__ __forceinline__ uint32_t lane_ends(const Args& a, uint32_t s, uint32_t bits, uint32_t rf, uint32_t rl) {
    const uint32_t T = uint32_t(a.seq_len);
    const uint32_t e = (rf + 1u) * T;                          // end of row rf
    const uint32_t k = e > s ? (e - s < uint32_t(VEC) ? e - s : uint32_t(VEC)) : 0u;
    uint32_t v = __builtin_popcount(bits & ((1u << k) - 1u));
    if (rl != rf) {
        const uint32_t b = rl * T;                             // start of row rl
        const uint32_t j = b > s ? (b - s < uint32_t(VEC) ? b - s : uint32_t(VEC)) : 0u;
        v |= uint32_t(__builtin_popcount(bits >> j)) << 16;
    }
    return v;
}

// The same for a lane of E-slot chunks (`bits` in the lane's element order):
// the sum of each chunk's counts.
template <int VEC, int E>
__device__ __forceinline__ uint32_t lane_ends_chunked(const Args& a, uint32_t s, uint32_t bits, uint32_t rf,
                                                      uint32_t rl) {
    if constexpr (E == VEC) {
        return lane_ends<VEC>(a, s, bits, rf, rl);
    } else {
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < VEC / E; ++c)
            v += lane_ends<E>(a, chunk_slot<VEC, E>(s, c), (bits >> (c * E)) & ((1u << E) - 1u), rf, rl);
        return v;
    }
}

// The tile's valid count of each row it touches (rows rf .. rf + nrows - 1)
// into cnt[row - rf] (LDS), from every lane's mask bits (E-slot chunks).
template <int VEC, int E = VEC>
__device__ __forceinline__ void tile_rows(const Args& a, uint32_t s, uint32_t bits, uint32_t rf, uint32_t nrows,
                                          uint32_t* cnt) {
    __syncthreads();                           // cnt[] may still hold scales being read
    for (uint32_t i = threadIdx.x; i < nrows; i += kThreads) cnt[i] = 0;
    __syncthreads();
    const uint32_t T = uint32_t(a.seq_len);
#pragma unroll
    for (int ch = 0; ch < VEC / E; ++ch) {
        uint32_t b = E == VEC ? bits : (bits >> (ch * E)) & ((1u << E) - 1u);
        uint32_t pos = chunk_slot<VEC, E>(s, ch);
        uint32_t r = row_of(a, pos), e = (r + 1u) * T;
        while (b) {
            const uint32_t k = e - pos < uint32_t(E) ? e - pos : uint32_t(E);   // slots of row r from pos
            const uint32_t c = __builtin_popcount(b & ((1u << k) - 1u));
            if (c) atomicAdd(&cnt[r - rf], c);
            b = k < uint32_t(E) ? b >> k : 0u;
            pos += k;
            ++r;
            e += T;
        }
    }
    __syncthreads();
}

// Scales of the rows of the tile [s0, ...) (rows rf .. rf + nrows - 1) other
// than the run's first and last row (r0, r1), into row_lds: the tile's first
// and last row take the counts `first` and `last`, the others their count in
// row_lds.  OWN also writes the count of each such row that starts in the
// tile (those of r0 and r1 are written where their total is formed).
template <bool OWN>
__device__ __forceinline__ void row_scales(const Args& a, uint32_t s0, uint32_t rf, uint32_t nrows, uint32_t first,
                                           uint32_t last, uint32_t r0, uint32_t r1, uint32_t* row_lds) {
    const uint32_t T = uint32_t(a.seq_len);
    for (uint32_t i = threadIdx.x; i < nrows; i += kThreads) {
        const uint32_t r = rf + i;
        if (r == r0 || r == r1) continue;
        const uint32_t n = i == 0 ? first : i + 1 == nrows ? last : row_lds[i];
        row_lds[i] = __float_as_uint(row_scale(a, n));
        if (OWN && a.n_out && r * T >= s0) a.n_out[r] = n;
    }
    __syncthreads();
}

// GRPO terms of one lane (slots s .. s+VEC-1, or its E-slot chunks): slots of
// the run's first row r0 add c to h and of its last row r1 (!= r0) to t,
// unscaled; those of any other row add c * scale[row - rf] to `in`.  g: each
// slot's derivative times its row's scale, with g0 and g1 standing for those
// of r0 and r1.
template <typename T, bool HAS_KL, int VEC, int E = VEC>
__device__ __forceinline__ void grpo_lane(const Args& a, uint32_t s, const Lane<T, VEC>& L, uint32_t r0, uint32_t r1,
                                          float g0, float g1, const float* scale, uint32_t rf, float& h, float& t,
                                          float& in, float (&g)[VEC]) {
    constexpr int C = VEC / E;   // chunks of E consecutive slots
    // Sums in locals, each class added branch-free (an if-chain over the three
    // outputs becomes an indexed array in private memory).
    float sh = 0.0f, st = 0.0f, si = 0.0f;
    h = 0.0f;
    t = 0.0f;
    in = 0.0f;
    if (!L.m.any()) return;                   // every slot masked: g is never stored
    const uint32_t TL = uint32_t(a.seq_len);
    const uint32_t bs = uint32_t(a.bs);
    // Row r's class (0: r0, 1: r1, 2: other), gradient scale and term scale.
    auto info = [&](uint32_t row, int& cls, float& gs, float& cs) __attribute__((always_inline)) {
        if (row == r0) {
            cls = 0;
            gs = g0;
            cs = 1.0f;
        } else if (row == r1) {
            cls = 1;
            gs = g1;
            cs = 1.0f;
        } else {
            cls = 2;
            gs = scale[row - rf];
            cs = gs;
        }
    };
    auto add = [&](int cls, float sum, float cs) __attribute__((always_inline)) {
        sh += cls == 0 ? sum : 0.0f;
        st += cls == 1 ? sum : 0.0f;
        si += cls == 2 ? sum * cs : 0.0f;
    };
    uint32_t rc[C], pc[C];
    bool one_row = true;                      // every chunk within one row
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint32_t sc = chunk_row_slot(a, chunk_slot<VEC, E>(s, c));
        rc[c] = row_of(a, sc);
        pc[c] = sc - rc[c] * TL;
        one_row = one_row && pc[c] + E <= TL;
    }
    if (one_row) {
        // Each chunk's slots in one row (always, when seq_len is a multiple of
        // E): straight-line code, each chunk's sum scaled once.
#pragma unroll
        for (int c = 0; c < C; ++c) {
            int cls;
            float gs, cs;
            info(rc[c], cls, gs, cs);
            const Coef k = row_coef<kModeGRPO>(a, load_adv<T>(a.adv, rc[c]), 1.0f, 1.0f);
            float sum = 0.0f;
#pragma unroll
            for (int i = c * E; i < c * E + E; ++i) {
                float cv, gi;
                token_terms<kModeGRPO, HAS_KL>(L.lp.get(i), L.old.get(i), HAS_KL ? L.ref.get(i) : 0.0f, k, cv, gi);
                sum += L.m.valid(i) ? cv : 0.0f;
                g[i] = gi * gs;
            }
            add(cls, sum, cs);
        }
        h = sh;
        t = st;
        in = si;
        return;
    }
    // A chunk crosses a row boundary (rare: one lane per row end): slot by slot
    // on a copy of the lane that rotates down one slot per step (static register
    // indices, one slot's terms live), tracking the row, found afresh at each
    // chunk's first slot.
    Lane<T, VEC> R = L;
    Coef k{};
    int cls_a = 0;
    float gs_a = 0.0f, cs_a = 0.0f;
    uint32_t r = 0, pos = 0;
    float out[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = 0.0f;
#pragma unroll 1
    for (int i = 0; i < VEC; ++i) {
        if ((i & (E - 1)) == 0) {
            const uint32_t sc = chunk_row_slot(a, chunk_slot<VEC, E>(s, i / E));
            r = row_of(a, sc);
            pos = sc - r * TL;
            k = row_coef<kModeGRPO>(a, load_adv<T>(a.adv, r), 1.0f, 1.0f);
            info(r, cls_a, gs_a, cs_a);
        }
        float c, gi;
        token_terms<kModeGRPO, HAS_KL>(R.lp.get(0), R.old.get(0), HAS_KL ? R.ref.get(0) : 0.0f, k, c, gi);
        add(cls_a, R.m.valid(0) ? c : 0.0f, cs_a);
#pragma unroll
        for (int j = 0; j + 1 < VEC; ++j) out[j] = out[j + 1];
        out[VEC - 1] = gi * gs_a;
        R.m.rotate();
        R.lp.rotate();
        R.old.rotate();
        if constexpr (HAS_KL) R.ref.rotate();
        if (++pos == TL) {
            pos = 0;
            if (++r < bs) {
                k = row_coef<kModeGRPO>(a, load_adv<T>(a.adv, r), 1.0f, 1.0f);
                info(r, cls_a, gs_a, cs_a);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) g[i] = out[i];
    h = sh;
    t = st;
    in = si;
}

// ONE_TILE kernels (G = tiles + 1): workgroup 0 closes the rows and writes the
// loss, workgroup w > 0 is worker w - 1 and owns tile w - 1.  The others (G at
// most the co-resident capacity) give each workgroup a run of `per` tiles,
// which it walks twice: the masks first (eight loads in flight; the counts of
// each tile's first and last row, and the mask bits of its first
// kBitTilesGrpo tiles), then the planes; workgroup 0 then also closes the rows.
template <typename T, bool HAS_KL, bool WRITE_GRAD, int VEC, bool ONE_TILE, bool NT_GRAD = false>
// (16-bit planes: at most 128 VGPRs, four workgroups per compute unit, which
// the striding kernel's LDS allows; fp32 planes need more registers.)
__global__ void __launch_bounds__(kThreads, sizeof(T) == 2 ? 4 : 1) grpo_kernel(const Args a) {
    constexpr int MODE = kModeGRPO;
    constexpr uint32_t kTileV = kThreads * VEC;
    constexpr uint32_t kBits = ONE_TILE ? 1u : uint32_t(kBitTilesGrpo);
    constexpr int E = chunk_slots<T, VEC>();   // slots per chunk of a lane
    __shared__ float red_f[3 * kWaves];
    __shared__ uint32_t red_u[8 * kWaves];
    __shared__ uint32_t list[kThreads + 1];      // workers whose entries workgroup 0 computes itself
    __shared__ uint32_t list_r[kThreads + 1];    // row gathers (which also run inside those computations)
    // Per-row counts, then scales, of the current tile; at the end workgroup 0's
    // per-thread state for closing the rows (7 words per thread).
    constexpr uint32_t kRowLds = kTileV + 2u > 7u * kThreads ? kTileV + 2u : 7u * kThreads;
    __shared__ uint32_t row_lds[kRowLds];
    __shared__ uint32_t pieces[ONE_TILE ? 1 : kMaxPer];         // per owned tile: first | last << 16
    __shared__ uint16_t mask_bits[kBits * kThreads];

    const __amdgpu_buffer_rsrc_t view = entry_view(a.ws);
    const Tag tg = launch_tag();
    const Limits lim = read_limits(a.ws);
    const uint32_t slots = uint32_t(a.slots);
    const uint32_t TL = uint32_t(a.seq_len);
    const uint32_t W = ONE_TILE ? gridDim.x - 1 : gridDim.x;   // workers
    const uint32_t lane_off = threadIdx.x * VEC;
    const bool local_rows = kTileV % TL == 0u;                  // no row crosses a tile boundary
    const float* scale = reinterpret_cast<const float*>(row_lds);

    // Row r's whole count, given `own`, worker w's count of it: that alone when
    // the row lies within w's run, else plus the other workers' counts.
    auto row_count = [&](uint32_t w, uint32_t r, uint32_t own) __attribute__((always_inline)) -> uint32_t {
        const Run ru = run_of(a, w, kTileV);
        const uint32_t b0 = r * TL, b1 = b0 + TL;
        if (b0 >= ru.lo && b1 <= ru.hi) return own;
        const uint32_t va = b0 / kTileV / a.per, vb = (b1 - 1u) / kTileV / a.per;
        auto off = [&](uint32_t i) __attribute__((always_inline)) -> uint32_t {
            const uint32_t v = va + i;
            if (v == w) return kNoEntry;
            return row_of(a, run_of(a, v, kTileV).lo) == r ? cnt_off(v) : tail_off(v);
        };
        auto piece = [&](uint32_t i) __attribute__((always_inline)) -> uint32_t {
            const Run rv = run_of(a, va + i, kTileV);
            return count_mask(a, b0 > rv.lo ? b0 : rv.lo, b1 < rv.hi ? b1 : rv.hi, red_u);
        };
        return own + gather<uint32_t>(view, off, vb - va + 1u, tg, lim.steal_now(), list_r, red_u, piece, [] {});
    };
    // Publishes a worker's pairs and inner sum (OWN workers, wavefront 1; the
    // last row's pair and the inner sum only when the run ends in another row).
    auto publish_sums = [&](uint32_t w, uint32_t n_first, uint32_t n_last, const float (&v)[3], bool multi)
        __attribute__((always_inline)) {
        if (threadIdx.x == kPartialThread) publish_pair(view, hpair_off(w), tg, n_first, __float_as_uint(v[0]));
        if (multi && threadIdx.x == kPartialThread + 1u)
            publish_pair(view, tpair_off(w), tg, n_last, __float_as_uint(v[1]));
        if (multi && threadIdx.x == kPartialThread + 2u) publish(view, par_off(w), tg, __float_as_uint(v[2]));
    };

    // Worker w of a one-tile kernel, whole: OWN (the worker itself) publishes its
    // entries and writes the gradient and the counts of its inner rows;
    // otherwise (workgroup 0 standing in for it) only the values are formed.
    auto one_tile = [&](uint32_t w, auto own) __attribute__((always_inline)) -> GrpoPart {
        constexpr bool OWN = decltype(own)::value;
        const uint32_t s0 = w * kTileV, s1 = s0 + kTileV < slots ? s0 + kTileV : slots;
        const uint32_t s = s0 + lane_off;
        Lane<T, VEC> L;
        (void)load_lane_count<T, MODE, HAS_KL, VEC, VEC == kVecSmall, true, E>(a, s, L);
        const uint32_t bits = L.m.bits();
        const uint32_t rf = row_of(a, s0), rl = row_of(a, s1 - 1u), nrows = rl - rf + 1u;
        const uint32_t ends = block_sum(lane_ends_chunked<VEC, E>(a, s, bits, rf, rl), red_u);
        const uint32_t n_first = ends & 0xFFFFu, n_last = rl != rf ? ends >> 16 : n_first;
        if (OWN && threadIdx.x == kHeadThread) publish(view, cnt_off(w), tg, n_first);
        if (OWN && rl != rf && threadIdx.x == kTailThread) publish(view, tail_off(w), tg, n_last);
        if (nrows > 2u) tile_rows<VEC, E>(a, s, bits, rf, nrows, row_lds);
        else __syncthreads();                  // row_lds may still hold scales being read
        row_scales<OWN>(a, s0, rf, nrows, 0u, 0u, rf, rl, row_lds);
        float h, t, in;
        float g[VEC];
        grpo_lane<T, HAS_KL, VEC, E>(a, s, L, rf, rl, 1.0f, 1.0f, scale, rf, h, t, in, g);
        float v[3] = {h, t, in};
        block_sum_n<3>(v, red_f);
        if (OWN) publish_sums(w, n_first, n_last, v, rl != rf);
        if constexpr (OWN && WRITE_GRAD) {
            // The first and last row's scales, from their whole counts.
            const float f0 = row_scale(a, row_count(w, rf, n_first));
            const float f1 = rl != rf ? row_scale(a, row_count(w, rl, n_last)) : f0;
            const uint32_t e0 = (rf + 1u) * TL, b1 = rl * TL;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const uint32_t p = chunk_slot<VEC, E>(s, i / E) + uint32_t(i % E);   // slot of element i
                g[i] *= p < e0 ? f0 : (rl != rf && p >= b1 ? f1 : 1.0f);
            }
            store_grad<T, VEC, false, false, true, E>(a, s, L.m, g, 1.0f);
        }
        return GrpoPart{n_first, n_last, v[0], v[1], v[2]};
    };

    // Worker w of a striding kernel, whole (OWN as above).
    auto run = [&](uint32_t w, auto own) __attribute__((always_inline)) -> GrpoPart {
        constexpr bool OWN = decltype(own)::value;
        const uint32_t t_lo = w * a.per;
        const uint32_t nt = (t_lo + a.per < a.tiles ? t_lo + a.per : a.tiles) - t_lo;
        const Run ru = run_of(a, w, kTileV);
        const uint32_t r0 = row_of(a, ru.lo), r1 = row_of(a, ru.hi - 1u);
        // Row r's count in this run: the sum of its owned tiles' counts of it.
        auto run_piece = [&](uint32_t r) __attribute__((always_inline)) -> uint32_t {
            const uint32_t b0 = r * TL, b1 = b0 + TL;
            const uint32_t ja = b0 / kTileV > t_lo ? b0 / kTileV - t_lo : 0u;
            const uint32_t jb = (b1 - 1u) / kTileV - t_lo < nt - 1u ? (b1 - 1u) / kTileV - t_lo : nt - 1u;
            uint32_t c = 0;
            for (uint32_t j = ja + threadIdx.x; j <= jb; j += kThreads) {
                const uint32_t p = pieces[j];
                c += row_of(a, (t_lo + j) * kTileV) == r ? (p & 0xFFFFu) : (p >> 16);
            }
            return block_sum(c, red_u);
        };
        uint32_t n_first = 0, n_last = 0;      // counts of rows r0 and r1 in the run
        float f0 = 1.0f, f1 = 1.0f;            // their gradient scales
        uint32_t n_bits = 0;
        if (!local_rows) {
            for (uint32_t j0 = 0; j0 < nt; j0 += 8u) {
                Mask<VEC> m[8];
                if (j0 + 8u <= nt && (t_lo + j0 + 8u) * kTileV <= slots) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        m[u].template load<true, false>(a.mask, (t_lo + j0 + u) * kTileV + lane_off, slots);
                } else {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (j0 + u < nt) m[u].template load<true>(a.mask, (t_lo + j0 + u) * kTileV + lane_off, slots);
                }
                uint32_t e[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    e[u] = 0;
                    if (j0 + u < nt) {
                        const uint32_t s0 = (t_lo + j0 + u) * kTileV;
                        const uint32_t s1 = s0 + kTileV < slots ? s0 + kTileV : slots;
                        const uint32_t b = m[u].bits();
                        if (j0 + u < kBits) mask_bits[(j0 + u) * kThreads + threadIdx.x] = uint16_t(b);
                        e[u] = lane_ends<VEC>(a, s0 + lane_off, b, row_of(a, s0), row_of(a, s1 - 1u));
                    }
                }
                block_sum_n<8>(e, red_u);
                if (threadIdx.x == 0) {
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (j0 + u < nt) pieces[j0 + u] = e[u];
                }
            }
            n_bits = nt < kBits ? nt : kBits;
            __syncthreads();
            n_first = run_piece(r0);
            n_last = r1 != r0 ? run_piece(r1) : n_first;
            if (OWN && threadIdx.x == kHeadThread) publish(view, cnt_off(w), tg, n_first);
            if (OWN && r1 != r0 && threadIdx.x == kTailThread) publish(view, tail_off(w), tg, n_last);
            if (OWN && WRITE_GRAD) {
                f0 = row_scale(a, row_count(w, r0, n_first));
                f1 = r1 != r0 ? row_scale(a, row_count(w, r1, n_last)) : f0;
            }
        }
        float v[3] = {0.0f, 0.0f, 0.0f};
        uint32_t cached_r = 0xFFFFFFFFu, cached_n = 0;
        Mask<VEC> next;
        if (n_bits == 0) next.template load<true, true, E>(a.mask, t_lo * kTileV + lane_off, slots);
        for (uint32_t j = 0; j < nt; ++j) {
            const uint32_t s0 = (t_lo + j) * kTileV, s1 = s0 + kTileV < slots ? s0 + kTileV : slots;
            const uint32_t s = s0 + lane_off;
            Lane<T, VEC> L;
            if (j < n_bits) L.m.from_bits(chunk_bits<VEC, E>(mask_bits + j * kThreads));
            else L.m = next;
            if (j + 1u < nt && j + 1u >= n_bits)
                next.template load<true, true, E>(a.mask, s0 + kTileV + lane_off, slots);
            load_planes<T, MODE, HAS_KL, VEC, true, true, E>(a, s, L);
            const uint32_t rf = row_of(a, s0), rl = row_of(a, s1 - 1u), nrows = rl - rf + 1u;
            uint32_t first = 0, last = 0;      // the tile's counts of its first and last row
            if (nrows > 2u) {
                tile_rows<VEC, E>(a, s, L.m.bits(), rf, nrows, row_lds);
                first = row_lds[0];
                last = row_lds[nrows - 1u];
            } else {
                const uint32_t ends =
                    local_rows ? block_sum(lane_ends_chunked<VEC, E>(a, s, L.m.bits(), rf, rl), red_u) : pieces[j];
                first = ends & 0xFFFFu;
                last = rl != rf ? ends >> 16 : first;
            }
            if (local_rows) {
                // Rows lie in their tile: the run's first and last row are counted here.
                if (j == 0) n_first = first;
                if (j + 1u == nt) n_last = last;
                if (OWN && WRITE_GRAD) {
                    if (j == 0) f0 = row_scale(a, first);
                    if (j + 1u == nt) f1 = row_scale(a, last);
                }
            } else {
                // A row other than r0 and r1 that crosses a tile boundary lies in the
                // run: its count is the sum of the run's tiles' counts of it.
                auto whole = [&](uint32_t r, uint32_t here) __attribute__((always_inline)) -> uint32_t {
                    if (r == r0 || r == r1 || (r * TL >= s0 && (r + 1u) * TL <= s1)) return here;
                    if (r != cached_r) {
                        cached_n = run_piece(r);
                        cached_r = r;
                    }
                    return cached_n;
                };
                first = whole(rf, first);
                last = rl != rf ? whole(rl, last) : first;
            }
            if (nrows <= 2u) __syncthreads();  // row_lds may still hold scales being read
            row_scales<OWN>(a, s0, rf, nrows, first, last, r0, r1, row_lds);
            float h, t, in;
            float g[VEC];
            grpo_lane<T, HAS_KL, VEC, E>(a, s, L, r0, r1, f0, f1, scale, rf, h, t, in, g);
            v[0] += h;
            v[1] += t;
            v[2] += in;
            if constexpr (OWN && WRITE_GRAD) store_grad<T, VEC, false, NT_GRAD, true, E>(a, s, L.m, g, 1.0f);
        }
        block_sum_n<3>(v, red_f);
        if (OWN) {
            if (local_rows) {
                if (threadIdx.x == kHeadThread) publish(view, cnt_off(w), tg, n_first);
                if (r1 != r0 && threadIdx.x == kTailThread) publish(view, tail_off(w), tg, n_last);
            }
            publish_sums(w, n_first, n_last, v, r1 != r0);
        }
        return GrpoPart{n_first, n_last, v[0], v[1], v[2]};
    };

    // Workgroup 0: every worker's pairs (computed here when not published in
    // time), the rows that cross runs closed, the loss (in every thread of
    // wavefront 0).  Thread t takes workers t*k .. t*k + k - 1, polled two at a
    // time, and adds up the pieces of the rows they share; wavefront 0 then
    // carries the rows that run on past a thread's workers (a segmented scan
    // over the threads), closes them, and sums the loss.
    auto close_rows = [&]() __attribute__((always_inline)) -> float {
        const uint32_t k = (W + kThreads - 1u) / kThreads;
        float acc = 0.0f;
        // The row being summed (its pieces in this thread's workers so far) and
        // whether it began before them; a row that did and ended here waits for
        // the pieces of the earlier threads.
        bool have = false, from_left = false, left = false;
        uint32_t cur_row = 0, cur_n = 0, left_row = 0, left_n = 0;
        float cur_s = 0.0f, left_s = 0.0f;
        auto close = [&](uint32_t row, uint32_t n, float sum) __attribute__((always_inline)) {
            acc += sum * row_scale(a, n);
            if (a.n_out) a.n_out[row] = n;
        };
#pragma unroll 1
        for (uint32_t j0 = 0; j0 < k; j0 += 2u) {
            // Entries of workers j0 and j0 + 1 of this thread: first-row pair,
            // last-row pair and inner sum (the last two only when the run ends in
            // another row).
            uint32_t at[6], x[6] = {0u, 0u, 0u, 0u, 0u, 0u}, y[6] = {0u, 0u, 0u, 0u, 0u, 0u}, miss = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t v = threadIdx.x * k + j0 + u;
                const bool live = j0 + u < k && v < W;
                const Run ru = run_of(a, live ? v : 0u, kTileV);
                const bool multi = live && row_of(a, ru.lo) != row_of(a, ru.hi - 1u);
                at[3 * u] = live ? hpair_off(v) : kNoEntry;
                at[3 * u + 1] = multi ? tpair_off(v) : kNoEntry;
                at[3 * u + 2] = multi ? par_off(v) : kNoEntry;
            }
#pragma unroll
            for (int q = 0; q < 6; ++q)
                if (at[q] != kNoEntry) miss |= 1u << q;
            auto poll = [&]() __attribute__((always_inline)) {
                u32x4 e[6];
#pragma unroll
                for (int q = 0; q < 6; ++q)
                    e[q] = __builtin_amdgcn_raw_buffer_load_b128(view, (miss >> q) & 1u ? at[q] : 0u, 0, kCoherent);
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    const bool pair = q % 3 != 2;
                    if (((miss >> q) & 1u) && e[q][1] == tg.t0 && e[q][3] == tg.t1 && (pair || e[q][0] == e[q][2])) {
                        x[q] = e[q][0];
                        y[q] = e[q][2];
                        miss &= ~(1u << q);
                    }
                }
            };
            poll();
            if (miss) {
                const uint64_t t0 = wall_clock64();
                const uint32_t limit = lim.steal_now();
                for (uint32_t n = 1; miss; ++n) {
                    poll_pause<1>();           // (one workgroup polls: a short pause)
                    poll();
                    if ((n & 7u) == 0u && uint64_t(wall_clock64()) - t0 > limit) break;
                }
            }
            // Workers still missing: their values computed here, one at a time.
            if (__syncthreads_or(miss != 0u)) {
                if (threadIdx.x == 0) list[kThreads] = 0;
                __syncthreads();
                if (miss & 7u) list[atomicAdd(&list[kThreads], 1u)] = threadIdx.x * 2u;
                if (miss & 56u) list[atomicAdd(&list[kThreads], 1u)] = threadIdx.x * 2u + 1u;
                __syncthreads();
                const uint32_t n_list = list[kThreads];
#pragma unroll 1
                for (uint32_t q = 0; q < n_list; ++q) {
                    const uint32_t th = list[q] >> 1, u = list[q] & 1u;
                    GrpoPart p;
                    if constexpr (ONE_TILE) p = one_tile(th * k + j0 + u, std::false_type{});
                    else p = run(th * k + j0 + u, std::false_type{});
                    if (threadIdx.x == th) {
                        const uint32_t b = u ? 3u : 0u;
#pragma unroll
                        for (int c = 0; c < 6; c += 3)
                            if (uint32_t(c) == b) {
                                x[c] = p.n_first;
                                y[c] = __float_as_uint(p.s_first);
                                x[c + 1] = p.n_last;
                                y[c + 1] = __float_as_uint(p.s_last);
                                x[c + 2] = __float_as_uint(p.inner);
                            }
                    }
                }
                __syncthreads();               // list[] is reused by the next batch
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t v = threadIdx.x * k + j0 + u;
                if (!(j0 + u < k && v < W)) continue;
                const Run ru = run_of(a, v, kTileV);
                const uint32_t r0 = row_of(a, ru.lo), r1 = row_of(a, ru.hi - 1u);
                const bool multi = r1 != r0;
                const bool cont_in = r0 * TL < ru.lo;          // the first row began in an earlier run
                const bool cont_out = (r1 + 1u) * TL > ru.hi;  // the last row goes on into a later run
                const float hs = __uint_as_float(y[3 * u]);
                if (!cont_in || !have) {
                    from_left = cont_in;       // (only the first worker's row can begin before them)
                    cur_row = r0;
                    cur_n = x[3 * u];
                    cur_s = hs;
                    have = true;
                } else {
                    cur_n = cur_n + x[3 * u];
                    cur_s = cur_s + hs;
                }
                if (multi || !cont_out) {      // the first row ends in this run
                    if (from_left) {
                        left = true;
                        left_row = cur_row;
                        left_n = cur_n;
                        left_s = cur_s;
                    } else {
                        close(cur_row, cur_n, cur_s);
                    }
                    have = false;
                    from_left = false;
                }
                if (multi) {
                    acc += __uint_as_float(x[3 * u + 2]);
                    cur_row = r1;
                    cur_n = x[3 * u + 1];
                    cur_s = __uint_as_float(y[3 * u + 1]);
                    have = true;
                    if (!cont_out) {
                        close(cur_row, cur_n, cur_s);
                        have = false;
                    }
                }
            }
        }
        // Carry the rows that run on across threads: a segmented scan over the
        // threads in worker order.  Thread t's element is the row it passes on
        // (its pieces; it restarts the carry unless its workers all lie in a row
        // begun before them); the carry into thread t then completes the row
        // begun before its workers and ended in them.  Each wavefront scans its
        // 64 lanes with DPP lane moves (within rows of 16 by 1, 2, 4, 8 lanes,
        // then across rows), the wavefronts' totals meet in LDS, and each
        // wavefront folds those of the wavefronts before it into its lanes'
        // carries: a fixed order, so the loss is deterministic.
        const uint32_t l = threadIdx.x & 63u, wv = threadIdx.x >> 6;
        uint32_t f = have && from_left ? 0u : 1u;
        uint32_t n = have ? cur_n : 0u;
        float sm = have ? cur_s : 0.0f;
        auto step = [&](auto ctl, bool take) __attribute__((always_inline)) {
            constexpr int kCtl = decltype(ctl)::value & 0xFFF, kRows = decltype(ctl)::value >> 12;
            const uint32_t pf = dpp_move<kCtl, kRows>(f);
            const uint32_t pn = dpp_move<kCtl, kRows>(n);
            const float ps = __uint_as_float(dpp_move<kCtl, kRows>(__float_as_uint(sm)));
            if (take && !f) {
                n = pn + n;
                sm = ps + sm;
                f = pf;
            }
        };
        step(std::integral_constant<int, 0xF111>{}, (l & 15u) >= 1u);    // row_shr:1
        step(std::integral_constant<int, 0xF112>{}, (l & 15u) >= 2u);    // row_shr:2
        step(std::integral_constant<int, 0xF114>{}, (l & 15u) >= 4u);    // row_shr:4
        step(std::integral_constant<int, 0xF118>{}, (l & 15u) >= 8u);    // row_shr:8
        step(std::integral_constant<int, 0xA142>{}, (l & 16u) != 0u);    // row_bcast:15
        step(std::integral_constant<int, 0xC143>{}, (l & 32u) != 0u);    // row_bcast:31
        // the lane's exclusive prefix within its wavefront (lane 0: nothing)
        uint32_t ef = dpp_move<0x138>(f), en = dpp_move<0x138>(n);       // wave_shr:1
        float es = __uint_as_float(dpp_move<0x138>(__float_as_uint(sm)));
        __syncthreads();                       // red_u / red_f are free
        if (l == 63u) {
            red_u[2u * wv] = f;
            red_u[2u * wv + 1u] = n;
            red_f[wv] = sm;
        }
        __syncthreads();
        uint32_t cf = 0, cn = 0;               // the carry into this wavefront
        float cs = 0.0f;
        for (uint32_t v = 0; v < wv; ++v) {
            const uint32_t vf = red_u[2u * v], vn = red_u[2u * v + 1u];
            const float vs = red_f[v];
            cn = vf ? vn : cn + vn;
            cs = vf ? vs : cs + vs;
            cf |= vf;
        }
        if (!ef) {
            en = cn + en;
            es = cs + es;
        }
        // A row begun before this thread's workers and ended in them: the carry,
        // then its own pieces.
        float loss = acc;
        if (left) {
            const uint32_t n_row = en + left_n;
            loss += (es + left_s) * row_scale(a, n_row);
            if (a.n_out) a.n_out[left_row] = n_row;
        }
        (void)cf;
        return block_sum(loss, red_f);
    };

    if constexpr (ONE_TILE) {
        if (blockIdx.x == 0) {
            const float total = close_rows();
            if (threadIdx.x == 0) *a.loss = total;
            return;
        }
        (void)one_tile(blockIdx.x - 1u, std::true_type{});
    } else {
        (void)run(blockIdx.x, std::true_type{});
        if (blockIdx.x == 0) {
            const float total = close_rows();
            if (threadIdx.x == 0) *a.loss = total;
        }
    }
}

// ----------------------------------------------------------------------------- host-side table

template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD>
static const void* kernel_ptr(int shape) {
    switch (shape) {
    case kShapeSmall: return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, WRITE_GRAD, kVecSmall, true>);
    case kShapeLarge: return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, WRITE_GRAD, kVecLarge, true>);
    case kShapeStream: return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, WRITE_GRAD, kVecLarge, false>);
    case kShapeStreamNt:   // (no gradient: the same kernel as kShapeStream)
        if constexpr (WRITE_GRAD)
            return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, true, kVecLarge, false, true>);
        else
            return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, false, kVecLarge, false>);
    }
    return nullptr;
}

template <typename T, bool HAS_KL, bool WRITE_GRAD>
static const void* grpo_ptr(int shape) {
    switch (shape) {
    case kShapeSmall: return reinterpret_cast<const void*>(&grpo_kernel<T, HAS_KL, WRITE_GRAD, kVecSmall, true>);
    case kShapeLarge: return reinterpret_cast<const void*>(&grpo_kernel<T, HAS_KL, WRITE_GRAD, kVecLarge, true>);
    case kShapeStream: return reinterpret_cast<const void*>(&grpo_kernel<T, HAS_KL, WRITE_GRAD, kVecLarge, false>);
    case kShapeStreamNt:
        if constexpr (WRITE_GRAD)
            return reinterpret_cast<const void*>(&grpo_kernel<T, HAS_KL, true, kVecLarge, false, true>);
        else
            return reinterpret_cast<const void*>(&grpo_kernel<T, HAS_KL, false, kVecLarge, false>);
    }
    return nullptr;
}

template <typename T>
const void* pick_typed(int mode, bool has_kl, bool write_grad, int shape) {
    switch (mode) {
    case kModeBNPO:
        if (has_kl) return write_grad ? kernel_ptr<T, kModeBNPO, true, true>(shape) : kernel_ptr<T, kModeBNPO, true, false>(shape);
        return write_grad ? kernel_ptr<T, kModeBNPO, false, true>(shape) : kernel_ptr<T, kModeBNPO, false, false>(shape);
    case kModeGRPO:
        if (has_kl) return write_grad ? grpo_ptr<T, true, true>(shape) : grpo_ptr<T, true, false>(shape);
        return write_grad ? grpo_ptr<T, false, true>(shape) : grpo_ptr<T, false, false>(shape);
    case kModeRKL:
        return write_grad ? kernel_ptr<T, kModeRKL, true, true>(shape) : kernel_ptr<T, kModeRKL, true, false>(shape);
    }
    return nullptr;
}

}  // namespace rlpl
