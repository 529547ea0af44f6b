// Fused forward+backward PPO-family policy losses for gfx950 (MI355X).
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
//  * A grid of G workgroups (at most what the device holds at once):
//    workgroup 0 coordinates, workers take tiles w, w+(G-1), ...  Per-token
//    math is fp32 in registers and branch-free: every slot of a lane is
//    computed and masked slots are selected away (their values never reach
//    a result).
//  * Reductions: per-lane sums -> wavefront shuffle tree -> LDS across the
//    4 waves -> one partial per worker in the workspace.  The coordinator
//    sums the partials in worker order, so the loss is deterministic and
//    identical between the fwd+bwd and forward-only kernels.
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
//  * GRPO needs only each row's own count: a workgroup counts the mask of
//    every row its tile touches into LDS (no cross-workgroup exchange before
//    the gradient is scaled), as the card's one-block-per-row design does.
//  * Plane loads wait for the mask and are skipped for lanes whose mask
//    bytes are all zero; when streaming several tiles per workgroup, the next
//    tile's mask is fetched while the current tile is computed.
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

// VEC mask bytes of one lane.
template <int VEC>
struct Mask {
    Dwords<VEC / 4> d;
    __device__ __forceinline__ void load(const uint8_t* __restrict__ mask, uint32_t s, uint32_t slots) {
        if (s + VEC <= slots) {
            d.load(mask + s);
        } else {
#pragma unroll
            for (int i = 0; i < VEC / 4; ++i) d.w[i] = 0;
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                if (s + k < slots) d.w[k >> 2] |= uint32_t(mask[s + k]) << (8 * (k & 3));
        }
    }
    __device__ __forceinline__ bool any() const {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) o |= d.w[i];
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
template <typename T, int MODE, bool HAS_KL, int VEC, bool SPEC>
__device__ __forceinline__ uint32_t load_lane_count(const Args& a, uint32_t s, Lane<T, VEC>& L) {
    const uint32_t slots = uint32_t(a.slots);
    if (s + VEC <= slots) {
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

// Loads one lane's planes once its mask has arrived; skipped when all of the
// mask's bytes are zero.
template <typename T, int MODE, bool HAS_KL, int VEC>
__device__ __forceinline__ void load_planes(const Args& a, uint32_t s, Lane<T, VEC>& L) {
    if (L.m.any()) {
        L.lp.load(static_cast<const T*>(a.lp), s, a.slots);
        if constexpr (MODE != kModeRKL) L.old.load(static_cast<const T*>(a.old), s, a.slots);
        if constexpr (HAS_KL) L.ref.load(static_cast<const T*>(a.ref), s, a.slots);
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

template <typename T, int MODE, bool HAS_KL, int VEC>
__device__ __forceinline__ float lane_terms(const Args& a, uint32_t s, const Lane<T, VEC>& L,
                                            const float* row_scale, uint32_t row_base, float gscale,
                                            float (&g)[VEC]) {
    float part = 0.0f;
    if (!L.m.any()) return part;
    const uint32_t T_len = uint32_t(a.seq_len);
    uint32_t r = row_of(a, s);
    uint32_t t = s - r * T_len;
    float A = 0.0f, rs = 1.0f;
    if constexpr (MODE != kModeRKL) A = load_adv<T>(a.adv, r);
    if constexpr (MODE == kModeGRPO) rs = row_scale[r - row_base];
    Coef k = row_coef<MODE>(a, A, rs, gscale);
    if (MODE == kModeRKL || t + VEC <= T_len) {
        // All VEC slots in one row (always, when seq_len is a multiple of VEC; the
        // reverse-KL terms do not depend on the row at all): branch-free.
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            float c, gi;
            token_terms<MODE, HAS_KL>(L.lp.get(i), MODE == kModeRKL ? 0.0f : L.old.get(i),
                                      HAS_KL ? L.ref.get(i) : 0.0f, k, c, gi);
            if constexpr (MODE == kModeGRPO) { c *= rs; gi *= rs; }
            part += L.m.valid(i) ? c : 0.0f;
            g[i] = gi;
        }
    } else {
        // The lane crosses a row boundary: slot by slot, tracking the row.  A rolled
        // loop keeps one slot's terms live (this path is rare: only lanes that
        // straddle a row end); it always works on slot 0 of a copy of the lane
        // that rotates down one slot per step, and the derivatives rotate in at
        // the top, so that every register index stays static.
        Lane<T, VEC> R = L;
        float out[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) out[i] = 0.0f;
#pragma unroll 1
        for (int i = 0; i < VEC; ++i) {
            float c, gi;
            token_terms<MODE, HAS_KL>(R.lp.get(0), MODE == kModeRKL ? 0.0f : R.old.get(0),
                                      HAS_KL ? R.ref.get(0) : 0.0f, k, c, gi);
            if constexpr (MODE == kModeGRPO) { c *= rs; gi *= rs; }
            part += R.m.valid(0) ? c : 0.0f;
#pragma unroll
            for (int j = 0; j + 1 < VEC; ++j) out[j] = out[j + 1];
            out[VEC - 1] = gi;
            R.m.rotate();
            R.lp.rotate();
            if constexpr (MODE != kModeRKL) R.old.rotate();
            if constexpr (HAS_KL) R.ref.rotate();
            if (++t == T_len) {
                t = 0;
                ++r;
                if (r < uint32_t(a.bs)) {
                    if constexpr (MODE != kModeRKL) A = load_adv<T>(a.adv, r);
                    if constexpr (MODE == kModeGRPO) rs = row_scale[r - row_base];
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
template <typename T, int VEC, bool SCALE>
__device__ __forceinline__ void store_grad(const Args& a, uint32_t s, const Mask<VEC>& m,
                                           const float (&g)[VEC], float scale) {
    float v[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) v[k] = m.valid(k) ? (SCALE ? g[k] * scale : g[k]) : 0.0f;
    store_values<T, VEC>(static_cast<T*>(a.grad), s, a.slots, v);
}


// ----------------------------------------------------------------------------- GRPO row counts

// For the tile [s0, s1): counts the mask of every row the tile touches into
// cnt[row - r_first] (LDS), then turns each count into the row's gradient
// scale 1 / (max(n_r, 1) * bs) in place.  Writes n_out for rows that start in
// the tile (exactly one tile per row does).
__device__ __forceinline__ void grpo_row_scales(const Args& a, uint32_t s0, uint32_t s1, uint32_t* cnt,
                                uint32_t& r_first) {
    const uint32_t T = uint32_t(a.seq_len);
    r_first = row_of(a, s0);
    const uint32_t r_last = row_of(a, s1 - 1);
    const uint32_t nrows = r_last - r_first + 1;
    const uint32_t e0 = r_first * T, e1 = (r_last + 1) * T;
    // cnt[] still holds the previous tile's scales, which other threads may be
    // reading: clear it only once every thread is done with them.
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nrows; i += kThreads) cnt[i] = 0;
    __syncthreads();
    for (uint32_t c = (e0 & ~15u) + threadIdx.x * 16u; c < e1; c += kThreads * 16u) {
        Mask<16> m;
        m.load(a.mask, c, uint32_t(a.slots));
        if (!m.any()) continue;
        uint32_t r = row_of(a, c);
        uint32_t row_end = (r + 1) * T;
        uint32_t run = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t i = c + k;
            if (i == row_end) {
                if (run && r >= r_first && r <= r_last) atomicAdd(&cnt[r - r_first], run);
                run = 0;
                ++r;
                row_end += T;
            }
            if (i >= e0 && i < e1 && m.valid(k)) ++run;
        }
        if (run && r >= r_first && r <= r_last) atomicAdd(&cnt[r - r_first], run);
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nrows; i += kThreads) {
        const uint32_t n = cnt[i];
        cnt[i] = __float_as_uint(1.0f / (float(n > 0 ? n : 1u) * float(a.bs)));
        const uint32_t r = r_first + i;
        if (a.n_out && r * T >= s0 && r * T < s1) a.n_out[r] = n;
    }
    __syncthreads();
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

// Streams worker `worker`'s tiles (worker, worker+G, ... for G workers): per
// tile, the lane's terms, its count and (WRITE_GRAD) the scaled gradient.  The
// plane loads wait for the mask, and the next tile's mask is fetched during
// the current tile.
template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD, int VEC>
__device__ __forceinline__ void stream_tiles(const Args& a, uint32_t worker, uint32_t G,
                                             uint32_t* row_lds, float& part, uint32_t& n_lane,
                                             float scale, const uint16_t* bits = nullptr,
                                             uint32_t n_bits = 0) {
    constexpr uint32_t kTileV = kThreads * VEC;
    const uint32_t lane_off = threadIdx.x * VEC;
    const uint32_t slots = uint32_t(a.slots);
    uint32_t tile = worker;
    // The worker's first n_bits tiles take their masks from `bits` (this lane's
    // entry of each, in LDS); later ones read the mask bytes again.
    Mask<VEC> next;
    if (tile < a.tiles && n_bits == 0) next.load(a.mask, tile * kTileV + lane_off, slots);
    for (uint32_t j = 0; tile < a.tiles; tile += G, ++j) {
        const uint32_t s = tile * kTileV + lane_off;
        uint32_t row_base = 0;
        if constexpr (MODE == kModeGRPO) {
            const uint32_t s0 = tile * kTileV;
            grpo_row_scales(a, s0, s0 + kTileV < slots ? s0 + kTileV : slots, row_lds, row_base);
        }
        Lane<T, VEC> L;
        if (j < n_bits) L.m.from_bits(bits[j * kThreads + threadIdx.x]);
        else L.m = next;
        if (tile + G < a.tiles && j + 1 >= n_bits) next.load(a.mask, (tile + G) * kTileV + lane_off, slots);
        load_planes<T, MODE, HAS_KL, VEC>(a, s, L);
        n_lane += L.m.count();
        float g[VEC];
        part += lane_terms<T, MODE, HAS_KL, VEC>(a, s, L, reinterpret_cast<const float*>(row_lds),
                                                 row_base, scale, g);
        if constexpr (WRITE_GRAD) store_grad<T, VEC, false>(a, s, L.m, g, 1.0f);
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
template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD, int VEC, bool ONE_TILE>
__global__ void __launch_bounds__(kThreads) loss_kernel(const Args a) {
    constexpr uint32_t kTileV = kThreads * VEC;
    __shared__ float red_f[kWaves];
    __shared__ uint32_t red_u[kWaves];
    __shared__ uint32_t word[2];
    __shared__ uint32_t list[kThreads + 1];
    // GRPO: per-row counts, then per-row scales, of the rows a tile touches.
    constexpr int kRowLds = (MODE == kModeGRPO) ? int(kTileV) + 2 : 1;
    __shared__ uint32_t row_lds[kRowLds];
    // Striding fwd+bwd BNPO / reverse-KL: the counting pass keeps each lane's
    // mask bits of the worker's first kBitTiles tiles, so that the streaming
    // pass does not read those mask bytes again.
    constexpr bool kKeepBits = !ONE_TILE && MODE != kModeGRPO && WRITE_GRAD;
    constexpr int kBitTiles = kKeepBits ? (MODE == kModeRKL ? kBitTilesRkl : kBitTilesPolicy) : 1;
    __shared__ uint16_t mask_bits[kBitTiles * kThreads];

    constexpr bool kGlobalN = MODE != kModeGRPO;
    constexpr bool kExchange = kGlobalN && WRITE_GRAD;
    const Workspace* ws = a.ws;
    const __amdgpu_buffer_rsrc_t view = entry_view(ws);
    const Tag tg = launch_tag();
    const Limits lim = read_limits(ws);
    const uint32_t slots = uint32_t(a.slots);
    const uint32_t W = ONE_TILE ? gridDim.x - 1 : gridDim.x;   // workers
    const uint32_t lane_off = threadIdx.x * VEC;

    // Worker w's valid count and partial loss, computed by the calling workgroup
    // (uniform), exactly as worker w forms its own.
    auto count_of = [&](uint32_t w) -> uint32_t {
        uint32_t n = 0;
        for (uint32_t tile = w; tile < a.tiles; tile += ONE_TILE ? a.tiles : W) {
            Mask<VEC> m;
            m.load(a.mask, tile * kTileV + lane_off, slots);
            n += m.count();
        }
        return block_sum(n, red_u);
    };
    auto partial_of = [&](uint32_t w) -> float {
        float part = 0.0f;
        if constexpr (ONE_TILE) {
            const uint32_t s = w * kTileV + lane_off;
            uint32_t row_base = 0;
            if constexpr (MODE == kModeGRPO) {
                const uint32_t s0 = w * kTileV;
                grpo_row_scales(a, s0, s0 + kTileV < slots ? s0 + kTileV : slots, row_lds, row_base);
            }
            Lane<T, VEC> L;
            (void)load_lane_count<T, MODE, HAS_KL, VEC, false>(a, s, L);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC>(a, s, L, reinterpret_cast<const float*>(row_lds), row_base,
                                                    1.0f, g);
        } else {
            uint32_t n_unused = 0;
            stream_tiles<T, MODE, HAS_KL, false, VEC>(a, w, W, row_lds, part, n_unused, 1.0f);
        }
        return block_sum(part, red_f);
    };
    auto nothing = [] {};
    auto gather_counts = [&]() -> uint32_t {
        return gather<uint32_t>(view, cnt_off(0), W, tg, lim.steal, list, red_u, count_of, nothing);
    };
    // The partials' first reads go out before the release (when there is one) is stored.
    auto gather_partials = [&](auto&& between) -> float {
        return gather<float>(view, par_off(0), W, tg, lim.steal, list, red_f, partial_of, between);
    };

    float part = 0.0f;
    uint32_t n_lane = 0;

    if constexpr (ONE_TILE) {
        // Workgroup 0 coordinates only; workgroup w > 0 is worker w - 1 and owns tile w - 1.
        if (blockIdx.x == 0) {
            uint32_t N = 0;
            if constexpr (kGlobalN) N = gather_counts();
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
            const uint32_t n_wg = block_sum(load_lane_count<T, MODE, HAS_KL, VEC, false>(a, s, L), red_u);
            if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC>(a, s, L, nullptr, 0, 1.0f, g);
            const float part_wg = block_sum(part, red_f);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
            const uint32_t N = await_release(view, lim.release, tg, word, gather_counts);
            store_grad<T, VEC, true>(a, s, L.m, g, inv_count<MODE>(N));
        } else {
            // Forward-only (any mode) and GRPO fwd+bwd.  GRPO first scans the masks of
            // the rows the tile touches (measured faster than overlapping the scan with
            // the tile's plane loads, whose completion the scan's loads would wait for).
            uint32_t row_base = 0;
            if constexpr (MODE == kModeGRPO) {
                const uint32_t s0 = worker * kTileV;
                grpo_row_scales(a, s0, s0 + kTileV < slots ? s0 + kTileV : slots, row_lds, row_base);
            }
            n_lane = load_lane_count<T, MODE, HAS_KL, VEC, VEC == kVecSmall>(a, s, L);
            float g[VEC];
            part = lane_terms<T, MODE, HAS_KL, VEC>(a, s, L, reinterpret_cast<const float*>(row_lds),
                                                    row_base, 1.0f, g);
            if constexpr (WRITE_GRAD) store_grad<T, VEC, false>(a, s, L.m, g, 1.0f);
            const float part_wg = block_sum(part, red_f);
            uint32_t n_wg = 0;
            if constexpr (kGlobalN) n_wg = block_sum(n_lane, red_u);
            if constexpr (kGlobalN) {
                if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            }
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
        }
    } else {
        // Every workgroup is a worker striding over the tiles; workgroup 0 also
        // coordinates (a dedicated coordinator would take one of the co-resident
        // slots, and with it a whole extra tile from some worker's share).
        const uint32_t worker = blockIdx.x;
        uint32_t N = 0;
        if constexpr (kExchange) {
            // Count every owned mask (eight loads in flight per lane) and keep the
            // bits of the first kBitTiles tiles, exchange, then stream.
            uint32_t tile = worker, j = 0;
            for (; tile + 7 * W < a.tiles; tile += 8 * W, j += 8) {
                Mask<VEC> m[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) m[u].load(a.mask, (tile + u * W) * kTileV + lane_off, slots);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t b = m[u].bits();
                    n_lane += __builtin_popcount(b);
                    if (j + u < uint32_t(kBitTiles)) mask_bits[(j + u) * kThreads + threadIdx.x] = uint16_t(b);
                }
            }
            for (; tile < a.tiles; tile += W, ++j) {
                Mask<VEC> m;
                m.load(a.mask, tile * kTileV + lane_off, slots);
                const uint32_t b = m.bits();
                n_lane += __builtin_popcount(b);
                if (j < uint32_t(kBitTiles)) mask_bits[j * kThreads + threadIdx.x] = uint16_t(b);
            }
            const uint32_t n_bits = j < uint32_t(kBitTiles) ? j : uint32_t(kBitTiles);
            const uint32_t n_wg = block_sum(n_lane, red_u);
            if (blockIdx.x == 0) {
                // The coordinator's own count goes out once its reads of the others' are issued.
                N = gather<uint32_t>(view, cnt_off(0), W, tg, lim.steal, list, red_u, count_of, [&] {
                    if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
                });
                if (threadIdx.x == kCountThread) publish(view, kReleaseOff, tg, N);
            } else {
                if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
                N = await_release(view, lim.release, tg, word, gather_counts);
            }
            uint32_t unused_n = 0;
            stream_tiles<T, MODE, HAS_KL, true, VEC>(a, worker, W, row_lds, part, unused_n, inv_count<MODE>(N),
                                                     mask_bits, n_bits);
            const float part_wg = block_sum(part, red_f);
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
        } else {
            // Forward-only (any mode) and GRPO fwd+bwd: one streaming pass, no exchange.
            stream_tiles<T, MODE, HAS_KL, WRITE_GRAD, VEC>(a, worker, W, row_lds, part, n_lane, 1.0f);
            const float part_wg = block_sum(part, red_f);
            uint32_t n_wg = 0;
            if constexpr (kGlobalN) n_wg = block_sum(n_lane, red_u);
            if constexpr (kGlobalN) {
                if (threadIdx.x == kCountThread) publish(view, cnt_off(worker), tg, n_wg);
            }
            if (threadIdx.x == kPartialThread) publish(view, par_off(worker), tg, __float_as_uint(part_wg));
            if (kGlobalN && blockIdx.x == 0) N = gather_counts();
        }
        if (blockIdx.x == 0) {
            const float total = gather_partials(nothing);
            if (threadIdx.x == 0) write_results<MODE>(a, total, N);
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
    }
    return nullptr;
}

template <typename T>
static const void* pick_typed(int mode, bool has_kl, bool write_grad, int shape) {
    switch (mode) {
    case kModeBNPO:
        if (has_kl) return write_grad ? kernel_ptr<T, kModeBNPO, true, true>(shape) : kernel_ptr<T, kModeBNPO, true, false>(shape);
        return write_grad ? kernel_ptr<T, kModeBNPO, false, true>(shape) : kernel_ptr<T, kModeBNPO, false, false>(shape);
    case kModeGRPO:
        if (has_kl) return write_grad ? kernel_ptr<T, kModeGRPO, true, true>(shape) : kernel_ptr<T, kModeGRPO, true, false>(shape);
        return write_grad ? kernel_ptr<T, kModeGRPO, false, true>(shape) : kernel_ptr<T, kModeGRPO, false, false>(shape);
    case kModeRKL:
        return write_grad ? kernel_ptr<T, kModeRKL, true, true>(shape) : kernel_ptr<T, kModeRKL, true, false>(shape);
    }
    return nullptr;
}

const void* pick_kernel(int dtype, int mode, bool has_kl, bool write_grad, int shape) {
    switch (dtype) {
    case kF32: return pick_typed<float>(mode, has_kl, write_grad, shape);
    case kF16: return pick_typed<_Float16>(mode, has_kl, write_grad, shape);
    case kBF16: return pick_typed<__bf16>(mode, has_kl, write_grad, shape);
    }
    return nullptr;
}

// ----------------------------------------------------------------------------- the library's own scratch

// The workspace of the entry point that allocates nothing: the header and the
// entry arrays of a Workspace (what the per-token kernels address), one copy
// per device, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// scratch_address(), per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(void** out) {
    return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)) == hipSuccess ? 0 : -1;
}

// Zero-fills n 16-byte words (the scratch's first use on a device).
__global__ void __launch_bounds__(kThreads) clear_kernel(uint4* p, uint32_t n) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}
const void* clear_kernel_ptr() { return reinterpret_cast<const void*>(&clear_kernel); }

}  // namespace rlpl
