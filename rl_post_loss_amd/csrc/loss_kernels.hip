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
//    is kThreads lanes x kVec consecutive slots; each lane moves its 16 mask
//    bytes with one 128-bit load and its 16 log-probs per plane with two
//    (16-bit dtypes) or four (fp32) 128-bit loads.  When streaming several
//    tiles per workgroup, plane loads are skipped for lanes whose 16 mask
//    bytes are all zero.
//  * A persistent grid of G <= (co-resident workgroups) takes tiles
//    wg, wg+G, wg+2G, ...  Per-token math is fp32 in registers.
//  * Reductions: per-lane sums -> wavefront shuffle tree -> LDS across the
//    4 waves -> one partial per workgroup in the workspace.  The last
//    workgroup to finish (ticket from an agent-scope atomic) sums the G
//    partials in workgroup order, so the loss is deterministic and identical
//    between the fwd+bwd and forward-only kernels.
//  * BNPO / RKL fwd+bwd need the global valid count N before any gradient is
//    scaled: each workgroup adds (1<<32 | its count) to one 64-bit word; the
//    last arrival publishes N (with a generation number) in another word the
//    others poll.  All cross-workgroup traffic is agent-scope relaxed atomics
//    and device-coherent loads/stores, never an L2-wide writeback/invalidate.
//    The grid never exceeds the co-resident capacity; the wait is bounded in
//    time anyway and sets a sticky flag if it ever gives up.  When a
//    workgroup owns a single tile, its plane loads are issued with its mask
//    load, stay in flight while it waits, and the tile never leaves
//    registers; with more tiles it counts its masks first and streams after.
//  * GRPO needs only each row's own count: a workgroup counts the mask of
//    every row its tile touches into LDS (no cross-workgroup exchange before
//    the gradient is scaled), as the card's one-block-per-row design does.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loss_kernels.h"

namespace rlpl {

// ----------------------------------------------------------------------------- element types

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float to_f32(uint32_t bits) { return __uint_as_float(bits); }
    static __device__ __forceinline__ uint32_t from_f32(float v) { return __float_as_uint(v); }
};
template <> struct Elem<_Float16> {
    static __device__ __forceinline__ float to_f32(uint32_t bits) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    }
    static __device__ __forceinline__ uint32_t from_f32(float v) {   // round to nearest even
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
    }
};
template <> struct Elem<__bf16> {
    static __device__ __forceinline__ float to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }
    static __device__ __forceinline__ uint32_t from_f32(float v) {   // round to nearest even
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
    }
};

// 16 consecutive elements of one plane held in registers as raw 128-bit words.
template <typename T>
struct Vec16 {
    static constexpr int kWords = kVec * (int)sizeof(T) / 4;
    static constexpr int kQuads = kWords / 4;
    uint32_t w[kWords];

    __device__ __forceinline__ void load(const T* __restrict__ base, int64_t s, int64_t slots) {
        if (s + kVec <= slots) {
            const uint4* p = reinterpret_cast<const uint4*>(base + s);
#pragma unroll
            for (int q = 0; q < kQuads; ++q) {
                uint4 v = p[q];
                w[4 * q + 0] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            }
        } else {
            const uint16_t* p16 = reinterpret_cast<const uint16_t*>(base);
            const uint32_t* p32 = reinterpret_cast<const uint32_t*>(base);
#pragma unroll
            for (int i = 0; i < kWords; ++i) w[i] = 0;
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (s + k < slots) {
                    if constexpr (sizeof(T) == 4) w[k] = p32[s + k];
                    else w[k >> 1] |= (uint32_t)p16[s + k] << (16 * (k & 1));
                }
            }
        }
    }
    __device__ __forceinline__ float get(int k) const {
        if constexpr (sizeof(T) == 4) return Elem<T>::to_f32(w[k]);
        else return Elem<T>::to_f32((w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
    }
    __device__ __forceinline__ void set(int k, float v) {
        if constexpr (sizeof(T) == 4) w[k] = Elem<T>::from_f32(v);
        else if ((k & 1) == 0) w[k >> 1] = Elem<T>::from_f32(v);
        else w[k >> 1] |= Elem<T>::from_f32(v) << 16;
    }
    __device__ __forceinline__ void store(T* __restrict__ base, int64_t s, int64_t slots) const {
        if (s + kVec <= slots) {
            uint4* p = reinterpret_cast<uint4*>(base + s);
#pragma unroll
            for (int q = 0; q < kQuads; ++q)
                p[q] = make_uint4(w[4 * q + 0], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        } else {
            uint16_t* p16 = reinterpret_cast<uint16_t*>(base);
            uint32_t* p32 = reinterpret_cast<uint32_t*>(base);
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                if (s + k < slots) {
                    if constexpr (sizeof(T) == 4) p32[s + k] = w[k];
                    else p16[s + k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
                }
            }
        }
    }
};

// 16 mask bytes of one lane.
struct Mask16 {
    uint32_t w[4];
    __device__ __forceinline__ void load(const uint8_t* __restrict__ mask, int64_t s, int64_t slots) {
        if (s + kVec <= slots) {
            uint4 v = *reinterpret_cast<const uint4*>(mask + s);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            w[0] = w[1] = w[2] = w[3] = 0;
#pragma unroll
            for (int k = 0; k < kVec; ++k)
                if (s + k < slots) w[k >> 2] |= (uint32_t)mask[s + k] << (8 * (k & 3));
        }
    }
    __device__ __forceinline__ bool any() const { return (w[0] | w[1] | w[2] | w[3]) != 0; }
    __device__ __forceinline__ bool valid(int k) const { return ((w[k >> 2] >> (8 * (k & 3))) & 0xFFu) != 0; }
    // Number of nonzero bytes: for each byte, (b & 0x7F) + 0x7F sets bit 7 iff the low 7 bits
    // are nonzero; OR-ing b itself covers bit 7.
    __device__ __forceinline__ uint32_t count() const {
        uint32_t n = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t x = ((w[i] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w[i];
            n += __builtin_popcount(x & 0x80808080u);
        }
        return n;
    }
};

// ----------------------------------------------------------------------------- per-token math

// exp on the hardware base-2 exponential unit.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Per-token contribution c = per_token + beta*kl and its derivative g in lp.
template <int MODE, bool HAS_KL>
__device__ __forceinline__ void token_terms(float lp, float old, float ref, float A,
                                            float beta, float lo, float hi, float& c, float& g) {
    if constexpr (MODE == kModeRKL) {
        const float x = ref - lp;                 // teacher - student
        const float em1 = fast_exp(x) - 1.0f;
        c = em1 - x;                              // exp(x) - x - 1
        g = -em1;                                 // d/dstudent = 1 - exp(x)
    } else {
        const float ratio = fast_exp(lp - old);
        const float clipped = fminf(fmaxf(ratio, lo), hi);
        const float chosen = fminf(ratio, clipped);
        c = -A * chosen;
        g = (ratio <= clipped) ? -A * ratio : 0.0f;   // ties take the unclipped branch
        if constexpr (HAS_KL) {
            const float x = ref - lp;
            const float em1 = fast_exp(x) - 1.0f;
            c += beta * (em1 - x);
            g -= beta * em1;
        }
    }
}

// ----------------------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Workgroup sum in a fixed order (lane tree, then waves 0..3); result valid in every thread.
template <typename V>
__device__ __forceinline__ V block_sum(V v, V* red) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();                       // red[] may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    V t = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) t += red[i];
    return t;
}

// ----------------------------------------------------------------------------- workspace protocol
//
// Everything one workgroup tells another travels inside an agent-scope atomic
// word (or a device-coherent store followed by a wait for its completion), so
// no L2-wide writeback or invalidate (what an agent-scope release/acquire
// costs on this chip, per workgroup and per poll) is ever issued.

__device__ __forceinline__ uint64_t atomic_add_relaxed(uint64_t* p, uint64_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_relaxed(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void store_relaxed(V* p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Makes `v` depend on `dep` as far as the compiler knows (no instruction is
// emitted): an atomic whose operand is laundered this way is issued only after
// `dep` has been loaded.
__device__ __forceinline__ uint64_t after(uint64_t v, uint32_t dep) {
    asm volatile("" : "+v"(v) : "v"(dep));
    return v;
}

// Tags published by the launch of generation `gen`.  A zero-filled workspace
// holds tag 0 everywhere, which is the tag of no launch's first use; a slot
// left from an older launch carries an older tag.
__device__ __forceinline__ uint32_t tag_of(uint32_t gen) { return gen + 1u; }

// Polls a tagged partial until it carries `tag` (bounded like every wait).
__device__ uint64_t wait_tagged(Workspace* ws, const uint64_t* slot, uint32_t tag) {
    uint64_t v = load_relaxed(slot);
    if (uint32_t(v >> 32) == tag) return v;
    const uint64_t t0 = wall_clock64();
    uint32_t polls = 0;
    while (uint32_t((v = load_relaxed(slot)) >> 32) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWaitLimitTicks || ++polls > kWaitLimitPolls) {
            __hip_atomic_fetch_or(&ws->flags, kFlagWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    return v;
}

// This workgroup's partial loss, tagged for the launch (one 64-bit
// device-coherent store: a reader sees either the old or the new pair).
__device__ __forceinline__ void publish_partial(Workspace* ws, uint32_t gen, float part) {
    store_relaxed(&ws->partial[blockIdx.x], (uint64_t(tag_of(gen)) << 32) | __float_as_uint(part));
}

// Sum of the G partials of this launch in workgroup order (each thread a strided
// run, then the fixed tree); waits for any partial still in flight.
__device__ float sum_partials(Workspace* ws, uint32_t gen, float* red) {
    float s = 0.0f;
    for (uint32_t i = threadIdx.x; i < gridDim.x; i += kThreads)
        s += __uint_as_float(uint32_t(wait_tagged(ws, &ws->partial[i], tag_of(gen))));
    return block_sum(s, red);
}

// Thread 0 of the launch's final ticket holder: every workgroup has read the
// generation by now, so the next launch may use the next one.
__device__ __forceinline__ void advance_generation(Workspace* ws, uint32_t gen) {
    store_relaxed(&ws->generation, gen + 1u);
}

// Device-wide count exchange (thread 0 works, the workgroup waits at the
// barrier with its outstanding loads in flight).  Every workgroup adds
// (1<<32 | its count) to ws->arrive; the last arrival publishes
// ws->release = [tag | N] and re-arms arrive; the others poll release until
// it carries this launch's tag.  Returns N in every thread and sets
// *is_last in every thread of the last arrival.  With `finalises`, the
// workgroup's partial is published first and the last arrival ends the launch
// (advances the generation).  `gen` is thread 0's copy of the launch
// generation; on return every thread holds it.
__device__ uint32_t grid_count_exchange(Workspace* ws, uint32_t& gen, uint32_t n_wg, bool finalises,
                                        float part, uint32_t* lds, bool* is_last) {
    if (threadIdx.x == 0) {
        lds[2] = gen;
        const uint32_t G = gridDim.x;
        if (finalises) publish_partial(ws, gen, part);
        const uint64_t prev = atomic_add_relaxed(&ws->arrive, after((uint64_t(1) << 32) | n_wg, gen));
        uint32_t total;
        lds[1] = 0;
        if (uint32_t(prev >> 32) == G - 1) {
            total = uint32_t(prev) + n_wg;
            store_relaxed(&ws->release, (uint64_t(tag_of(gen)) << 32) | total);
            store_relaxed(&ws->arrive, uint64_t(0));
            if (finalises) advance_generation(ws, gen);
            lds[1] = 1;
        } else {
            // Bounded wait: the grid never exceeds the co-resident capacity, so every
            // workgroup arrives within microseconds; give up after ~1 s of the 100 MHz
            // clock (or, should that clock not advance, after kWaitLimitPolls polls).
            const uint64_t t0 = wall_clock64();
            uint32_t polls = 0;
            uint64_t rel;
            while (uint32_t((rel = load_relaxed(&ws->release)) >> 32) != tag_of(gen)) {
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > kWaitLimitTicks || ++polls > kWaitLimitPolls) {
                    __hip_atomic_fetch_or(&ws->flags, kFlagWaitTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            total = uint32_t(rel);
        }
        lds[0] = total;
    }
    __syncthreads();
    *is_last = lds[1] != 0;
    gen = lds[2];
    return lds[0];
}

// Publish this workgroup's partial and take a finish ticket on ws->depart
// ([63:32 done | 31:0 count]).  Returns true in every thread of the last
// workgroup, which re-arms depart, advances the generation and owns the
// finalise; lds[0] then holds the sum of the counts passed by all workgroups.
// `gen` as for grid_count_exchange.
__device__ bool finish_ticket(Workspace* ws, uint32_t& gen, float part, uint32_t n_wg, uint32_t* lds) {
    if (threadIdx.x == 0) {
        lds[2] = gen;
        publish_partial(ws, gen, part);
        const uint64_t prev = atomic_add_relaxed(&ws->depart, after((uint64_t(1) << 32) | n_wg, gen));
        const bool last = uint32_t(prev >> 32) == gridDim.x - 1;
        if (last) {
            lds[0] = uint32_t(prev) + n_wg;
            store_relaxed(&ws->depart, uint64_t(0));
            advance_generation(ws, gen);
        }
        lds[1] = last;
    }
    __syncthreads();
    gen = lds[2];
    return lds[1] != 0;
}

// ----------------------------------------------------------------------------- row cursor

template <typename T>
__device__ __forceinline__ float load_adv(const T* adv, int32_t r) {
    if constexpr (sizeof(T) == 4) return reinterpret_cast<const float*>(adv)[r];
    else return Elem<T>::to_f32(reinterpret_cast<const uint16_t*>(adv)[r]);
}

// ----------------------------------------------------------------------------- one tile of one lane

// Computes c and g for the lane's 16 slots starting at s; returns the lane's
// partial sum of c over valid slots.  g[k] is left at 0 for masked slots.
template <typename T, int MODE, bool HAS_KL>
__device__ __forceinline__ float lane_terms(const Args& a, int64_t s, const Mask16& m,
                                            const Vec16<T>& lp, const Vec16<T>& old,
                                            const Vec16<T>& ref, const float* row_scale_lds,
                                            int32_t row_base, float g[kVec]) {
    float part = 0.0f;
    if (!m.any()) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) g[k] = 0.0f;
        return part;
    }
    const T* adv = static_cast<const T*>(a.adv);
    // s < slots < 2^31 here (a lane past the end has an all-zero mask).
    int32_t r = int32_t(uint32_t(s) / uint32_t(a.seq_len));
    int32_t t = int32_t(s) - r * a.seq_len;
    float A = 0.0f, scale = 1.0f;
    if constexpr (MODE != kModeRKL) A = load_adv<T>(adv, r);
    if constexpr (MODE == kModeGRPO) scale = row_scale_lds[r - row_base];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
        float c = 0.0f, gk = 0.0f;
        if (m.valid(k)) {
            token_terms<MODE, HAS_KL>(lp.get(k), MODE == kModeRKL ? 0.0f : old.get(k),
                                      HAS_KL ? ref.get(k) : 0.0f, A, a.beta, a.lo, a.hi, c, gk);
            if constexpr (MODE == kModeGRPO) { c *= scale; gk *= scale; }
            part += c;
        }
        g[k] = gk;
        if (k + 1 < kVec && ++t == a.seq_len) {
            t = 0;
            ++r;
            if (r < a.bs) {
                if constexpr (MODE != kModeRKL) A = load_adv<T>(adv, r);
                if constexpr (MODE == kModeGRPO) scale = row_scale_lds[r - row_base];
            }
        }
    }
    return part;
}

template <typename T, bool HAS_KL, int MODE>
__device__ __forceinline__ void load_planes(const Args& a, int64_t s, Vec16<T>& lp, Vec16<T>& old,
                                            Vec16<T>& ref) {
    lp.load(static_cast<const T*>(a.lp), s, a.slots);
    if constexpr (MODE != kModeRKL) old.load(static_cast<const T*>(a.old), s, a.slots);
    if constexpr (HAS_KL) ref.load(static_cast<const T*>(a.ref), s, a.slots);
}

template <typename T>
__device__ __forceinline__ void store_grad(const Args& a, int64_t s, const Mask16& m,
                                           const float g[kVec], float scale) {
    Vec16<T> out;
#pragma unroll
    for (int k = 0; k < kVec; ++k) out.set(k, m.valid(k) ? g[k] * scale : 0.0f);
    out.store(static_cast<T*>(a.grad), s, a.slots);
}

// ----------------------------------------------------------------------------- GRPO row counts

// For the tile [s0, s1): counts the mask of every row the tile touches into
// cnt[row - r_first] (LDS), then turns each count into the row's gradient
// scale 1 / (max(n_r, 1) * bs).  Writes n_out for rows that start in the tile.
__device__ void grpo_row_scales(const Args& a, int64_t s0, int64_t s1, uint32_t* cnt,
                                int32_t& r_first) {
    const int64_t T = a.seq_len;
    r_first = int32_t(uint32_t(s0) / uint32_t(T));
    const int32_t r_last = int32_t(uint32_t(s1 - 1) / uint32_t(T));
    const int32_t nrows = r_last - r_first + 1;
    const int64_t e0 = int64_t(r_first) * T, e1 = int64_t(r_last + 1) * T;
    for (int i = threadIdx.x; i < nrows; i += kThreads) cnt[i] = 0;
    __syncthreads();
    for (int64_t c = (e0 & ~int64_t(kVec - 1)) + int64_t(threadIdx.x) * kVec; c < e1;
         c += int64_t(kThreads) * kVec) {
        Mask16 m;
        m.load(a.mask, c, a.slots);
        if (!m.any()) continue;
        int32_t r = int32_t(uint32_t(c) / uint32_t(T));
        int64_t row_end = int64_t(r + 1) * T;
        uint32_t run = 0;
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
            const int64_t i = c + k;
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
    // Each thread turns its own entries from counts into scales in place.
    for (int i = threadIdx.x; i < nrows; i += kThreads) {
        const uint32_t n = cnt[i];
        const float scale = 1.0f / (float(n > 0 ? n : 1u) * float(a.bs));
        cnt[i] = __float_as_uint(scale);
        const int32_t r = r_first + i;
        if (a.n_out && int64_t(r) * T >= s0 && int64_t(r) * T < s1) a.n_out[r] = n;
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------- the kernel

// Loads one lane's mask and planes.  SPECULATIVE issues the plane loads
// together with the mask load (one memory round trip; used when each
// workgroup owns one tile and the call is latency-bound); otherwise the plane
// loads wait for the mask and are skipped when all 16 bytes are zero (no plane
// bytes move for masked slots; used when streaming many tiles).
template <typename T, int MODE, bool HAS_KL, bool SPECULATIVE>
__device__ __forceinline__ void load_lane(const Args& a, int64_t s, Mask16& m, Vec16<T>& lp,
                                          Vec16<T>& old, Vec16<T>& ref) {
    m.load(a.mask, s, a.slots);
    if (SPECULATIVE || m.any()) load_planes<T, HAS_KL, MODE>(a, s, lp, old, ref);
}

template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD, bool SPECULATIVE>
__device__ __forceinline__ void stream_tiles(const Args& a, uint32_t* row_lds, float& part,
                                             uint32_t& n_lane, float scale) {
    const int64_t G = gridDim.x;
    const int64_t lane_off = int64_t(threadIdx.x) * kVec;
    for (int64_t tile = blockIdx.x; tile < a.tiles; tile += G) {
        const int64_t s = tile * kTile + lane_off;
        int32_t row_base = 0;
        if constexpr (MODE == kModeGRPO) {
            const int64_t s0 = tile * kTile;
            const int64_t s1 = s0 + kTile < a.slots ? s0 + kTile : a.slots;
            grpo_row_scales(a, s0, s1, row_lds, row_base);
        }
        Mask16 m;
        Vec16<T> lp, old, ref;
        load_lane<T, MODE, HAS_KL, SPECULATIVE>(a, s, m, lp, old, ref);
        n_lane += m.count();
        float g[kVec];
        part += lane_terms<T, MODE, HAS_KL>(a, s, m, lp, old, ref,
                                            reinterpret_cast<const float*>(row_lds), row_base, g);
        if constexpr (WRITE_GRAD) store_grad<T>(a, s, m, g, scale);
    }
}

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

template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD>
__global__ void __launch_bounds__(kThreads) loss_kernel(const Args a) {
    __shared__ float red_f[kWaves];
    __shared__ uint32_t red_u[kWaves];
    __shared__ uint32_t word[3];
    // GRPO: per-row counts, then per-row scales, of the rows a tile touches.
    constexpr int kRowLds = (MODE == kModeGRPO) ? kTile + 2 : 1;
    __shared__ uint32_t row_lds[kRowLds];

    Workspace* ws = a.ws;
    // The launch generation tags this launch's partials and count release; thread 0
    // reads it first so that the read is in flight together with the data loads.
    uint32_t gen = 0;
    if (threadIdx.x == 0) gen = load_relaxed(&ws->generation);

    const int64_t G = gridDim.x;
    const bool one_tile = a.tiles <= G;     // uniform: each workgroup owns at most one tile
    constexpr bool kGlobalN = MODE != kModeGRPO;
    constexpr bool kExchange = kGlobalN && WRITE_GRAD;

    float part = 0.0f;
    uint32_t n_lane = 0;

    if constexpr (kExchange) {
        if (one_tile) {
            // The tile stays in registers across the count exchange.  The partial loss is
            // published with the arrival, so the last arrival also finalises the loss and
            // no workgroup waits for anything after the exchange.
            const int64_t s = int64_t(blockIdx.x) * kTile + int64_t(threadIdx.x) * kVec;
            Mask16 m;
            Vec16<T> lp, old, ref;
            load_lane<T, MODE, HAS_KL, true>(a, s, m, lp, old, ref);
            float g[kVec];
            part = lane_terms<T, MODE, HAS_KL>(a, s, m, lp, old, ref, nullptr, 0, g);
            const uint32_t n_wg = block_sum(m.count(), red_u);
            const float part_wg = block_sum(part, red_f);
            bool last;
            const uint32_t N = grid_count_exchange(ws, gen, n_wg, true, part_wg, word, &last);
            store_grad<T>(a, s, m, g, inv_count<MODE>(N));
            if (last) {
                const float total = sum_partials(ws, gen, red_f);
                if (threadIdx.x == 0) {
                    *a.loss = final_loss<MODE>(total, N);
                    if (a.n_out) a.n_out[0] = N;
                }
            }
        } else {
            // Several tiles per workgroup: count every owned mask, exchange, then stream.
            const int64_t lane_off = int64_t(threadIdx.x) * kVec;
            for (int64_t tile = blockIdx.x; tile < a.tiles; tile += G) {
                Mask16 m;
                m.load(a.mask, tile * kTile + lane_off, a.slots);
                n_lane += m.count();
            }
            bool unused_last;
            const uint32_t N = grid_count_exchange(ws, gen, block_sum(n_lane, red_u), false, 0.0f,
                                                   word, &unused_last);
            uint32_t unused_n = 0;
            stream_tiles<T, MODE, HAS_KL, true, false>(a, row_lds, part, unused_n, inv_count<MODE>(N));
            if (finish_ticket(ws, gen, block_sum(part, red_f), 0u, word)) {
                const float total = sum_partials(ws, gen, red_f);
                if (threadIdx.x == 0) {
                    *a.loss = final_loss<MODE>(total, N);
                    if (a.n_out) a.n_out[0] = N;
                }
            }
        }
    } else {
        // Forward-only (any mode) and GRPO fwd+bwd: one streaming pass, no exchange.
        if (one_tile) stream_tiles<T, MODE, HAS_KL, WRITE_GRAD, true>(a, row_lds, part, n_lane, 1.0f);
        else stream_tiles<T, MODE, HAS_KL, WRITE_GRAD, false>(a, row_lds, part, n_lane, 1.0f);
        uint32_t n_wg = 0;
        if constexpr (kGlobalN) n_wg = block_sum(n_lane, red_u);
        if (finish_ticket(ws, gen, block_sum(part, red_f), n_wg, word)) {
            const uint32_t N = word[0];
            const float total = sum_partials(ws, gen, red_f);
            if (threadIdx.x == 0) {
                if constexpr (MODE == kModeGRPO) {
                    *a.loss = total;
                } else {
                    *a.loss = final_loss<MODE>(total, N);
                    if (a.n_out) a.n_out[0] = N;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------- host-side table

template <typename T, int MODE, bool HAS_KL, bool WRITE_GRAD>
static const void* kernel_ptr() {
    return reinterpret_cast<const void*>(&loss_kernel<T, MODE, HAS_KL, WRITE_GRAD>);
}

template <typename T>
static const void* pick_typed(int mode, bool has_kl, bool write_grad) {
    switch (mode) {
    case kModeBNPO:
        if (has_kl) return write_grad ? kernel_ptr<T, kModeBNPO, true, true>() : kernel_ptr<T, kModeBNPO, true, false>();
        return write_grad ? kernel_ptr<T, kModeBNPO, false, true>() : kernel_ptr<T, kModeBNPO, false, false>();
    case kModeGRPO:
        if (has_kl) return write_grad ? kernel_ptr<T, kModeGRPO, true, true>() : kernel_ptr<T, kModeGRPO, true, false>();
        return write_grad ? kernel_ptr<T, kModeGRPO, false, true>() : kernel_ptr<T, kModeGRPO, false, false>();
    case kModeRKL:
        return write_grad ? kernel_ptr<T, kModeRKL, true, true>() : kernel_ptr<T, kModeRKL, true, false>();
    }
    return nullptr;
}

const void* pick_kernel(int dtype, int mode, bool has_kl, bool write_grad) {
    switch (dtype) {
    case kF32: return pick_typed<float>(mode, has_kl, write_grad);
    case kF16: return pick_typed<_Float16>(mode, has_kl, write_grad);
    case kBF16: return pick_typed<__bf16>(mode, has_kl, write_grad);
    }
    return nullptr;
}

}  // namespace rlpl
