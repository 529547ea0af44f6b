// Device-side pieces shared by the kernel files: element conversion, lane
// loads and stores, workgroup reductions and the cross-workgroup protocol on
// the caller's workspace.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "loss_kernels.h"

namespace rlpl {

// ----------------------------------------------------------------------------- element types

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float get(const uint32_t* w, int k) { return __uint_as_float(w[k]); }
};
template <> struct Elem<_Float16> {
    static __device__ __forceinline__ float get(const uint32_t* w, int k) {
        return (float)__builtin_bit_cast(_Float16, uint16_t(w[k >> 1] >> (16 * (k & 1))));
    }
    // two floats -> two fp16 (round to nearest even, subnormals kept) in one dword
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
};
template <> struct Elem<__bf16> {
    static __device__ __forceinline__ float get(const uint32_t* w, int k) {
        return __uint_as_float((k & 1) ? (w[k >> 1] & 0xFFFF0000u) : (w[k >> 1] << 16));
    }
    // two floats -> two bf16 (round to nearest even) in one dword
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
};

// ----------------------------------------------------------------------------- lane registers

// N dwords moved with the widest aligned accesses (N * 4 bytes aligned to min(N * 4, 16)).
template <int N>
struct Dwords {
    uint32_t w[N];
    __device__ __forceinline__ void load(const void* p) {
        if constexpr (N == 1) {
            w[0] = *static_cast<const uint32_t*>(p);
        } else if constexpr (N == 2) {
            const uint2 v = *static_cast<const uint2*>(p);
            w[0] = v.x; w[1] = v.y;
        } else {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const uint4 v = static_cast<const uint4*>(p)[q];
                w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            }
        }
    }
    __device__ __forceinline__ void store(void* p) const {
        if constexpr (N == 1) {
            *static_cast<uint32_t*>(p) = w[0];
        } else if constexpr (N == 2) {
            *static_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else {
#pragma unroll
            for (int q = 0; q < N / 4; ++q)
                static_cast<uint4*>(p)[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
    }
};

// VEC consecutive elements of one plane.  A lane that runs past `slots` (only
// in the last tile) moves its in-range elements one by one and zero-fills.
template <typename T, int VEC>
struct Plane {
    static constexpr int kWords = VEC * int(sizeof(T)) / 4;
    Dwords<kWords> d;

    __device__ __forceinline__ void load(const T* __restrict__ base, uint32_t s, uint32_t slots) {
        if (s + VEC <= slots) {
            d.load(base + s);
        } else {
#pragma unroll
            for (int i = 0; i < kWords; ++i) d.w[i] = 0;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (s + k < slots) {
                    if constexpr (sizeof(T) == 4) d.w[k] = reinterpret_cast<const uint32_t*>(base)[s + k];
                    else d.w[k >> 1] |= uint32_t(reinterpret_cast<const uint16_t*>(base)[s + k]) << (16 * (k & 1));
                }
            }
        }
    }
    __device__ __forceinline__ float get(int k) const { return Elem<T>::get(d.w, k); }
    // Moves every element down one position (element k+1 becomes k; the last
    // becomes 0), with static register indices only.
    __device__ __forceinline__ void rotate() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            const uint32_t next = i + 1 < kWords ? d.w[i + 1] : 0u;
            if constexpr (sizeof(T) == 4) d.w[i] = next;
            else d.w[i] = __builtin_amdgcn_alignbit(next, d.w[i], 16);
        }
    }
};

// A lane's gradient values, converted to T and stored.
template <typename T, int VEC>
__device__ __forceinline__ void store_values(T* __restrict__ base, uint32_t s, uint32_t slots,
                                             const float (&v)[VEC]) {
    Dwords<VEC * int(sizeof(T)) / 4> out;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) out.w[k] = __float_as_uint(v[k]);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; k += 2) out.w[k >> 1] = Elem<T>::pack(v[k], v[k + 1]);
    }
    if (s + VEC <= slots) {
        out.store(base + s);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            if (s + k < slots) {
                if constexpr (sizeof(T) == 4) reinterpret_cast<uint32_t*>(base)[s + k] = out.w[k];
                else reinterpret_cast<uint16_t*>(base)[s + k] = uint16_t(out.w[k >> 1] >> (16 * (k & 1)));
            }
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
// Cross-workgroup traffic uses no read-modify-write atomics at all (on this
// chip device-scope atomics to one line serialise at several ns each, which a
// grid of a thousand workgroups turns into microseconds).  Instead every
// workgroup owns one slot of the workspace and publishes two tagged 64-bit
// words there: its valid-token count and its partial loss.  A tag is the
// launch generation + 1, so a reader can tell this launch's words from older
// ones.  A workgroup that needs the global count reads every slot's count
// word (all-gather by polling); workgroup 0 reads every partial word in slot
// order, writes the loss and advances the generation for the next launch.
// All accesses are agent-scope relaxed atomic loads/stores (device-coherent,
// never an L2-wide writeback or invalidate).

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

// Tags published by the launch of generation `gen`.  A zero-filled workspace
// holds tag 0 everywhere, which is the tag of no launch's first use; a slot
// left from an older launch carries an older tag (32-bit, so a stale tag
// could only match after 2^32 launches on one workspace).
__device__ __forceinline__ uint32_t tag_of(uint32_t gen) { return gen + 1u; }
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t value) {
    return (uint64_t(tag) << 32) | value;
}

// Polls a tagged word until it carries `tag`.  Bounded: the grid never exceeds
// the co-resident capacity, so every workgroup publishes within microseconds;
// the wait gives up after ~1 s of the 100 MHz clock (or kWaitLimitPolls polls,
// should that clock not advance) and leaves a sticky flag.
__device__ inline uint64_t wait_tagged(Workspace* ws, const uint64_t* word, uint32_t tag) {
    uint64_t v = load_relaxed(word);
    if (uint32_t(v >> 32) == tag) return v;
    // The clock is read once per 64 polls: reading it is itself a slow scalar
    // memory access that would otherwise sit between consecutive polls.
    const uint64_t t0 = wall_clock64();
    uint32_t polls = 0;
    while (uint32_t((v = load_relaxed(word)) >> 32) != tag) {
        __builtin_amdgcn_s_sleep(kPollSleep);
        if ((++polls & 63) == 0 && (wall_clock64() - t0 > kWaitLimitTicks || polls > kWaitLimitPolls)) {
            __hip_atomic_fetch_or(&ws->flags, kFlagWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    return v;
}

// Thread 0 of worker `w` publishes its count / partial for the launch of generation `gen`.
__device__ __forceinline__ void publish_count(Workspace* ws, uint32_t w, uint32_t gen, uint32_t n) {
    store_relaxed(&ws->slot[w].count, tagged(tag_of(gen), n));
}
__device__ __forceinline__ void publish_partial(Workspace* ws, uint32_t w, uint32_t gen, float part) {
    store_relaxed(&ws->slot[w].partial, tagged(tag_of(gen), __float_as_uint(part)));
}

// Sum over the W workers' slots of this launch's count words (COUNTS) or
// partial words (otherwise), in every thread.  Each thread owns slots tid, tid+256, ...: eight
// independent loads in flight, then any word still carrying an older tag is
// waited for, then the values are added in slot order and reduced with the fixed
// workgroup tree, so the result is deterministic.
template <bool COUNTS>
__device__ inline auto gather_slots(Workspace* ws, uint32_t G, uint32_t gen, float* red_f, uint32_t* red_u) {
    using V = typename std::conditional<COUNTS, uint32_t, float>::type;
    constexpr int kBatch = 8;
    const uint32_t tag = tag_of(gen);
    V s = 0;
    for (uint32_t base = threadIdx.x; base < G; base += kThreads * kBatch) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t i = base + u * kThreads;
            const uint64_t* w = COUNTS ? &ws->slot[i].count : &ws->slot[i].partial;
            v[u] = i < G ? load_relaxed(w) : tagged(tag, 0);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t i = base + u * kThreads;
            const uint64_t* w = COUNTS ? &ws->slot[i].count : &ws->slot[i].partial;
            if (i < G && uint32_t(v[u] >> 32) != tag) v[u] = wait_tagged(ws, w, tag);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (base + u * kThreads < G) {
                if constexpr (COUNTS) s += uint32_t(v[u]);
                else s += __uint_as_float(uint32_t(v[u]));
            }
        }
    }
    if constexpr (COUNTS) return block_sum(s, red_u);
    else return block_sum(s, red_f);
}

// The global count: the coordinator gathers every count word and publishes the
// total on the release line; every worker reads the release line (one poller
// per workgroup on one line, one reader per slot line).
__device__ __forceinline__ void release_count(Workspace* ws, uint32_t gen, uint32_t n) {
    if (threadIdx.x == 0) store_relaxed(&ws->release, tagged(tag_of(gen), n));
}
__device__ inline uint32_t await_count(Workspace* ws, uint32_t gen, uint32_t* word) {
    __syncthreads();
    if (threadIdx.x == 0) *word = uint32_t(wait_tagged(ws, &ws->release, tag_of(gen)));
    __syncthreads();
    return *word;
}

// The coordinator, once it has read every partial of the launch: every workgroup
// has read the generation by then, so the next launch may use the next one.
__device__ __forceinline__ void advance_generation(Workspace* ws, uint32_t gen, uint32_t by = 1u) {
    if (threadIdx.x == 0) store_relaxed(&ws->generation, gen + by);
}

// Thread 0's generation, made known to the whole workgroup (call where every
// thread passes; `word` is LDS).
__device__ __forceinline__ uint32_t share_generation(uint32_t gen, uint32_t* word) {
    __syncthreads();
    if (threadIdx.x == 0) *word = gen;
    __syncthreads();
    return *word;
}

}  // namespace rlpl
