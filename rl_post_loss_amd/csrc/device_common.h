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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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
// NT: non-temporal accesses (loads of 4, 8 or 16 bytes, stores of 16), for data
// that streams through once (they do not displace what the caches hold).
template <int N>
struct Dwords {
    uint32_t w[N];
    template <bool NT = false>
    __device__ __forceinline__ void load(const void* p) {
        if constexpr (NT && N == 1) {
            w[0] = __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
        } else if constexpr (NT && N == 2) {
            const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
            w[0] = v[0]; w[1] = v[1];
        } else if constexpr (NT) {
            static_assert(N % 4 == 0, "non-temporal accesses move 4, 8 or a multiple of 16 bytes");
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p) + q);
                w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
            }
        } else if constexpr (N == 1) {
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
    template <bool NT = false>
    __device__ __forceinline__ void store(void* p) const {
        static_assert(!NT || N % 4 == 0, "non-temporal accesses move 16 bytes");
        if constexpr (NT) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q)
                __builtin_nontemporal_store(u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]},
                                            static_cast<u32x4*>(p) + q);
        } else if constexpr (N == 1) {
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

// Where a lane's VEC slots lie.  A lane whose slots would take more than 16
// bytes of a plane takes them as C = VEC / E chunks of E slots (E = 16 bytes
// of the plane's elements), chunk c of lane l of a wavefront at
// wave_start + (c * 64 + l) * E, so that each 16-byte access of a wavefront
// covers 1 KB of the plane without a gap; with one chunk per lane (E == VEC)
// the slots are s .. s+VEC-1.  `s` is always the lane's slot in the one-chunk
// layout (tile * lanes * VEC + lane * VEC): the wavefront covers the same
// slots either way.  Measured on fwd+bwd BNPO, bf16: a lane of 16 consecutive
// slots (two 16-byte accesses per plane, each wavefront access covering every
// other 16 bytes of 2 KB) ran 8 % slower at 2^22, 2^26 and 2^27 slots than two
// chunks of 8.
template <typename T, int VEC>
constexpr int chunk_slots() {
    return VEC * int(sizeof(T)) > 16 ? 16 / int(sizeof(T)) : VEC;
}
template <int VEC, int E>
__device__ __forceinline__ uint32_t chunk_slot(uint32_t s, int c) {
    if constexpr (E == VEC) return s;
    const uint32_t lane = threadIdx.x & 63u;
    return s - lane * uint32_t(VEC) + (uint32_t(c) * 64u + lane) * uint32_t(E);
}

// VEC elements of one plane (in E-slot chunks, as above).  A chunk that runs
// past `slots` (only in the last tile) moves its in-range elements one by one
// and zero-fills.
template <typename T, int VEC>
struct Plane {
    static constexpr int kWords = VEC * int(sizeof(T)) / 4;
    Dwords<kWords> d;

    // CHECK: the lane may run past `slots` (else the caller knows that its whole
    // tile is in range, and the test, a branch per lane, is left out).
    template <bool NT = false, bool CHECK = true, int E = VEC>
    __device__ __forceinline__ void load(const T* __restrict__ base, uint32_t s, uint32_t slots) {
        if constexpr (E == VEC) {
            load_run<NT, CHECK, VEC>(base, s, slots, d.w);
        } else {
#pragma unroll
            for (int c = 0; c < VEC / E; ++c) load_chunk<NT, CHECK, E>(base, s, slots, c);
        }
    }
    // Chunk c of the lane (E slots) only.
    template <bool NT, bool CHECK, int E>
    __device__ __forceinline__ void load_chunk(const T* __restrict__ base, uint32_t s, uint32_t slots, int c) {
        constexpr int kW = E * int(sizeof(T)) / 4;   // words per chunk (4: 16 bytes)
        uint32_t w[kW];
        load_run<NT, CHECK, E>(base, chunk_slot<VEC, E>(s, c), slots, w);
#pragma unroll
        for (int i = 0; i < kW; ++i) d.w[c * kW + i] = w[i];
    }
    // N consecutive elements from slot s into N * sizeof(T) / 4 words.
    template <bool NT, bool CHECK, int N>
    static __device__ __forceinline__ void load_run(const T* __restrict__ base, uint32_t s, uint32_t slots,
                                                    uint32_t (&w)[N * int(sizeof(T)) / 4]) {
        constexpr int kW = N * int(sizeof(T)) / 4;
        if (!CHECK || s + N <= slots) {
            Dwords<kW> v;
            v.template load<NT>(base + s);
#pragma unroll
            for (int i = 0; i < kW; ++i) w[i] = v.w[i];
        } else {
#pragma unroll
            for (int i = 0; i < kW; ++i) w[i] = 0;
#pragma unroll
            for (int k = 0; k < N; ++k) {
                if (s + k < slots) {
                    if constexpr (sizeof(T) == 4) w[k] = reinterpret_cast<const uint32_t*>(base)[s + k];
                    else w[k >> 1] |= uint32_t(reinterpret_cast<const uint16_t*>(base)[s + k]) << (16 * (k & 1));
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

// N consecutive values converted to T and stored from slot s.
template <typename T, int N, bool NT, bool CHECK>
__device__ __forceinline__ void store_run(T* __restrict__ base, uint32_t s, uint32_t slots, const float* v) {
    Dwords<N * int(sizeof(T)) / 4> out;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < N; ++k) out.w[k] = __float_as_uint(v[k]);
    } else {
#pragma unroll
        for (int k = 0; k < N; k += 2) out.w[k >> 1] = Elem<T>::pack(v[k], v[k + 1]);
    }
    if (!CHECK || s + N <= slots) {
        out.template store<NT>(base + s);
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            if (s + k < slots) {
                if constexpr (sizeof(T) == 4) reinterpret_cast<uint32_t*>(base)[s + k] = out.w[k];
                else reinterpret_cast<uint16_t*>(base)[s + k] = uint16_t(out.w[k >> 1] >> (16 * (k & 1)));
            }
        }
    }
}

// A lane's gradient values (in E-slot chunks, as the planes), converted to T and stored.
template <typename T, int VEC, bool NT = false, bool CHECK = true, int E = VEC>
__device__ __forceinline__ void store_values(T* __restrict__ base, uint32_t s, uint32_t slots,
                                             const float (&v)[VEC]) {
#pragma unroll
    for (int c = 0; c < VEC / E; ++c) store_run<T, E, NT, CHECK>(base, chunk_slot<VEC, E>(s, c), slots, v + c * E);
}

// ----------------------------------------------------------------------------- reductions

// A wavefront's sum, in every lane, from DPP lane moves (each a plain VALU
// operand modifier; a shuffle would go through the LDS crossbar, about a
// hundred cycles per step): pairs and quads (quad_perm), half-rows and rows
// of 16 (row_half_mirror, row_mirror), then rows 1 and 3 take the last lane
// of rows 0 and 2 (row_bcast:15) and rows 2 and 3 that of row 1
// (row_bcast:31), which leaves the total in lane 63.  A fixed order, so the
// float sum is deterministic.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
    // Rows outside ROW_MASK receive 0 (the identity of the sums below).
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xF, false));
}
template <typename V>
__device__ __forceinline__ V wave_sum_dpp(V v) {
    auto bits = [](V x) { return __builtin_bit_cast(uint32_t, x); };
    auto from = [](uint32_t x) { return __builtin_bit_cast(V, x); };
    v = v + from(dpp_move<0xB1>(bits(v)));          // quad_perm [1, 0, 3, 2]
    v = v + from(dpp_move<0x4E>(bits(v)));          // quad_perm [2, 3, 0, 1]
    v = v + from(dpp_move<0x141>(bits(v)));         // row_half_mirror
    v = v + from(dpp_move<0x140>(bits(v)));         // row_mirror
    v = v + from(dpp_move<0x142, 0xA>(bits(v)));    // row_bcast:15
    v = v + from(dpp_move<0x143, 0xC>(bits(v)));    // row_bcast:31
    return from(uint32_t(__builtin_amdgcn_readlane(int(bits(v)), 63)));
}
__device__ __forceinline__ float wave_sum(float v) { return wave_sum_dpp(v); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return wave_sum_dpp(v); }

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

// N workgroup sums at once (one pair of barriers), in every thread, each in
// the fixed order of block_sum.  `red` is LDS of N * kWaves values.
template <int N, typename V>
__device__ __forceinline__ void block_sum_n(V (&v)[N], V* red) {
#pragma unroll
    for (int u = 0; u < N; ++u) v[u] = wave_sum(v[u]);
    const int wave = threadIdx.x >> 6;
    __syncthreads();                       // red[] may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int u = 0; u < N; ++u) red[u * kWaves + wave] = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < N; ++u) {
        V t = red[u * kWaves];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) t += red[u * kWaves + i];
        v[u] = t;
    }
}

// ----------------------------------------------------------------------------- launch identity

// The dispatch id of the running launch: the index of its packet in its
// hardware queue (the LLVM intrinsic behind the code object's dispatch-id
// register; it has no clang builtin).
extern "C" __device__ uint64_t rlpl_dispatch_id(void) __asm("llvm.amdgcn.dispatch.id");

// A launch's pair of 32-bit tags: its dispatch id plus two independent hashes
// of its queue's address.  Two launches on one queue differ in both tags (for
// 2^32 launches); two launches on different queues agree in both only where
// the queues' two hash differences coincide (chance 2^-32 per queue pair) and
// the dispatch ids differ by exactly that amount.  Never zero, so a
// zero-filled entry is never taken for a published one.
struct Tag {
    uint32_t t0, t1;
};
__device__ __forceinline__ uint32_t mix32(uint32_t h) {   // MurmurHash3's finaliser
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}
__device__ __forceinline__ Tag launch_tag() {
    const uint32_t did = uint32_t(rlpl_dispatch_id());
    const uint64_t q = uint64_t(reinterpret_cast<uintptr_t>(__builtin_amdgcn_queue_ptr()));
    const uint32_t lo = uint32_t(q), hi = uint32_t(q >> 32);
    Tag t{did + mix32(lo ^ mix32(hi)), did + mix32(lo ^ mix32(hi ^ 0x9e3779b9u))};
    if (t.t0 == 0u) t.t0 = 0x80000000u;
    if (t.t1 == 0u) t.t1 = 0x80000000u;
    return t;
}

// ----------------------------------------------------------------------------- published entries
//
// The policy-loss kernels exchange values through Entry records of the
// workspace (per worker: its valid count and its partial loss; from the
// coordinator: the global count).  No read-modify-write atomics: on this chip
// device-scope atomics to one line serialise at several ns each.  Entries are
// packed 16 bytes apart, because reading lines that other compute units have
// just written costs per line read; each is written and read with one 16-byte
// device-coherent access (cache policy sc1, the bits of an agent-scope atomic).

constexpr int kCoherent = 16;   // buffer cache policy: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t entry_view(const Workspace* ws) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<Workspace*>(ws), 0, int(kEntryViewBytes), 0x00020000);
}
constexpr uint32_t kReleaseOff = uint32_t(offsetof(Workspace, release));
__device__ __forceinline__ uint32_t cnt_off(uint32_t w) { return uint32_t(offsetof(Workspace, cnt)) + 16u * w; }
__device__ __forceinline__ uint32_t par_off(uint32_t w) { return uint32_t(offsetof(Workspace, par)) + 16u * w; }
__device__ __forceinline__ uint32_t tail_off(uint32_t w) { return uint32_t(offsetof(Workspace, tail)) + 16u * w; }
__device__ __forceinline__ uint32_t hpair_off(uint32_t w) { return uint32_t(offsetof(Workspace, hpair)) + 16u * w; }
__device__ __forceinline__ uint32_t tpair_off(uint32_t w) { return uint32_t(offsetof(Workspace, tpair)) + 16u * w; }
// An item of a gather that has no entry: it adds nothing and is never awaited.
constexpr uint32_t kNoEntry = 0xFFFFFFFFu;

__device__ __forceinline__ void publish(__amdgpu_buffer_rsrc_t v, uint32_t off, Tag t, uint32_t value) {
    const u32x4 x = {value, t.t0, value, t.t1};
    __builtin_amdgcn_raw_buffer_store_b128(x, v, off, 0, kCoherent);
}
// A pair entry: values a and b, each beside one of the launch's tags.
__device__ __forceinline__ void publish_pair(__amdgpu_buffer_rsrc_t v, uint32_t off, Tag t, uint32_t a, uint32_t b) {
    const u32x4 x = {a, t.t0, b, t.t1};
    __builtin_amdgcn_raw_buffer_store_b128(x, v, off, 0, kCoherent);
}
// One read of an entry: true, with its value, when it holds this launch's value.
__device__ __forceinline__ bool read_entry(__amdgpu_buffer_rsrc_t v, uint32_t off, Tag t, uint32_t& value) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(v, off, 0, kCoherent);
    value = x[0];
    return x[1] == t.t0 && x[3] == t.t1 && x[0] == x[2];
}
// Between two polls: a pause of SLEEP x 64 clocks, and a compiler barrier so
// that the next poll is a new load.  Each poll is a read that goes to the
// memory side; the pauses (longer for the release, which up to every worker
// polls) keep that traffic small without delaying the waits measurably.
constexpr int kGatherSleep = 4;
constexpr int kReleaseSleep = 8;
template <int SLEEP>
__device__ __forceinline__ void poll_pause() {
    __builtin_amdgcn_s_sleep(SLEEP);
    __asm__ volatile("" ::: "memory");
}

// One poll of up to N entries: the reads of those still awaited (bit j of
// `miss`) go out together, and are checked once all have returned; an entry
// not awaited reads the workspace's first 16 bytes instead (in bounds, not
// used), so that no read waits behind the check of another.
template <int N>
__device__ __forceinline__ void poll_entries(__amdgpu_buffer_rsrc_t view, const uint32_t (&at)[N], Tag tg,
                                             uint32_t& miss, uint32_t (&val)[N]) {
    u32x4 x[N];
#pragma unroll
    for (int j = 0; j < N; ++j)
        x[j] = __builtin_amdgcn_raw_buffer_load_b128(view, (miss >> j) & 1u ? at[j] : 0u, 0, kCoherent);
#pragma unroll
    for (int j = 0; j < N; ++j)
        if (((miss >> j) & 1u) && x[j][1] == tg.t0 && x[j][3] == tg.t1 && x[j][0] == x[j][2]) {
            val[j] = x[j][0];
            miss &= ~(1u << j);
        }
}

// The wait limits of the policy-loss kernels in 100 MHz ticks: the caller's
// overrides in the workspace header (written by the host only), else the
// defaults.  Read once at the start of a workgroup, where the read overlaps
// the first data loads: a read just before a poll would hold the poll up by
// a memory round trip.
struct Limits {
    uint32_t steal, release, giveup;
    bool steal_set, release_set;   // set by the caller (else the defaults)
    uint64_t begin;                // the workgroup's start, on the same clock
    // The limit of a wait that follows this workgroup's own share of the work:
    // the other workers, doing shares like it, may finish as much later as it
    // took, so a default limit grows by the time since the start; a limit the
    // caller set is kept as it is.
    __device__ __forceinline__ uint32_t steal_now() const {
        return steal_set ? steal : steal + uint32_t(uint64_t(wall_clock64()) - begin);
    }
    __device__ __forceinline__ uint32_t release_now() const {
        return release_set ? release : release + uint32_t(uint64_t(wall_clock64()) - begin);
    }
};
__device__ __forceinline__ Limits read_limits(const Workspace* ws) {
    const uint4 v = *reinterpret_cast<const uint4*>(&ws->steal_ticks);
    return Limits{v.x != 0u ? v.x : kStealTicks, v.y != 0u ? v.y : kReleaseTicks, v.z != 0u ? v.z : kGiveUpTicks,
                  v.x != 0u, v.y != 0u, uint64_t(wall_clock64())};
}

// Sum over W items' entries (valid counts, or the float bits of partial
// losses: V = uint32_t / float), in every thread; item i's entry is at byte
// off(i) of the view, or off(i) == kNoEntry for an item that adds nothing.
// Thread i takes items i, i + kThreads, ... in turn, B at a time (a chunk).
// Entries not yet published are polled until they are, or until `limit`
// ticks have passed; entries still missing then are computed here, one item
// at a time by the whole workgroup (compute(i) is workgroup-uniform and
// bit-identical to what the item's owner publishes).  The sum is taken in one
// fixed order (each thread's items in turn, then the workgroup tree), so it
// never depends on which entries were computed here.  `list` is LDS of
// kThreads + 1 words, not used by compute().
//
// between() runs once the first chunk's reads are issued and before they are
// used: a store made there (the release) does not hold them up.  Loads and
// stores of a wavefront share one in-order completion counter, so a load
// issued after a device-coherent store waits for that store's write-through.
template <typename V, typename O, typename F, typename G>
__device__ inline V gather(__amdgpu_buffer_rsrc_t view, O&& off, uint32_t W, Tag tg, uint32_t limit,
                           uint32_t* list, V* red, F&& compute, G&& between) {
    constexpr int B = 4;
    V s = 0;
    for (uint32_t c0 = 0; c0 < W; c0 += B * kThreads) {
        u32x4 raw[B];
        uint32_t at[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t i = c0 + threadIdx.x + j * kThreads;
            at[j] = i < W ? off(i) : kNoEntry;
            // (an item with no entry reads the workspace's first 16 bytes, unused)
            raw[j] = __builtin_amdgcn_raw_buffer_load_b128(view, at[j] != kNoEntry ? at[j] : 0u, 0, kCoherent);
        }
        if (c0 == 0) between();
        uint32_t val[B];
        uint32_t miss = 0;                     // bit j: item c0 + tid + j * kThreads not seen yet
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const u32x4 x = raw[j];
            val[j] = at[j] != kNoEntry ? x[0] : 0u;
            if (at[j] != kNoEntry && !(x[1] == tg.t0 && x[3] == tg.t1 && x[0] == x[2])) miss |= 1u << j;
        }
        if (miss) {
            const uint64_t t0 = wall_clock64();
            for (uint32_t n = 1; miss; ++n) {
                poll_pause<kGatherSleep>();
                poll_entries<B>(view, at, tg, miss, val);
                if ((n & 7u) == 0u && uint64_t(wall_clock64()) - t0 > limit) break;
            }
        }
        // Workers still missing: computed here.  The list holds the threads that
        // have any (their order does not matter: each value lands in its own place).
        if (__syncthreads_or(miss != 0u)) {
            if (threadIdx.x == 0) list[kThreads] = 0;
            __syncthreads();
            if (miss) list[atomicAdd(&list[kThreads], 1u)] = threadIdx.x | (miss << 16);
            __syncthreads();
            const uint32_t n_list = list[kThreads];
            for (uint32_t k = 0; k < n_list; ++k) {
                const uint32_t t = list[k] & 0xFFFFu, bits = list[k] >> 16;
                // One copy of compute() (a rolled loop); the value lands in val[] by
                // static indices.
#pragma unroll 1
                for (uint32_t j = 0; j < uint32_t(B); ++j) {
                    if (!(bits & (1u << j))) continue;
                    const V v = compute(c0 + t + j * kThreads);
                    uint32_t u;
                    if constexpr (std::is_same<V, float>::value) u = __float_as_uint(v);
                    else u = v;
                    if (threadIdx.x == t) {
#pragma unroll
                        for (int q = 0; q < B; ++q)
                            if (uint32_t(q) == j) val[q] = u;
                    }
                }
            }
            __syncthreads();                   // list[] is reused by the next chunk
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if constexpr (std::is_same<V, float>::value) s += __uint_as_float(val[j]);
            else s += val[j];
        }
    }
    return block_sum(s, red);
}

// The thread of each workgroup that publishes its count, the one that
// publishes its partial, and the one that polls for the release: each in a
// wavefront of its own, so that no poll waits for the write-through of a
// store made before it in the same wavefront.
constexpr uint32_t kCountThread = 0;
constexpr uint32_t kPartialThread = 64;
constexpr uint32_t kReleaseThread = 128;

// The global count, in every thread: the coordinator's release, or, when it
// has not come within the release limit, this workgroup's own gather of the
// counts (gather_counts(), workgroup-uniform).  `word` is LDS of two words.
template <typename F>
__device__ inline uint32_t await_release(__amdgpu_buffer_rsrc_t view, uint32_t limit, Tag tg, uint32_t* word,
                                         F&& gather_counts) {
    __syncthreads();
    if (threadIdx.x == kReleaseThread) {
        uint32_t v = 0;
        bool ok = read_entry(view, kReleaseOff, tg, v);
        if (!ok) {
            const uint64_t t0 = wall_clock64();
            for (uint32_t n = 1; !ok; ++n) {
                poll_pause<kReleaseSleep>();
                ok = read_entry(view, kReleaseOff, tg, v);
                if ((n & 7u) == 0u && uint64_t(wall_clock64()) - t0 > limit) break;
            }
        }
        word[0] = v;
        word[1] = ok ? 1u : 0u;
    }
    __syncthreads();
    if (word[1]) return word[0];
    return gather_counts();
}

// ----------------------------------------------------------------------------- full-vocab protocol
//
// The full-vocab kernels publish generation-tagged 64-bit words in per-
// workgroup slots: [63:32 tag | 31:0 value], with tag = generation + 1 (+ the
// exchange round); workgroup 0 advances the generation once it has read every
// partial of the launch (after which no workgroup of the launch reads it).

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

__device__ __forceinline__ uint32_t tag_of(uint32_t gen) { return gen + 1u; }
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t value) {
    return (uint64_t(tag) << 32) | value;
}

// Polls a tagged word until it carries `tag`, for at most `limit` ticks of the
// 100 MHz clock (and kWaitLimitPolls polls, should that clock not advance).
// Returns whether it did; `v` holds the last word read.
__device__ inline bool wait_tagged(const uint64_t* word, uint32_t tag, uint64_t limit, uint64_t& v) {
    v = load_relaxed(word);
    if (uint32_t(v >> 32) == tag) return true;
    // The clock is read after the first failed poll and then once per 64 polls:
    // reading it is itself a slow scalar memory access that would otherwise sit
    // between consecutive polls.
    const uint64_t t0 = wall_clock64();
    uint32_t polls = 0;
    while (uint32_t((v = load_relaxed(word)) >> 32) != tag) {
        __builtin_amdgcn_s_sleep(kPollSleep);
        ++polls;
        if ((polls == 1u || (polls & 63u) == 0u) &&
            (uint64_t(wall_clock64()) - t0 > limit || polls > kWaitLimitPolls))
            return false;
    }
    return true;
}

__device__ __forceinline__ void publish_partial(Workspace* ws, uint32_t w, uint32_t gen, float part) {
    store_relaxed(&ws->slot[w].partial, tagged(tag_of(gen), __float_as_uint(part)));
}

// Workgroup 0's sum of the G workgroups' partial words of this launch, in
// every thread, in slot order then the fixed workgroup tree (deterministic).
// Each thread owns slots tid, tid+256, ...: eight loads in flight, then any
// word still carrying an older tag is waited for.  A wait that gives up (after
// `limit` ticks) sets the sticky flag and makes the sum NaN.
__device__ inline float gather_partials(Workspace* ws, uint32_t G, uint32_t gen, uint32_t limit, float* red_f) {
    constexpr int kBatch = 8;
    const uint32_t tag = tag_of(gen);
    float s = 0.0f;
    bool lost = false;
    for (uint32_t base = threadIdx.x; base < G; base += kThreads * kBatch) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t i = base + u * kThreads;
            v[u] = i < G ? load_relaxed(&ws->slot[i].partial) : tagged(tag, 0);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const uint32_t i = base + u * kThreads;
            if (i < G && uint32_t(v[u] >> 32) != tag && !wait_tagged(&ws->slot[i].partial, tag, limit, v[u]))
                lost = true;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (base + u * kThreads < G) s += __uint_as_float(uint32_t(v[u]));
    }
    if (lost) {
        __hip_atomic_fetch_or(&ws->flags, kFlagWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s = __builtin_nanf("");
    }
    return block_sum(s, red_f);
}

// Workgroup 0, once it has read every partial of the launch: every workgroup
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
