// Internal interface between the C ABI layer (abi.cpp) and the kernels
// (loss_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rlpl {

constexpr int kThreads = 256;               // lanes per workgroup (4 wave64)
constexpr int kWaves = kThreads / 64;
// Consecutive slots per lane: kVecLarge (one 128-bit mask load per lane) for
// large problems, kVecSmall (so that a small problem spreads over every
// compute unit) when there would be fewer than kSmallTilesPerCu large tiles
// per compute unit.  A tile is kThreads * VEC slots.
constexpr int kVecLarge = 16;
constexpr int kVecSmall = 4;
// Tiles per worker whose mask bits the striding fwd+bwd kernels keep in LDS
// (512 B per tile): 56 (28 KB) for BNPO and 40 (20 KB) for reverse-KL, which
// leaves each kernel's register-bound occupancy (4 and 6 workgroups per CU)
// within the 128 KB of LDS per CU that the host budgets.
#ifndef RLPL_BIT_TILES_POLICY
#define RLPL_BIT_TILES_POLICY 56
#endif
#ifndef RLPL_BIT_TILES_RKL
#define RLPL_BIT_TILES_RKL 40
#endif
constexpr int kBitTilesPolicy = RLPL_BIT_TILES_POLICY;
constexpr int kBitTilesRkl = RLPL_BIT_TILES_RKL;
// Kernel shapes: one tile per worker with the narrow or the wide lane, or the
// wide lane striding over several tiles per worker.
enum { kShapeSmall = 0, kShapeLarge = 1, kShapeStream = 2, kShapes = 3 };
#ifndef RLPL_SMALL_TILES_PER_CU
#define RLPL_SMALL_TILES_PER_CU 1
#endif
constexpr int kSmallTilesPerCu = RLPL_SMALL_TILES_PER_CU;
constexpr int kMaxGrid = 4096;              // upper bound on the persistent grid (gfx950: <= 256 CUs x 8)
constexpr uint64_t kWaitLimitTicks = 100000000ull;   // ~1 s of the 100 MHz wall clock
constexpr uint32_t kWaitLimitPolls = 1u << 24;        // second bound on the same wait
constexpr uint32_t kFlagWaitTimeout = 1u;
// Pause between two polls of a word another workgroup will publish, in units
// of 64 clocks (s_sleep); spaces out the polling of a whole grid.
#ifndef RLPL_POLL_SLEEP
#define RLPL_POLL_SLEEP 1
#endif
constexpr int kPollSleep = RLPL_POLL_SLEEP;

enum { kModeBNPO = 0, kModeGRPO = 1, kModeRKL = 2 };
enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

// One workgroup's published words: [63:32 tag (generation + 1) | 31:0 value].
// One slot per 256-byte line: stores from many workgroups to a shared line
// become visible to the other compute units markedly later than stores to
// lines of their own.
struct alignas(256) Slot {
    uint64_t count;            // valid-token count of the workgroup's tiles
    uint64_t partial;          // float bits of the workgroup's partial loss
    uint64_t stats[2][5];      // full-vocab reverse KL: a row chunk's online sums,
                               // double-buffered by round (tag = generation + 1 + round)
};

// Device workspace.  Zero-filled once by the caller; every launch advances
// `generation` by one and leaves nothing else that the next launch depends on.
struct Workspace {
    uint32_t generation;       // launch counter: read by every workgroup at its start,
    uint32_t pad0[63];         // advanced by workgroup 0 at the end of the launch
    uint32_t flags;            // sticky error bits (kFlagWaitTimeout)
    uint32_t pad1[63];
    uint64_t release;          // [63:32 tag | 31:0 global count], published by workgroup 0
    uint64_t pad2[31];
    Slot slot[kMaxGrid];
};
static_assert(offsetof(Workspace, flags) == 256, "header words on separate lines");
static_assert(offsetof(Workspace, release) == 512, "header words on separate lines");
static_assert(offsetof(Workspace, slot) == 768, "workspace header");
constexpr size_t kWorkspaceBytes = sizeof(Workspace);
constexpr size_t kFlagsOffset = offsetof(Workspace, flags);

// Kernel arguments (passed by value).
struct Args {
    const void* lp;        // policy / student log-probs
    const void* old;       // old-policy log-probs (BNPO, GRPO)
    const void* ref;       // reference / teacher log-probs (when the KL term is on)
    const void* adv;       // advantages (bs,) (BNPO, GRPO)
    const uint8_t* mask;
    void* grad;            // d loss / d lp (fused fwd+bwd only)
    float* loss;
    uint32_t* n_out;       // valid count(s) or NULL
    Workspace* ws;
    int64_t slots;         // bs * seq_len  (< 2^31)
    uint32_t tiles;        // ceil(slots / (kThreads * VEC))
    int32_t seq_len;
    int32_t bs;
    uint32_t row_magic;    // s / seq_len == (s * row_magic) >> row_shift for every s < 2^31
    uint32_t row_shift;
    float beta;
    float lo;              // 1 - epsilon (used only by the sign-aware form, where A < 0)
    float hi;              // 1 + epsilon_high
    uint32_t sign_aware;   // per_token = -min(A*ratio, A*clipped) instead of -A*min(ratio, clipped)
};

// The kernel instantiation for (dtype, mode, KL on/off, gradient on/off, VEC), or NULL.
const void* pick_kernel(int dtype, int mode, bool has_kl, bool write_grad, int shape);

}  // namespace rlpl
