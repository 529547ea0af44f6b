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
// (512 B per tile): 60 (30 KB) for BNPO and 40 (20 KB) for reverse-KL, which
// leaves each kernel's register-bound occupancy (4 and 6 workgroups per CU)
// within the 128 KB of LDS per CU that the host budgets.  Tiles past them
// read their mask bytes a second time (slower per tile than kept bits).
constexpr int kBitTilesPolicy = 60;
constexpr int kBitTilesRkl = 40;
// GRPO's striding kernels own contiguous runs of at most kMaxPer tiles per
// worker (the host sizes the grid so), keep one word per owned tile in LDS
// (the counts of the tile's first and last row) and the mask bits of the
// first kBitTilesGrpo tiles: with the per-row counts of a tile (16 KB) that
// is 28 KB, four workgroups per compute unit.
constexpr int kMaxPer = 1024;
constexpr int kBitTilesGrpo = 12;
// Kernel shapes: one tile per worker with the narrow or the wide lane, or the
// wide lane striding over several tiles per worker, its gradient stored
// through the caches or, from kNtGradBytes of inputs and gradient on,
// non-temporally.
enum { kShapeSmall = 0, kShapeLarge = 1, kShapeStream = 2, kShapeStreamNt = 3, kShapes = 4 };
// Bytes of mask, planes and gradient (whole arrays) from which a striding
// fwd+bwd launch stores its gradient non-temporally.  Measured crossover on
// gfx950 (interleaved A/B, fused BNPO bf16 at seq_len 4096): cached stores
// 6 % faster at 1.28 GB, non-temporal ones 1 % faster at 1.36 GB and 6-8 %
// from 1.5 GB on; fp32 BNPO, reverse KL and GRPO cross in the same range.
constexpr int64_t kNtGradBytes = int64_t(5) << 28;   // 1.25 GiB
// The narrow lane is taken when a problem has fewer wide tiles than compute units.
constexpr int kSmallTilesPerCu = 1;
constexpr int kMaxGrid = 4096;              // upper bound on the persistent grid (gfx950: <= 256 CUs x 8)
// Waits of the policy-loss kernels, in ticks of the 100 MHz wall clock.  A
// coordinator that has waited kStealTicks for a worker's published count or
// partial computes that value itself from the inputs; a worker that has waited
// kReleaseTicks for the global count gathers it itself.  Either way the result
// is bit-identical, so no wait depends on another workgroup being resident.
// Unless the caller sets them, both limits grow by the time the waiting
// workgroup has run, since the peers it waits for do shares of work like its own.
constexpr uint32_t kStealTicks = 5000;      // 50 us
constexpr uint32_t kReleaseTicks = 20000;   // 200 us
// The full-vocab kernels' waits for the partial sums of their peers give up
// after ~1 s (kGiveUpTicks, or kWaitLimitPolls polls should the clock not
// advance): the loss is then NaN and a sticky flag is set.
constexpr uint32_t kGiveUpTicks = 100000000u;
constexpr uint32_t kWaitLimitPolls = 1u << 24;
constexpr uint32_t kFlagWaitTimeout = 1u;
// Pause between two polls of a word another workgroup will publish, in units
// of 64 clocks (s_sleep).
constexpr int kPollSleep = 1;

enum { kModeBNPO = 0, kModeGRPO = 1, kModeRKL = 2 };
enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

// One value published by one workgroup for the others: two 64-bit words
// [63:32 tag t0 | 31:0 value] and [63:32 tag t1 | 31:0 value], written and
// read as one 16-byte access.  A reader takes it only when both tags are its
// launch's and both values agree, so a torn or stale entry is never taken.
// A pair entry holds two values instead, [t0 | a] and [t1 | b]: each 8-byte
// half carries its own tag, so a read that mixes the halves of two stores
// fails a tag check.
struct alignas(16) Entry {
    uint64_t w[2];
};

// Per-workgroup words of the full-vocab kernels: [63:32 tag (generation + 1 +
// round) | 31:0 value].  One slot per 256-byte line: stores from many
// workgroups to a shared line become visible to the other compute units
// markedly later than stores to lines of their own.
struct alignas(256) Slot {
    uint64_t partial;          // float bits of the workgroup's partial loss
    uint64_t stats[2][5];      // a row piece's online sums, double-buffered by exchange
};

// Device workspace.  Zero-filled once by the caller.  The policy-loss kernels
// tag what they publish with their launch's identity (no state carried from
// one launch to the next); the full-vocab kernels advance `generation` by the
// number of tags they used.  Header words sit on 128-byte lines of their own.
struct Workspace {
    uint32_t generation;       // full-vocab kernels: launch counter
    uint32_t pad0[31];
    uint32_t flags;            // sticky error bits (kFlagWaitTimeout)
    uint32_t pad1[31];
    uint32_t steal_ticks;      // caller-set wait limits (0 selects kStealTicks,
    uint32_t release_ticks;    // kReleaseTicks and kGiveUpTicks); written by the
    uint32_t giveup_ticks;     // host only (rlpl_workspace_set_limits)
    uint32_t pad2[29];
    Entry release;             // the global valid count N, published by the coordinator
    uint64_t pad3[14];
    Entry cnt[kMaxGrid];       // per worker: its valid-token count (GRPO: that of its run's first row)
    Entry par[kMaxGrid];       // per worker: float bits of its partial loss (GRPO: of the rows inside its run)
    Entry tail[kMaxGrid];      // GRPO, per worker: the valid count of its run's last row
    Entry hpair[kMaxGrid];     // GRPO, per worker: its run's first row's count and unscaled sum of terms
    Entry tpair[kMaxGrid];     // GRPO, per worker: the same for its run's last row
    Slot slot[kMaxGrid];       // full-vocab kernels
};
static_assert(offsetof(Workspace, flags) == 128, "header words on separate lines");
static_assert(offsetof(Workspace, steal_ticks) == 256, "header words on separate lines");
static_assert(offsetof(Workspace, release) == 384, "header words on separate lines");
static_assert(offsetof(Workspace, cnt) == 512, "workspace header");
static_assert(sizeof(Slot) == 256, "one slot per line");
constexpr size_t kWorkspaceBytes = sizeof(Workspace);
constexpr size_t kFlagsOffset = offsetof(Workspace, flags);
constexpr size_t kLimitsOffset = offsetof(Workspace, steal_ticks);
// Bytes from the workspace's start that the policy-loss kernels address with
// 16-byte buffer accesses (the header and the five entry arrays).
constexpr size_t kEntryViewBytes = offsetof(Workspace, slot);

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
    uint32_t per;          // striding GRPO kernels: tiles per worker (each worker owns a contiguous run)
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
// The same for one element type T of the log-probs (float, _Float16, __bf16);
// instantiated by that dtype's source file.
template <typename T>
const void* pick_typed(int mode, bool has_kl, bool write_grad, int shape);

// The library's own scratch (the per-token kernels' part of a workspace), for
// the entry point that allocates nothing: its device address on the current
// device (0 on success), and a kernel that zero-fills n 16-byte words.
constexpr size_t kScratchBytes = kEntryViewBytes;
int scratch_address(void** out);
const void* clear_kernel_ptr();

}  // namespace rlpl
