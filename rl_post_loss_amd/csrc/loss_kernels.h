// Internal interface between the C ABI layer (abi.cpp) and the kernels
// (loss_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rlpl {

constexpr int kVec = 16;                    // consecutive slots per lane (one 128-bit mask load)
constexpr int kThreads = 256;               // lanes per workgroup (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kTile = kVec * kThreads;      // slots per workgroup tile
constexpr int kMaxGrid = 8192;              // upper bound on the persistent grid
constexpr uint64_t kWaitLimitTicks = 100000000ull;   // ~1 s of the 100 MHz wall clock
constexpr uint32_t kWaitLimitPolls = 1u << 24;        // second bound on the same wait
constexpr uint32_t kFlagWaitTimeout = 1u;

enum { kModeBNPO = 0, kModeGRPO = 1, kModeRKL = 2 };
enum { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Device workspace.  Zero-filled once by the caller.  Each protocol word sits
// on its own 256-byte line so that polling one never contends with atomics on
// another.  Every launch leaves `arrive` and `depart` at zero and advances
// `generation` by one, ready for the next call.
struct Workspace {
    uint32_t generation;       // launch counter: read by every workgroup at its start and
    uint32_t pad0[63];         // advanced by the launch's final ticket holder
    uint64_t arrive;           // count exchange: [63:32 workgroups arrived | 31:0 their count]
    uint64_t pad1[31];
    uint64_t release;          // [63:32 tag (generation + 1) of the exchange | 31:0 total count]
    uint64_t pad2[31];
    uint64_t depart;           // finish tickets: [63:32 workgroups done | 31:0 their count]
    uint64_t pad3[31];
    uint32_t flags;            // sticky error bits (kFlagWaitTimeout)
    uint32_t pad4[63];
    uint64_t partial[kMaxGrid];   // per-workgroup partial loss: [63:32 tag (generation + 1) | 31:0 float]
};
static_assert(offsetof(Workspace, arrive) == 256, "protocol words on separate lines");
static_assert(offsetof(Workspace, release) == 512, "protocol words on separate lines");
static_assert(offsetof(Workspace, depart) == 768, "protocol words on separate lines");
static_assert(offsetof(Workspace, flags) == 1024, "protocol words on separate lines");
static_assert(offsetof(Workspace, partial) == 1280, "workspace header");
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
    int64_t tiles;         // ceil(slots / kTile)
    int32_t seq_len;
    int32_t bs;
    float beta;
    float lo;              // 1 - epsilon
    float hi;              // 1 + epsilon_high
};

// The kernel instantiation for (dtype, mode, KL on/off, gradient on/off), or NULL.
const void* pick_kernel(int dtype, int mode, bool has_kl, bool write_grad);

}  // namespace rlpl
