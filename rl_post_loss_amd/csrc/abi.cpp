// C ABI of the fused policy-loss library (declared in include/rl_post_loss.h).
//
// Each entry point validates its arguments on the host (no HIP call before
// they pass), then picks the kernel instantiation <dtype, mode, KL on/off,
// gradient on/off>, sizes the persistent grid from the per-device
// occupancy cache and enqueues exactly one launch on the caller's stream.
// Nothing here allocates device memory or synchronises the stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "logprob_kernels.h"
#include "loss_kernels.h"
#include "rl_post_loss.h"
#include "row_divisor.h"
#include "vocab_kernels.h"

namespace {

using rlpl::Args;
using rlpl::kModeBNPO;
using rlpl::kModeGRPO;
using rlpl::kModeRKL;

constexpr int kAbiVersion = 1;
constexpr int kMaxDevices = 64;
constexpr size_t kLdsPerCu = 128 * 1024;   // LDS budget per CU for co-residency

// Per-device launch facts, filled once per device (thread-safe) and then read-only.
struct DeviceInfo {
    int status = RLPL_ERR_DEVICE;
    int cus = 0;
    int grid_cap[3][3][rlpl::kShapes] = {};  // [dtype][mode][kernel shape]: co-resident workgroups
    int vocab_cap[3] = {};                   // [dtype]: co-resident workgroups of the full-vocab kernels
};

// Co-resident workgroups of `kernel` per CU: the occupancy query, limited so
// that the workgroups' LDS stays within kLdsPerCu (all of a CU's 160 KB is
// not always usable: five workgroups of 32 KB are not co-resident on gfx950).
// 0 when the query fails.
int blocks_per_cu(const void* kernel) {
    int nb = 0;
    hipFuncAttributes attr;
    if (!kernel || hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, rlpl::kThreads, 0) != hipSuccess ||
        nb < 1 || hipFuncGetAttributes(&attr, kernel) != hipSuccess)
        return 0;
    if (attr.sharedSizeBytes > 0) {
        const int by_lds = int(kLdsPerCu / attr.sharedSizeBytes);
        if (by_lds < nb) nb = by_lds;
    }
    return nb;
}
DeviceInfo g_info[kMaxDevices];
std::once_flag g_once[kMaxDevices];

void init_device(int dev, DeviceInfo& info) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return;
    if (cus <= 0) return;
    info.cus = cus;
    for (int dt = 0; dt < 3; ++dt)
        for (int mode = 0; mode < 3; ++mode)
            for (int shape = 0; shape < rlpl::kShapes; ++shape) {
                // The whole family shares one grid size so that its forward-only and
                // fwd+bwd kernels reduce over identical partitions (identical losses);
                // the size is what the device holds at once, so that on an idle
                // device no workgroup waits for another to be dispatched.
                int occ = 1 << 30;
                for (int kl = 0; kl < 2; ++kl)
                    for (int wg = 0; wg < 2; ++wg) {
                        const int nb = blocks_per_cu(
                            rlpl::pick_kernel(dt, mode, kl != 0 || mode == kModeRKL, wg != 0, shape));
                        if (nb < 1) return;
                        if (nb < occ) occ = nb;
                    }
                long cap = long(occ) * cus;
                if (cap > rlpl::kMaxGrid) cap = rlpl::kMaxGrid;
                info.grid_cap[dt][mode][shape] = int(cap);
            }
    // The contraction kernels take their LDS ring as dynamic LDS beyond the default limit.
    for (int dt : {RLPL_F16, RLPL_BF16})
        for (int epi = 0; epi < 4; ++epi)
            for (int ab = 0; ab < 4; ++ab) {
                const void* k = rlpl::pick_gemm_kernel(dt, epi, ab & 1, ab >> 1);
                if (k && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, rlpl::kGemmDynLds) !=
                             hipSuccess)
                    return;
            }
    for (int dt = 0; dt < 3; ++dt) {
        // Every variant shares one co-resident capacity (the smallest one).
        int occ = 0;
        for (int mode : {rlpl::kVocabFwd, rlpl::kVocabResident, rlpl::kVocabStream}) {
            const int nb = blocks_per_cu(rlpl::pick_vocab_kernel(dt, mode));
            if (nb < 1) return;
            if (occ == 0 || nb < occ) occ = nb;
        }
        long cap = long(occ) * cus;
        if (cap > rlpl::kMaxGrid) cap = rlpl::kMaxGrid;
        info.vocab_cap[dt] = int(cap);
    }
    info.status = RLPL_OK;
}

int current_device(const DeviceInfo** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RLPL_ERR_DEVICE;
    std::call_once(g_once[dev], [dev] { init_device(dev, g_info[dev]); });
    *out = &g_info[dev];
    return g_info[dev].status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t elem_bytes(int dtype) { return dtype == RLPL_F32 ? 4 : 2; }

// Shape, dtype and the pointers every operation shares.
int check_common(const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype,
                 const float* loss_out, const uint32_t* n_valid_out, const void* workspace,
                 size_t workspace_bytes) {
    // The per-token kernels address the workspace's header and entry arrays only.
    if (!mask || !loss_out) return RLPL_ERR_NULL;
    if (bs < 1 || seq_len < 1 || bs > (int64_t(1) << 31) / seq_len ||
        bs * seq_len >= (int64_t(1) << 31))
        return RLPL_ERR_SHAPE;
    if (dtype != RLPL_F32 && dtype != RLPL_F16 && dtype != RLPL_BF16) return RLPL_ERR_DTYPE;
    if (mask_dtype != RLPL_MASK_BOOL && mask_dtype != RLPL_MASK_INT8) return RLPL_ERR_DTYPE;
    if (!aligned(mask, 16) || !aligned(loss_out, 4) || (n_valid_out && !aligned(n_valid_out, 4)))
        return RLPL_ERR_ALIGN;
    if (!workspace || workspace_bytes < rlpl::kEntryViewBytes) return RLPL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return RLPL_ERR_ALIGN;
    return RLPL_OK;
}

// A plain launch.  The grid is capped at what the device holds at once, so on
// an idle device every workgroup of an exchange kernel is resident together;
// correctness does not rest on it (a workgroup that waits too long for another
// computes the awaited value itself).  A cooperative launch would guarantee
// co-residency but costs ~16 us of extra dispatch latency per call here.
template <typename A>
int launch(const void* kernel, const A& a, dim3 grid, hipStream_t stream, int threads = rlpl::kThreads,
           size_t dyn_lds = 0) {
    void* params[] = {const_cast<A*>(&a)};
    const hipError_t e = hipLaunchKernel(kernel, grid, dim3(threads), params, dyn_lds, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // clear the sticky launch error
        return RLPL_ERR_LAUNCH;
    }
    return RLPL_OK;
}

struct Shape {
    int kernel;      // rlpl::kShapeSmall / kShapeLarge / kShapeStream / kShapeStreamNt
    int vec;
    uint32_t tiles;
    int64_t grid;
    uint32_t per;    // GRPO: tiles per worker (a contiguous run each)
};

// Kernel shape, tile count and grid of a call on this device: one
// coordinating workgroup plus one worker per tile whenever that many
// workgroups of the one-tile kernel are co-resident (small problems take the
// narrow lane so that every compute unit gets a tile), else the striding
// kernel: per is the fewest tiles per worker that fit the co-resident
// workgroups, and the grid the runs of `per` tiles it takes (so that every
// worker has one).  GRPO's workers own those contiguous runs; BNPO's and
// reverse-KL's share the tiles out in groups (Sweep in loss_kernels_impl.h).
// nt_grad: a striding launch stores its gradient non-temporally.
int launch_shape(const DeviceInfo* info, int dtype, int mode, int64_t slots, bool nt_grad, Shape* out) {
    const int64_t large_tile = int64_t(rlpl::kThreads) * rlpl::kVecLarge;
    const int64_t small_tile = int64_t(rlpl::kThreads) * rlpl::kVecSmall;
    const int* cap = info->grid_cap[dtype][mode];
    const int64_t small_tiles = (slots + small_tile - 1) / small_tile;
    const int64_t large_tiles = (slots + large_tile - 1) / large_tile;
    if (slots < int64_t(info->cus) * rlpl::kSmallTilesPerCu * large_tile && small_tiles + 1 <= cap[rlpl::kShapeSmall]) {
        *out = {rlpl::kShapeSmall, rlpl::kVecSmall, uint32_t(small_tiles), small_tiles + 1, 1};
    } else if (large_tiles + 1 <= cap[rlpl::kShapeLarge]) {
        *out = {rlpl::kShapeLarge, rlpl::kVecLarge, uint32_t(large_tiles), large_tiles + 1, 1};
    } else {
        const int shape = nt_grad ? rlpl::kShapeStreamNt : rlpl::kShapeStream;
        const int64_t c = cap[shape];
        if (c < 1) return RLPL_ERR_DEVICE;
        const int64_t per = (large_tiles + c - 1) / c;
        if (mode == kModeGRPO && per > rlpl::kMaxPer) return RLPL_ERR_SHAPE;
        *out = {shape, rlpl::kVecLarge, uint32_t(large_tiles), (large_tiles + per - 1) / per, uint32_t(per)};
    }
    return RLPL_OK;
}

// Whether a fwd+bwd launch stores its gradient non-temporally: from
// kNtGradBytes of mask, planes and gradient on (whole arrays).
bool nt_grad(int mode, bool write_grad, bool has_kl, int64_t slots, int dtype) {
    if (!write_grad) return false;
    const int64_t planes = mode == kModeRKL ? 2 : (has_kl ? 3 : 2);
    const int64_t e = int64_t(elem_bytes(dtype));
    return slots * (1 + planes * e + e) >= rlpl::kNtGradBytes;
}

// Shared tail of every entry point: launch shape, row divisor and the launch.
int run(int mode, bool write_grad, bool has_kl, Args& a, int dtype, hipStream_t stream) {
    const DeviceInfo* info = nullptr;
    int st = current_device(&info);
    if (st != RLPL_OK) return st;
    Shape sh;
    st = launch_shape(info, dtype, mode, a.slots, nt_grad(mode, write_grad, has_kl, a.slots, dtype), &sh);
    if (st != RLPL_OK) return st;
    const void* kernel = rlpl::pick_kernel(dtype, mode, has_kl, write_grad, sh.kernel);
    if (!kernel) return RLPL_ERR_DTYPE;
    a.tiles = sh.tiles;
    a.per = sh.per;
    if (!rlpl::row_divisor(uint32_t(a.seq_len), &a.row_magic, &a.row_shift)) return RLPL_ERR_SHAPE;
    return launch(kernel, a, dim3(unsigned(sh.grid)), stream);
}

// Validates a policy-loss call (host only, nothing enqueued) and fills its kernel arguments.
int policy_args(bool write_grad, bool sign_aware, const void* policy_lp, const void* old_lp, const void* ref_lp,
                const void* advantages, const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype,
                float beta, float epsilon, float epsilon_high, float* loss_out, void* grad_out,
                uint32_t* n_valid_out, void* workspace, size_t workspace_bytes, Args* out) {
    int st = check_common(mask, bs, seq_len, dtype, mask_dtype, loss_out, n_valid_out, workspace,
                          workspace_bytes);
    if (st != RLPL_OK) return st;
    const bool has_kl = beta != 0.0f;
    if (!policy_lp || !old_lp || !advantages || (has_kl && !ref_lp) || (write_grad && !grad_out))
        return RLPL_ERR_NULL;
    if (!aligned(policy_lp, 16) || !aligned(old_lp, 16) || (has_kl && !aligned(ref_lp, 16)) ||
        (write_grad && !aligned(grad_out, 16)) || !aligned(advantages, elem_bytes(dtype)))
        return RLPL_ERR_ALIGN;
    if (!std::isfinite(beta) || !std::isfinite(epsilon) || !std::isfinite(epsilon_high))
        return RLPL_ERR_PARAM;
    const float lo = 1.0f - epsilon, hi = 1.0f + epsilon_high;
    if (!(lo <= hi)) return RLPL_ERR_PARAM;

    Args a{};
    a.lp = policy_lp;
    a.old = old_lp;
    a.ref = has_kl ? ref_lp : nullptr;
    a.adv = advantages;
    a.mask = static_cast<const uint8_t*>(mask);
    a.grad = write_grad ? grad_out : nullptr;
    a.loss = loss_out;
    a.n_out = n_valid_out;
    a.ws = static_cast<rlpl::Workspace*>(workspace);
    a.slots = bs * seq_len;
    a.seq_len = int32_t(seq_len);
    a.bs = int32_t(bs);
    a.beta = beta;
    a.lo = lo;
    a.hi = hi;
    a.sign_aware = sign_aware ? 1u : 0u;
    *out = a;
    return RLPL_OK;
}

int policy_loss(int mode, bool write_grad, bool sign_aware, const void* policy_lp, const void* old_lp,
                const void* ref_lp, const void* advantages, const void* mask, int64_t bs,
                int64_t seq_len, int dtype, int mask_dtype, float beta, float epsilon,
                float epsilon_high, float* loss_out, void* grad_out, uint32_t* n_valid_out,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Args a{};
    const int st = policy_args(write_grad, sign_aware, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                               dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, grad_out, n_valid_out,
                               workspace, workspace_bytes, &a);
    if (st != RLPL_OK) return st;
    return run(mode, write_grad, beta != 0.0f, a, dtype, stream);
}

int rkl_loss(bool write_grad, const void* student_lp, const void* teacher_lp, const void* mask,
             int64_t bs, int64_t seq_len, int dtype, int mask_dtype, float* loss_out,
             void* grad_out, uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
    int st = check_common(mask, bs, seq_len, dtype, mask_dtype, loss_out, n_valid_out, workspace,
                          workspace_bytes);
    if (st != RLPL_OK) return st;
    if (!student_lp || !teacher_lp || (write_grad && !grad_out)) return RLPL_ERR_NULL;
    if (!aligned(student_lp, 16) || !aligned(teacher_lp, 16) || (write_grad && !aligned(grad_out, 16)))
        return RLPL_ERR_ALIGN;
    Args a{};
    a.lp = student_lp;
    a.ref = teacher_lp;
    a.mask = static_cast<const uint8_t*>(mask);
    a.grad = write_grad ? grad_out : nullptr;
    a.loss = loss_out;
    a.n_out = n_valid_out;
    a.ws = static_cast<rlpl::Workspace*>(workspace);
    a.slots = bs * seq_len;
    a.seq_len = int32_t(seq_len);
    a.bs = int32_t(bs);
    a.beta = 1.0f;
    return run(kModeRKL, write_grad, true, a, dtype, stream);
}

// Full-vocab reverse KL: shape limits of the (rows, vocab) slabs.
bool vocab_shape_ok(int64_t rows, int64_t vocab) {
    return rows >= 1 && vocab >= 1 && rows < (int64_t(1) << 31) && vocab <= (int64_t(1) << 62) / rows;
}

int vocab_loss(bool write_grad, const void* student, const void* teacher, const void* mask,
               int64_t rows, int64_t vocab, int dtype, int mask_dtype, float* loss_out, void* grad_out,
               uint32_t* n_valid_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!student || !teacher || !mask || !loss_out || (write_grad && !grad_out)) return RLPL_ERR_NULL;
    if (!vocab_shape_ok(rows, vocab)) return RLPL_ERR_SHAPE;
    if (dtype != RLPL_F32 && dtype != RLPL_F16 && dtype != RLPL_BF16) return RLPL_ERR_DTYPE;
    if (mask_dtype != RLPL_MASK_BOOL && mask_dtype != RLPL_MASK_INT8) return RLPL_ERR_DTYPE;
    if (!aligned(student, 16) || !aligned(teacher, 16) || !aligned(mask, 16) ||
        (write_grad && !aligned(grad_out, 16)) || !aligned(loss_out, 4) ||
        (n_valid_out && !aligned(n_valid_out, 4)))
        return RLPL_ERR_ALIGN;
    if (!workspace || workspace_bytes < rlpl::kWorkspaceBytes) return RLPL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return RLPL_ERR_ALIGN;
    const DeviceInfo* info = nullptr;
    const int st = current_device(&info);
    if (st != RLPL_OK) return st;
    const int64_t cap = info->vocab_cap[dtype];
    if (cap < 1) return RLPL_ERR_DEVICE;
    // groups of `chunks` workgroups (one per piece of a row), sized to be co-resident.
    const rlpl::VocabSplit sp = rlpl::vocab_split(rows, vocab, int(elem_bytes(dtype)), cap, write_grad);
    rlpl::VocabArgs a{};
    a.student = student;
    a.teacher = teacher;
    a.mask = static_cast<const uint8_t*>(mask);
    a.grad = write_grad ? grad_out : nullptr;
    a.loss = loss_out;
    a.n_out = n_valid_out;
    a.ws = static_cast<rlpl::Workspace*>(workspace);
    a.rows = rows;
    a.vocab = vocab;
    a.chunks = uint32_t(sp.chunks);
    a.chunk_blocks = uint64_t(sp.chunk_blocks);
    const void* kernel = rlpl::pick_vocab_kernel(dtype, rlpl::vocab_mode(write_grad, sp.chunk_blocks));
    if (!kernel) return RLPL_ERR_DTYPE;
    return launch(kernel, a, dim3(unsigned(sp.groups * sp.chunks)), stream);
}

// ----------------------------------------------------------------------------- selective log-probs

constexpr int64_t kLpMaxVocab = int64_t(1) << 22;   // the kernels address a 256-row panel with 32-bit offsets
constexpr int64_t kLpMaxHidden = 65536;
constexpr int64_t kLpMaxTiles = int64_t(1) << 24;   // workgroups per launch (x 256 lanes < 2^32)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace carve-up of a selective log-prob call: per-tile (max, sum) partials
// and target logits of one group (forward), and the group's logits gradient
// (ld = vocab rounded up to 8), the split-K partial planes of the hidden
// gradient and the per-row-tile column sums of the logits gradient (backward).
struct LpLayout {
    int64_t chunk, tiles_n, tiles_m, ld_dz, k_split;
    size_t part, target, dz, split, col, total;
};

bool lp_shape_ok(int64_t n, int64_t h, int64_t vocab) {
    if (n < 1 || n >= (int64_t(1) << 31) || h < 8 || h > kLpMaxHidden || h % 8 != 0 || vocab < 1 ||
        vocab >= kLpMaxVocab)
        return false;
    const int64_t chunk = n < rlpl::kLogprobChunk ? n : rlpl::kLogprobChunk;
    const int64_t tn_v = ceil_div(vocab, rlpl::kGemmBN), tm_v = ceil_div(vocab, rlpl::kGemmBM);
    const int64_t t_h = ceil_div(h, rlpl::kGemmBN), t_c = ceil_div(chunk, rlpl::kGemmBM);
    return t_c * tn_v < kLpMaxTiles && tm_v * t_h < kLpMaxTiles && t_c * t_h < kLpMaxTiles;
}

LpLayout lp_layout(int64_t n, int64_t h, int64_t vocab, int backward) {
    LpLayout L{};
    L.chunk = n < rlpl::kLogprobChunk ? n : rlpl::kLogprobChunk;
    L.tiles_n = ceil_div(vocab, rlpl::kGemmBN);
    L.tiles_m = ceil_div(L.chunk, rlpl::kGemmBM);
    L.ld_dz = (vocab + 7) & ~int64_t(7);
    L.k_split = ceil_div(ceil_div(vocab, rlpl::kSplitK), rlpl::kGemmBK) * rlpl::kGemmBK;
    if (!backward) {
        L.part = round256(size_t(L.chunk) * size_t(L.tiles_n) * 2 * sizeof(float));
        L.target = round256(size_t(L.chunk) * sizeof(float));
    } else {
        L.dz = round256(size_t(L.chunk) * size_t(L.ld_dz) * 2);
        L.split = round256(size_t(rlpl::kSplitK) * size_t(L.chunk) * size_t(h) * sizeof(float));
        L.col = round256(size_t(L.tiles_m) * size_t(vocab) * sizeof(float));
    }
    L.total = L.part + L.target + L.dz + L.split + L.col;
    return L;
}

int lp_check(const void* hidden, const void* weight, const void* bias, const int64_t* targets, int64_t n,
             int64_t h, int64_t vocab, int dtype, const void* workspace, size_t workspace_bytes, int backward) {
    if (!hidden || !weight || !targets) return RLPL_ERR_NULL;
    if (!lp_shape_ok(n, h, vocab)) return RLPL_ERR_SHAPE;
    if (dtype != RLPL_F16 && dtype != RLPL_BF16) return RLPL_ERR_DTYPE;
    if (!aligned(hidden, 16) || !aligned(weight, 16) || (bias && !aligned(bias, 2)) || !aligned(targets, 8))
        return RLPL_ERR_ALIGN;
    if (!workspace || workspace_bytes < lp_layout(n, h, vocab, backward).total) return RLPL_ERR_WORKSPACE;
    return aligned(workspace, 256) ? RLPL_OK : RLPL_ERR_ALIGN;
}

int lp_device() {
    const DeviceInfo* info = nullptr;
    return current_device(&info);
}

rlpl::GemmArgs logits_gemm(const void* hidden, const void* weight, const void* bias, const int64_t* targets,
                           int64_t r0, int64_t m, int64_t h, int64_t vocab, size_t elem) {
    rlpl::GemmArgs g{};
    g.a = static_cast<const char*>(hidden) + size_t(r0) * size_t(h) * elem;
    g.b = weight;
    g.lda = h;
    g.ldb = h;
    g.M = int32_t(m);
    g.N = int32_t(vocab);
    g.K = int32_t(h);
    g.k_split = int32_t(h);
    g.tiles_m = uint32_t(ceil_div(m, rlpl::kGemmBM));
    g.tiles_n = uint32_t(ceil_div(vocab, rlpl::kGemmBN));
    g.bias = bias;
    g.targets = targets + r0;
    return g;
}

int launch_gemm(int dtype, int epi, bool ak, bool bk, const rlpl::GemmArgs& g, unsigned splits,
                hipStream_t stream) {
    const void* k = rlpl::pick_gemm_kernel(dtype, epi, ak, bk);
    if (!k) return RLPL_ERR_DTYPE;
    return launch(k, g, dim3(g.tiles_m * g.tiles_n, 1, splits), stream, rlpl::kGemmThreads, rlpl::kGemmDynLds);
}

// The library's scratch on the current device: its address is found once per
// device (hipGetSymbolAddress, in the file that defines it) and the scratch is
// zero-filled by a kernel enqueued on the first caller's stream, ahead of that
// caller's launch.  Nothing is allocated.
struct Scratch {
    std::once_flag once;
    void* ptr = nullptr;
    int status = RLPL_ERR_DEVICE;
};
Scratch g_scratch[kMaxDevices];

int scratch_on_current_device(void** out, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RLPL_ERR_DEVICE;
    Scratch& s = g_scratch[dev];
    std::call_once(s.once, [&s, stream] {
        void* p = nullptr;
        if (rlpl::scratch_address(&p) != 0 || !p) {
            (void)hipGetLastError();
            return;
        }
        void* words = p;
        uint32_t n = uint32_t(rlpl::kScratchBytes / 16);
        void* params[] = {&words, &n};
        if (hipLaunchKernel(rlpl::clear_kernel_ptr(), dim3(32), dim3(rlpl::kThreads), params, 0, stream) !=
            hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        s.ptr = p;
        s.status = RLPL_OK;
    });
    *out = s.ptr;
    return s.status;
}

}  // namespace

extern "C" {

size_t selective_logprob_workspace_bytes(int64_t n, int64_t hidden_size, int64_t vocab, int backward) {
    if (!lp_shape_ok(n, hidden_size, vocab)) return 0;
    return lp_layout(n, hidden_size, vocab, backward).total;
}

int selective_logprob_fwd(const void* hidden, const void* weight, const void* bias, const int64_t* targets,
                          int64_t n, int64_t hidden_size, int64_t vocab, int dtype, float* logp_out,
                          float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!logp_out) return RLPL_ERR_NULL;
    int st = lp_check(hidden, weight, bias, targets, n, hidden_size, vocab, dtype, workspace, workspace_bytes, 0);
    if (st != RLPL_OK) return st;
    if (!aligned(logp_out, 4) || (lse_out && !aligned(lse_out, 4))) return RLPL_ERR_ALIGN;
    if ((st = lp_device()) != RLPL_OK) return st;
    const LpLayout L = lp_layout(n, hidden_size, vocab, 0);
    char* ws = static_cast<char*>(workspace);
    float* part = reinterpret_cast<float*>(ws);
    float* target = reinterpret_cast<float*>(ws + L.part);
    const size_t elem = elem_bytes(dtype);
    for (int64_t r0 = 0; r0 < n; r0 += L.chunk) {
        const int64_t m = n - r0 < L.chunk ? n - r0 : L.chunk;
        rlpl::GemmArgs g = logits_gemm(hidden, weight, bias, targets, r0, m, hidden_size, vocab, elem);
        g.part = part;
        g.target_logit = target;
        st = launch_gemm(dtype, rlpl::kEpiLse, true, true, g, 1, stream);
        if (st != RLPL_OK) return st;
        rlpl::LseArgs a{};
        a.part = part;
        a.target_logit = target;
        a.targets = targets + r0;
        a.logp = logp_out + r0;
        a.lse = lse_out ? lse_out + r0 : nullptr;
        a.vocab = vocab;
        a.rows = int32_t(m);
        a.tiles = int32_t(L.tiles_n);
        st = launch(rlpl::lse_combine_kernel(), a, dim3(unsigned(m)), stream);
        if (st != RLPL_OK) return st;
    }
    return RLPL_OK;
}

int selective_logprob_bwd(const void* hidden, const void* weight, const void* bias, const int64_t* targets,
                          const float* lse, const float* grad_logp, int64_t n, int64_t hidden_size,
                          int64_t vocab, int dtype, void* grad_hidden, float* grad_weight, float* grad_bias,
                          int accumulate, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!lse || !grad_logp) return RLPL_ERR_NULL;
    int st = lp_check(hidden, weight, bias, targets, n, hidden_size, vocab, dtype, workspace, workspace_bytes, 1);
    if (st != RLPL_OK) return st;
    if (!aligned(lse, 4) || !aligned(grad_logp, 4) || (grad_hidden && !aligned(grad_hidden, 4)) ||
        (grad_weight && !aligned(grad_weight, 4)) || (grad_bias && !aligned(grad_bias, 4)))
        return RLPL_ERR_ALIGN;
    if ((st = lp_device()) != RLPL_OK) return st;
    const LpLayout L = lp_layout(n, hidden_size, vocab, 1);
    char* ws = static_cast<char*>(workspace);
    void* dz = ws;
    float* split = reinterpret_cast<float*>(ws + L.dz);
    float* col_part = reinterpret_cast<float*>(ws + L.dz + L.split);
    const size_t elem = elem_bytes(dtype);
    for (int64_t r0 = 0; r0 < n; r0 += L.chunk) {
        const int64_t m = n - r0 < L.chunk ? n - r0 : L.chunk;
        const int acc = (accumulate || r0 > 0) ? 1 : 0;
        const void* h0 = static_cast<const char*>(hidden) + size_t(r0) * size_t(hidden_size) * elem;
        // dz = g (onehot - softmax(z)) for the group's rows.
        rlpl::GemmArgs g = logits_gemm(hidden, weight, bias, targets, r0, m, hidden_size, vocab, elem);
        g.c = dz;
        g.ldc = L.ld_dz;
        g.lse = lse + r0;
        g.grad = grad_logp + r0;
        g.col_part = grad_bias ? col_part : nullptr;
        st = launch_gemm(dtype, rlpl::kEpiDlogits, true, true, g, 1, stream);
        if (st != RLPL_OK) return st;
        if (grad_hidden) {
            // (m x vocab) . (vocab x hidden): split over vocab into fp32 planes, summed in split order.
            rlpl::GemmArgs d{};
            d.a = dz;
            d.b = weight;
            d.lda = L.ld_dz;
            d.ldb = hidden_size;
            d.M = int32_t(m);
            d.N = int32_t(hidden_size);
            d.K = int32_t(vocab);
            d.k_split = int32_t(L.k_split);
            d.tiles_m = uint32_t(ceil_div(m, rlpl::kGemmBM));
            d.tiles_n = uint32_t(ceil_div(hidden_size, rlpl::kGemmBN));
            d.c = split;
            d.ldc = hidden_size;
            st = launch_gemm(dtype, rlpl::kEpiSplit, true, false, d, rlpl::kSplitK, stream);
            if (st != RLPL_OK) return st;
            rlpl::SplitSumArgs s{};
            s.part = split;
            s.out = static_cast<char*>(grad_hidden) + size_t(r0) * size_t(hidden_size) * elem;
            s.plane = m * hidden_size;
            s.splits = rlpl::kSplitK;
            const int64_t blocks = ceil_div(s.plane, rlpl::kThreads);
            st = launch(rlpl::pick_split_sum_kernel(dtype), s, dim3(unsigned(blocks < 8192 ? blocks : 8192)), stream);
            if (st != RLPL_OK) return st;
        }
        if (grad_weight) {
            // (vocab x m) . (m x hidden), accumulated in fp32 over the groups.
            rlpl::GemmArgs w{};
            w.a = dz;
            w.b = h0;
            w.lda = L.ld_dz;
            w.ldb = hidden_size;
            w.M = int32_t(vocab);
            w.N = int32_t(hidden_size);
            w.K = int32_t(m);
            w.k_split = int32_t(m);
            w.tiles_m = uint32_t(ceil_div(vocab, rlpl::kGemmBM));
            w.tiles_n = uint32_t(ceil_div(hidden_size, rlpl::kGemmBN));
            w.c = grad_weight;
            w.ldc = hidden_size;
            w.accumulate = acc;
            st = launch_gemm(dtype, rlpl::kEpiAccum, false, false, w, 1, stream);
            if (st != RLPL_OK) return st;
        }
        if (grad_bias) {
            // the row tiles' column sums of dz, added in row-tile order
            rlpl::ColSumArgs c{};
            c.x = col_part;
            c.out = grad_bias;
            c.rows = int32_t(ceil_div(m, rlpl::kGemmBM));
            c.cols = int32_t(vocab);
            c.accumulate = acc;
            st = launch(rlpl::col_sum_kernel(), c, dim3(unsigned(ceil_div(vocab, rlpl::kThreads))), stream);
            if (st != RLPL_OK) return st;
        }
    }
    return RLPL_OK;
}



int reverse_kl_logits(const void* student_logits, const void* teacher_logits, const void* mask,
                      int64_t rows, int64_t vocab, int dtype, int mask_dtype, float* loss_out,
                      void* grad_out, uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    return vocab_loss(true, student_logits, teacher_logits, mask, rows, vocab, dtype, mask_dtype,
                      loss_out, grad_out, n_valid_out, workspace, workspace_bytes, stream);
}

int reverse_kl_logits_fwd(const void* student_logits, const void* teacher_logits, const void* mask,
                          int64_t rows, int64_t vocab, int dtype, int mask_dtype, float* loss_out,
                          uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return vocab_loss(false, student_logits, teacher_logits, mask, rows, vocab, dtype, mask_dtype,
                      loss_out, nullptr, n_valid_out, workspace, workspace_bytes, stream);
}

int bnpo_loss(const void* policy_lp, const void* old_lp, const void* ref_lp, const void* advantages,
              const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype, float beta,
              float epsilon, float epsilon_high, float* loss_out, void* grad_out,
              uint32_t* n_valid_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return policy_loss(kModeBNPO, true, false, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                       dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, grad_out,
                       n_valid_out, workspace, workspace_bytes, stream);
}

int bnpo_loss_noalloc(const void* policy_lp, const void* old_lp, const void* ref_lp, const void* advantages,
                      const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype, float beta,
                      float epsilon, float epsilon_high, float* loss_out, void* grad_out,
                      uint32_t* n_valid_out, hipStream_t stream) {
    // Validate first (the scratch stands in as an aligned placeholder), so that a
    // rejected call enqueues nothing; then the scratch of the current device.
    alignas(256) static const unsigned char placeholder[256] = {};
    Args a{};
    int st = policy_args(true, false, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len, dtype, mask_dtype,
                         beta, epsilon, epsilon_high, loss_out, grad_out, n_valid_out,
                         const_cast<unsigned char*>(placeholder), rlpl::kScratchBytes, &a);
    if (st != RLPL_OK) return st;
    const DeviceInfo* info = nullptr;
    if ((st = current_device(&info)) != RLPL_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws, stream)) != RLPL_OK) return st;
    a.ws = static_cast<rlpl::Workspace*>(ws);
    return run(kModeBNPO, true, beta != 0.0f, a, dtype, stream);
}

int bnpo_loss_fwd(const void* policy_lp, const void* old_lp, const void* ref_lp,
                  const void* advantages, const void* mask, int64_t bs, int64_t seq_len, int dtype,
                  int mask_dtype, float beta, float epsilon, float epsilon_high, float* loss_out,
                  uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    return policy_loss(kModeBNPO, false, false, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                       dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, nullptr,
                       n_valid_out, workspace, workspace_bytes, stream);
}

int grpo_loss(const void* policy_lp, const void* old_lp, const void* ref_lp, const void* advantages,
              const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype, float beta,
              float epsilon, float epsilon_high, float* loss_out, void* grad_out,
              uint32_t* n_valid_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return policy_loss(kModeGRPO, true, false, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                       dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, grad_out,
                       n_valid_out, workspace, workspace_bytes, stream);
}

int grpo_loss_fwd(const void* policy_lp, const void* old_lp, const void* ref_lp,
                  const void* advantages, const void* mask, int64_t bs, int64_t seq_len, int dtype,
                  int mask_dtype, float beta, float epsilon, float epsilon_high, float* loss_out,
                  uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    return policy_loss(kModeGRPO, false, false, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                       dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, nullptr,
                       n_valid_out, workspace, workspace_bytes, stream);
}

int rlpl_policy_loss(int op, uint32_t flags, const void* policy_lp, const void* old_lp,
                     const void* ref_lp, const void* advantages, const void* mask, int64_t bs,
                     int64_t seq_len, int dtype, int mask_dtype, float beta, float epsilon,
                     float epsilon_high, float* loss_out, void* grad_out, uint32_t* n_valid_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if ((flags & ~uint32_t(RLPL_CLIP_SIGN_AWARE)) != 0u) return RLPL_ERR_PARAM;
    const bool sign_aware = (flags & RLPL_CLIP_SIGN_AWARE) != 0u;
    int mode;
    bool fused;
    switch (op) {
    case RLPL_OP_BNPO: mode = kModeBNPO; fused = true; break;
    case RLPL_OP_BNPO_FWD: mode = kModeBNPO; fused = false; break;
    case RLPL_OP_GRPO: mode = kModeGRPO; fused = true; break;
    case RLPL_OP_GRPO_FWD: mode = kModeGRPO; fused = false; break;
    default: return RLPL_ERR_PARAM;
    }
    return policy_loss(mode, fused, sign_aware, policy_lp, old_lp, ref_lp, advantages, mask, bs, seq_len,
                       dtype, mask_dtype, beta, epsilon, epsilon_high, loss_out, fused ? grad_out : nullptr,
                       n_valid_out, workspace, workspace_bytes, stream);
}

int reverse_kl(const void* student_lp, const void* teacher_lp, const void* mask, int64_t bs,
               int64_t seq_len, int dtype, int mask_dtype, float* loss_out, void* grad_out,
               uint32_t* n_valid_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return rkl_loss(true, student_lp, teacher_lp, mask, bs, seq_len, dtype, mask_dtype, loss_out,
                    grad_out, n_valid_out, workspace, workspace_bytes, stream);
}

int reverse_kl_fwd(const void* student_lp, const void* teacher_lp, const void* mask, int64_t bs,
                   int64_t seq_len, int dtype, int mask_dtype, float* loss_out,
                   uint32_t* n_valid_out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    return rkl_loss(false, student_lp, teacher_lp, mask, bs, seq_len, dtype, mask_dtype, loss_out,
                    nullptr, n_valid_out, workspace, workspace_bytes, stream);
}

size_t rlpl_workspace_bytes(int64_t bs, int64_t seq_len, int op) {
    (void)bs;
    (void)seq_len;
    if (op < RLPL_OP_BNPO || op > RLPL_OP_RKL_LOGITS_FWD) return 0;
    return rlpl::kWorkspaceBytes;
}

int rlpl_launch_shape(int64_t bs, int64_t seq_len, int dtype, int op, int* grid_out, int* vec_out,
                      int* tiles_out) {
    if (!grid_out || !vec_out || !tiles_out) return RLPL_ERR_NULL;
    if (dtype != RLPL_F32 && dtype != RLPL_F16 && dtype != RLPL_BF16) return RLPL_ERR_DTYPE;
    if (op == RLPL_OP_RKL_LOGITS || op == RLPL_OP_RKL_LOGITS_FWD) {
        if (!vocab_shape_ok(bs, seq_len)) return RLPL_ERR_SHAPE;
        const DeviceInfo* info = nullptr;
        const int st = current_device(&info);
        if (st != RLPL_OK) return st;
        const int64_t cap = info->vocab_cap[dtype];
        if (cap < 1) return RLPL_ERR_DEVICE;
        const rlpl::VocabSplit sp =
            rlpl::vocab_split(bs, seq_len, int(elem_bytes(dtype)), cap, op == RLPL_OP_RKL_LOGITS);
        *grid_out = int(sp.groups * sp.chunks);
        *vec_out = int(32 / elem_bytes(dtype));
        *tiles_out = int(bs * sp.chunks > INT32_MAX ? INT32_MAX : bs * sp.chunks);
        return RLPL_OK;
    }
    if (bs < 1 || seq_len < 1 || bs > (int64_t(1) << 31) / seq_len || bs * seq_len >= (int64_t(1) << 31))
        return RLPL_ERR_SHAPE;
    int mode;
    switch (op) {
    case RLPL_OP_BNPO: case RLPL_OP_BNPO_FWD: mode = kModeBNPO; break;
    case RLPL_OP_GRPO: case RLPL_OP_GRPO_FWD: mode = kModeGRPO; break;
    case RLPL_OP_RKL: case RLPL_OP_RKL_FWD: mode = kModeRKL; break;
    default: return RLPL_ERR_PARAM;
    }
    const DeviceInfo* info = nullptr;
    int st = current_device(&info);
    if (st != RLPL_OK) return st;
    Shape sh;
    const bool fused = op == RLPL_OP_BNPO || op == RLPL_OP_GRPO || op == RLPL_OP_RKL;
    st = launch_shape(info, dtype, mode, bs * seq_len, nt_grad(mode, fused, true, bs * seq_len, dtype), &sh);
    if (st != RLPL_OK) return st;
    *grid_out = int(sh.grid);
    *vec_out = sh.vec;
    *tiles_out = int(sh.tiles);
    return RLPL_OK;
}

int rlpl_workspace_flags(const void* workspace, uint32_t* flags_out, hipStream_t stream) {
    if (!workspace || !flags_out) return RLPL_ERR_NULL;
    if (!aligned(workspace, 256)) return RLPL_ERR_ALIGN;
    const auto* src = static_cast<const unsigned char*>(workspace) + rlpl::kFlagsOffset;
    if (hipMemcpyAsync(flags_out, src, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return RLPL_ERR_LAUNCH;
    return RLPL_OK;
}

int rlpl_workspace_set_limits(void* workspace, uint32_t steal_ticks, uint32_t release_ticks,
                              uint32_t giveup_ticks, hipStream_t stream) {
    if (!workspace) return RLPL_ERR_NULL;
    if (!aligned(workspace, 256)) return RLPL_ERR_ALIGN;
    auto* w = static_cast<unsigned char*>(workspace) + rlpl::kLimitsOffset;
    const uint32_t v[3] = {steal_ticks, release_ticks, giveup_ticks};
    for (int i = 0; i < 3; ++i)
        if (hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(w + 4 * i), int(v[i]), 1, stream) != hipSuccess) {
            (void)hipGetLastError();
            return RLPL_ERR_LAUNCH;
        }
    return RLPL_OK;
}

const char* rlpl_status_string(int status) {
    switch (status) {
    case RLPL_OK: return "RLPL_OK";
    case RLPL_ERR_NULL: return "RLPL_ERR_NULL: a required pointer is NULL";
    case RLPL_ERR_SHAPE: return "RLPL_ERR_SHAPE: need bs >= 1, seq_len >= 1, bs*seq_len < 2^31";
    case RLPL_ERR_ALIGN: return "RLPL_ERR_ALIGN: a pointer breaks the alignment contract";
    case RLPL_ERR_DTYPE: return "RLPL_ERR_DTYPE: unknown dtype or mask dtype";
    case RLPL_ERR_PARAM: return "RLPL_ERR_PARAM: non-finite parameter or 1-epsilon > 1+epsilon_high";
    case RLPL_ERR_WORKSPACE: return "RLPL_ERR_WORKSPACE: workspace missing or too small";
    case RLPL_ERR_DEVICE: return "RLPL_ERR_DEVICE: no usable gfx950 device is current";
    case RLPL_ERR_LAUNCH: return "RLPL_ERR_LAUNCH: the kernel launch failed";
    }
    return "unknown rlpl status";
}

int rlpl_version(void) { return kAbiVersion; }

}  // extern "C"
