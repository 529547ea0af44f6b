/*
 * rl_post_loss: fused forward+backward PPO-family policy losses on AMD
 * Instinct MI355X (gfx950).
 *
 * One call = one kernel launch on the caller's stream that returns the scalar
 * loss and, for the fused forward+backward entry points, the gradient of the
 * loss with respect to the policy (student) log-probs, with no host
 * synchronisation.  The operations are defined on the model card
 * "Geometric-AI Kernels" (Hugging Face, Geometric-AI/geometric-ai-kernels),
 * sections "BNPO Loss", "GRPO Loss" and "Reverse KL".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are device pointers (hipMalloc'd or torch CUDA-tensor storage)
 * unless stated otherwise.  The caller allocates and owns every buffer; the
 * library never allocates or frees device memory.
 *
 * Layouts: log-prob planes and the mask are dense row-major (bs, seq_len) with
 * no strides; `advantages` is dense (bs,).  The planes, the mask and grad_out
 * must be 16-byte aligned (every kernel streams them with 128-bit accesses);
 * advantages needs only element alignment, loss_out and n_valid_out 4-byte
 * alignment.
 *
 * dtype (RLPL_F32 / RLPL_F16 / RLPL_BF16) applies to the log-prob planes, the
 * advantages and grad_out.  mask_dtype (RLPL_MASK_BOOL / RLPL_MASK_INT8) is one
 * byte per slot; any nonzero byte marks a valid (completion) token.  Masked
 * slots contribute nothing, get a +0 gradient and their log-probs are never
 * read.  All arithmetic is float32 in registers; the loss is always written as
 * one float32 (device memory); grad_out is written in `dtype`, rounded to
 * nearest even, for every slot (masked slots included).
 *
 * Workspace: `workspace` is device memory of at least
 * rlpl_workspace_bytes(bs, seq_len, op) bytes, 256-byte aligned, zero-filled
 * once by the caller before its first use.  Every call leaves it in the state
 * the next call needs, so it is re-used as is.  Only one call may be in flight
 * per workspace (calls on one stream are serialised and may share one).
 * Calls on other streams or workspaces may run concurrently.
 *
 * The per-token losses form their global count without host synchronisation:
 * workgroups publish values in the workspace tagged with their launch's
 * identity (its dispatch id on its hardware queue), and a coordinating
 * workgroup combines them.  No workgroup relies on any other being resident:
 * a value not published within a time limit is computed by the waiting
 * workgroup itself, with the same arithmetic, so results are bit-identical
 * however the launch was scheduled (for instance beside other kernels that
 * hold compute units).  Bytes 256..267 of the workspace hold optional limits
 * for these waits (rlpl_workspace_set_limits); zero selects the defaults.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a
 * rejected call enqueues nothing and returns a nonzero rlpl_status.  A failed
 * launch returns RLPL_ERR_LAUNCH.  RLPL_OK means the launch was enqueued; the
 * call does not synchronise, so device faults surface at the caller's next
 * synchronisation.  Results of an enqueued call are valid once the stream has
 * reached it.  Inputs must be finite (masked slots excepted).
 *
 * The functions are thread-safe; the first call on a device queries and caches
 * that device's compute-unit count and kernel occupancies.
 */
#ifndef RL_POST_LOSS_H
#define RL_POST_LOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, as hip_runtime_api.h declares it. */
typedef struct ihipStream_t* hipStream_t;

enum rlpl_dtype { RLPL_F32 = 0, RLPL_F16 = 1, RLPL_BF16 = 2 };
enum rlpl_mask_dtype { RLPL_MASK_BOOL = 0, RLPL_MASK_INT8 = 1 };

/* Operation selector for rlpl_workspace_bytes and rlpl_launch_shape. */
enum rlpl_op {
    RLPL_OP_BNPO = 0, RLPL_OP_BNPO_FWD = 1, RLPL_OP_GRPO = 2, RLPL_OP_GRPO_FWD = 3,
    RLPL_OP_RKL = 4, RLPL_OP_RKL_FWD = 5, RLPL_OP_RKL_LOGITS = 6, RLPL_OP_RKL_LOGITS_FWD = 7
};

enum rlpl_status {
    RLPL_OK = 0,
    RLPL_ERR_NULL = 1,       /* a required pointer is NULL                                 */
    RLPL_ERR_SHAPE = 2,      /* bs < 1, seq_len < 1, or bs*seq_len >= 2^31 (for the logit    */
                             /* slabs: rows < 1, vocab < 1, rows >= 2^31 or rows*vocab > 2^62)*/
    RLPL_ERR_ALIGN = 3,      /* a plane, mask or grad pointer is not 16-byte aligned, or     */
                             /* advantages / loss / counts / workspace misaligned            */
    RLPL_ERR_DTYPE = 4,      /* unknown dtype or mask_dtype                                  */
    RLPL_ERR_PARAM = 5,      /* non-finite beta/epsilon/epsilon_high, or 1-eps > 1+eps_high  */
    RLPL_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than rlpl_workspace_bytes          */
    RLPL_ERR_DEVICE = 7,     /* no current HIP device, or it is not gfx950-capable           */
    RLPL_ERR_LAUNCH = 8      /* the kernel launch failed                                     */
};

/*
 * BNPO, fused forward + backward (model card, "BNPO Loss").
 *
 *   ratio     = exp(policy_lp - old_lp)
 *   clipped   = clip(ratio, 1 - epsilon, 1 + epsilon_high)
 *   per_token = -advantages[row] * min(ratio, clipped)
 *   kl        = exp(ref_lp - policy_lp) - (ref_lp - policy_lp) - 1
 *   loss      = sum((per_token + beta * kl) * mask) / max(sum(mask), 1)
 *
 * The global valid-token count sum(mask) is formed on the GPU in the same
 * launch (no host round trip).  grad_out[i] = d loss / d policy_lp[i]; where
 * ratio equals its clipped value the unclipped branch is taken, so the
 * policy part of the gradient is -A*ratio/N unless clipping lowered ratio to
 * 1+epsilon_high (then 0).  With beta == 0.0f the KL term is compiled out and
 * ref_lp is never read (it may be NULL).
 *
 * policy_lp, old_lp, ref_lp : (bs, seq_len) `dtype`, 16-byte aligned
 * advantages                : (bs,) `dtype`
 * mask                      : (bs, seq_len) bytes, 16-byte aligned
 * loss_out                  : 1 float (written)
 * grad_out                  : (bs, seq_len) `dtype`, 16-byte aligned (written, every slot)
 * n_valid_out               : 1 uint32 = sum(mask != 0) (written), or NULL
 */
int bnpo_loss(const void* policy_lp, const void* old_lp, const void* ref_lp,
              const void* advantages, const void* mask, int64_t bs, int64_t seq_len,
              int dtype, int mask_dtype, float beta, float epsilon, float epsilon_high,
              float* loss_out, void* grad_out, uint32_t* n_valid_out,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* BNPO, forward only: the same loss as bnpo_loss (bit-identical for the same
 * inputs on the same device), no gradient buffer. */
int bnpo_loss_fwd(const void* policy_lp, const void* old_lp, const void* ref_lp,
                  const void* advantages, const void* mask, int64_t bs, int64_t seq_len,
                  int dtype, int mask_dtype, float beta, float epsilon, float epsilon_high,
                  float* loss_out, uint32_t* n_valid_out,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * GRPO, fused forward + backward (model card, "GRPO Loss"): the per-token
 * terms of bnpo_loss, normalised per response and averaged over the batch:
 *
 *   loss = (1/bs) * sum_r [ sum_t((per_token + beta*kl) * mask) / max(sum_t(mask), 1) ]
 *
 * All bs rows count in the mean; a fully masked row adds 0.  Each row's count
 * is reduced inside the workgroups that touch the row (no cross-workgroup
 * exchange before the gradient is scaled).  n_valid_out, if not NULL, receives
 * bs uint32 per-row counts.  Arguments as for bnpo_loss.
 */
int grpo_loss(const void* policy_lp, const void* old_lp, const void* ref_lp,
              const void* advantages, const void* mask, int64_t bs, int64_t seq_len,
              int dtype, int mask_dtype, float beta, float epsilon, float epsilon_high,
              float* loss_out, void* grad_out, uint32_t* n_valid_out,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* GRPO, forward only: the same loss as grpo_loss (bit-identical), no gradient. */
int grpo_loss_fwd(const void* policy_lp, const void* old_lp, const void* ref_lp,
                  const void* advantages, const void* mask, int64_t bs, int64_t seq_len,
                  int dtype, int mask_dtype, float beta, float epsilon, float epsilon_high,
                  float* loss_out, uint32_t* n_valid_out,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Flags of rlpl_policy_loss. */
enum rlpl_flags {
    RLPL_CLIP_SIGN_AWARE = 1   /* per_token = -min(A*ratio, A*clipped) (see below) */
};

/*
 * The policy losses with options (model card, "BNPO Loss" and "GRPO Loss").
 * op is RLPL_OP_BNPO, RLPL_OP_BNPO_FWD, RLPL_OP_GRPO or RLPL_OP_GRPO_FWD;
 * flags 0 gives exactly the corresponding entry point above (grad_out is
 * ignored, and may be NULL, for the _FWD ops).
 *
 * RLPL_CLIP_SIGN_AWARE replaces the card's literal per_token
 * -A*min(ratio, clipped) by the standard PPO clipped objective that the card
 * calls "PPO-clipped":
 *
 *   per_token = -min(A*ratio, A*clip(ratio, 1 - epsilon, 1 + epsilon_high))
 *
 * which is the same where A >= 0 and -A*max(ratio, 1 - epsilon) where A < 0
 * (so epsilon matters).  Where the two objectives tie, the unclipped branch
 * is taken: the policy part of the gradient is -A*ratio on the unclipped
 * branch and 0 on the clipped one.  Unknown flag bits give RLPL_ERR_PARAM;
 * every other argument is as for bnpo_loss / grpo_loss.
 */
int rlpl_policy_loss(int op, uint32_t flags, const void* policy_lp, const void* old_lp,
                     const void* ref_lp, const void* advantages, const void* mask, int64_t bs,
                     int64_t seq_len, int dtype, int mask_dtype, float beta, float epsilon,
                     float epsilon_high, float* loss_out, void* grad_out, uint32_t* n_valid_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Reverse KL(student || teacher) self-distillation on per-token log-probs
 * (model card, "Reverse KL": global token mean with the unclamped
 * inv_n_valid = 1/sum(mask), gradient scaled by mask[r]*inv_n_valid), using
 * the card's per-token KL estimator with x = teacher_lp - student_lp:
 *
 *   loss = sum(mask * (exp(x) - x - 1)) / sum(mask)
 *   grad_out[i] = mask[i] ? (1 - exp(x_i)) / sum(mask) : +0
 *
 * A batch with no valid token gives loss = NaN (0/0, as on the card) and an
 * all +0 gradient; it is not an error.  student_lp, teacher_lp: (bs, seq_len)
 * `dtype`, 16-byte aligned; the rest as for bnpo_loss.
 */
int reverse_kl(const void* student_lp, const void* teacher_lp, const void* mask,
               int64_t bs, int64_t seq_len, int dtype, int mask_dtype,
               float* loss_out, void* grad_out, uint32_t* n_valid_out,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Reverse KL, forward only: the same loss as reverse_kl (bit-identical), no gradient. */
int reverse_kl_fwd(const void* student_lp, const void* teacher_lp, const void* mask,
                   int64_t bs, int64_t seq_len, int dtype, int mask_dtype,
                   float* loss_out, uint32_t* n_valid_out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Reverse KL over full logit rows, fused forward + backward (model card,
 * "Reverse KL"): for each row r of the (rows, vocab) slabs,
 *
 *   p = softmax(student_logits[r]),  q = softmax(teacher_logits[r])
 *   kl_r = sum_v p_v (log p_v - log q_v)
 *   loss = sum_r mask[r] kl_r / N,  N = number of rows with a nonzero mask byte
 *   grad_out[r][v] = mask[r] ? p_v (log p_v - log q_v - kl_r) / N : +0
 *
 * N is not clamped (as on the card): with no valid row the loss is NaN and
 * the gradient all +0; that is not an error.  Rows whose mask byte is zero are
 * never read.  A valid row is split among workgroups in pieces of about
 * 32 KB per slab, which exchange their softmax sums through the workspace;
 * each holds its piece in registers until the row's sums are known, so the
 * row is read once.  (Rows of more than 256 such pieces, above about 4.2 M
 * 16-bit or 2.1 M fp32 logits, are read twice.)
 *
 * student_logits, teacher_logits : (rows, vocab) `dtype`, dense row-major,
 *                                  16-byte aligned (rows themselves need not
 *                                  start on a 16-byte boundary); finite
 * mask        : (rows,) bytes (the card's completions_mask over the leading
 *               dims of the logits, flattened), 16-byte aligned
 * loss_out    : 1 float (written)
 * grad_out    : (rows, vocab) `dtype`, 16-byte aligned (written, every element)
 * n_valid_out : 1 uint32 = N (written), or NULL
 * workspace   : as for bnpo_loss
 */
int reverse_kl_logits(const void* student_logits, const void* teacher_logits, const void* mask,
                      int64_t rows, int64_t vocab, int dtype, int mask_dtype,
                      float* loss_out, void* grad_out, uint32_t* n_valid_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Reverse KL over full logit rows, forward only: the same loss as
 * reverse_kl_logits, one read of each valid row, no gradient.  The two losses
 * are bit-identical when both split the rows alike (when rows times the
 * pieces per row fit in the device's co-resident workgroups); otherwise they
 * agree to float32 summation rounding. */
int reverse_kl_logits_fwd(const void* student_logits, const void* teacher_logits, const void* mask,
                          int64_t rows, int64_t vocab, int dtype, int mask_dtype,
                          float* loss_out, uint32_t* n_valid_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Selective log-probabilities: the producer of the policy log-probs above
 * (page "Add SM100 CuTe DSL GRPO fast path", section "Summary": the logits of
 * a group of up to 1024 tokens come from one matrix multiplication, the
 * cross-entropy is taken in place and the full logits are never kept; the
 * weight gradient is accumulated in float32 across groups).  For token i,
 *
 *   z_i      = hidden[i] . weight^T + bias          (vocab logits, temperature 1)
 *   lse_i    = log sum_v exp(z_i[v])
 *   logp_i   = z_i[targets[i]] - lse_i
 *
 * and, for an upstream gradient g_i = d L / d logp_i, the gradients of L:
 *
 *   dz_i[v]         = g_i ((v == targets[i]) - exp(z_i[v] - lse_i))
 *   grad_hidden[i]  = sum_v dz_i[v] weight[v]
 *   grad_weight[v]  = sum_i dz_i[v] hidden[i]
 *   grad_bias[v]    = sum_i dz_i[v]
 *
 * The matrix products run on the matrix cores with `dtype` operands (RLPL_F16
 * or RLPL_BF16 only) and float32 accumulation.  The forward keeps per token
 * only lse and logp; the backward recomputes z in groups of 1024 tokens and
 * forms dz in `dtype` (rounded to nearest even) in the workspace, the operand
 * of its two gradient products.  Each call enqueues several kernels on
 * `stream` (no host synchronisation, no allocation); results are
 * deterministic (fixed reduction orders, no atomics).
 *
 * hidden      : (n, hidden_size) `dtype`, dense row-major, 16-byte aligned
 * weight      : (vocab, hidden_size) `dtype`, dense row-major, 16-byte aligned
 * bias        : (vocab,) `dtype`, or NULL (no bias)
 * targets     : (n,) int64 token ids, 8-byte aligned; a target outside
 *               [0, vocab) gives logp = NaN (forward) and no one-hot term in dz
 * lse_out     : (n,) float32, written (may be NULL in the forward); the
 *               backward reads the forward's lse through `lse`
 * logp_out    : (n,) float32, written
 * grad_logp   : (n,) float32 upstream gradient g
 * grad_hidden : (n, hidden_size) `dtype` written, or NULL (not wanted)
 * grad_weight : (vocab, hidden_size) float32, or NULL; accumulate != 0 adds
 *               to its contents, else overwrites them
 * grad_bias   : (vocab,) float32, or NULL; accumulate as for grad_weight
 * workspace   : device memory of at least
 *               selective_logprob_workspace_bytes(n, hidden_size, vocab,
 *               backward) bytes, 256-byte aligned, no initial contents needed;
 *               one call in flight per workspace
 *
 * Shapes: 1 <= n < 2^31, hidden_size a multiple of 8 in [8, 65536],
 * 1 <= vocab < 2^22; otherwise RLPL_ERR_SHAPE.  Pointers 4-byte aligned
 * where not stated.  Errors as for the other entry points.
 */
size_t selective_logprob_workspace_bytes(int64_t n, int64_t hidden_size, int64_t vocab, int backward);

int selective_logprob_fwd(const void* hidden, const void* weight, const void* bias, const int64_t* targets,
                          int64_t n, int64_t hidden_size, int64_t vocab, int dtype,
                          float* logp_out, float* lse_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

int selective_logprob_bwd(const void* hidden, const void* weight, const void* bias, const int64_t* targets,
                          const float* lse, const float* grad_logp,
                          int64_t n, int64_t hidden_size, int64_t vocab, int dtype,
                          void* grad_hidden, float* grad_weight, float* grad_bias, int accumulate,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* bnpo_loss for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels,
 * results bit-identical to bnpo_loss, with no workspace argument.  The
 * exchange entries live in the library's own scratch, a static device array
 * of 328,192 bytes per GPU, held until the process ends; this entry point
 * never calls hipMalloc, hipFree or an allocating routine.  Its first call on
 * a device finds the scratch's address and enqueues a kernel on `stream` that
 * zero-fills it.  Every bnpo_loss_noalloc call on a GPU shares that GPU's
 * scratch: calls that overlap on one GPU (on different streams) race and
 * must not be made.  Limits: those of bnpo_loss (bs * seq_len < 2^31); the
 * scratch holds the entries of every grid these kernels launch, so no problem
 * size that bnpo_loss accepts is refused for lack of space.  Returns
 * RLPL_ERR_DEVICE when the scratch cannot be set up. */
int bnpo_loss_noalloc(const void* policy_lp, const void* old_lp, const void* ref_lp, const void* advantages,
                      const void* mask, int64_t bs, int64_t seq_len, int dtype, int mask_dtype, float beta,
                      float epsilon, float epsilon_high, float* loss_out, void* grad_out,
                      uint32_t* n_valid_out, hipStream_t stream);

/* Bytes of workspace an `op` call on a (bs, seq_len) problem needs (0 for a bad op). */
size_t rlpl_workspace_bytes(int64_t bs, int64_t seq_len, int op);

/* Launch shape a call of `op` on a (bs, seq_len) problem of `dtype` would use
 * on the current device (host pointers, written): workgroups in the grid (one
 * coordinator plus one worker per tile when tiles < grid; else every
 * workgroup strides over the tiles), consecutive slots per lane (4 or 16) and
 * tiles of 256 lanes.  For the logit-slab ops, bs and seq_len are rows and
 * vocab, tiles are rows, and the lane width is elements per 32-byte step.  For
 * profiling and tests; enqueues nothing.  Returns RLPL_OK, or an rlpl_status
 * for bad arguments or no usable device. */
int rlpl_launch_shape(int64_t bs, int64_t seq_len, int dtype, int op, int* grid_out, int* vec_out,
                      int* tiles_out);

/* Sticky error bits the kernels left in a workspace (host pointer `flags_out`
 * receives them; synchronises `stream`).  Bit 0: workgroup 0 of a full-vocab
 * reverse-KL call gave up its wait for the other workgroups' row partials
 * after its time limit (~1 s; every other workgroup publishes its partial
 * without waiting on anything unbounded, so this happens only when no other
 * workgroup of the launch could run in that time); that call's loss was
 * written as NaN, and the workspace must be zero-filled again before its next
 * use.  The other waits never give up: the sums of a split row's pieces and
 * the per-token losses' values are computed by the waiting workgroup when they
 * do not come within the steal limit (see Workspace above). */
int rlpl_workspace_flags(const void* workspace, uint32_t* flags_out, hipStream_t stream);

/* Limits of the cross-workgroup waits of calls that use `workspace`, in ticks
 * of the GPU's 100 MHz clock; 0 selects the default.  steal_ticks: how long a
 * coordinating workgroup waits for a value another workgroup publishes before
 * computing it itself (default 5,000 = 50 us; the same limit holds for the
 * piece sums of a full-vocab call's split rows); release_ticks: how long a
 * workgroup waits for the global count before forming it itself (default
 * 20,000); giveup_ticks: how long a full-vocab reverse-KL call waits before it
 * gives up (default 100,000,000 = 1 s).  Results never depend on these limits
 * (tests set them small to exercise every path); only timing does.
 * Enqueued on `stream` (three 4-byte fills, not synchronised); the workspace
 * must be 256-byte aligned and at least rlpl_workspace_bytes long. */
int rlpl_workspace_set_limits(void* workspace, uint32_t steal_ticks, uint32_t release_ticks,
                              uint32_t giveup_ticks, hipStream_t stream);

/* Human-readable name of an rlpl_status value (static string). */
const char* rlpl_status_string(int status);

/* ABI version of this library. */
int rlpl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RL_POST_LOSS_H */
