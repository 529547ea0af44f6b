/*
 * CPU oracle for the fused PPO-family policy losses.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path (the
 * HIP kernels behind include/rl_post_loss.h) never does, and shares no code
 * with it.
 *
 * Plain C99, every quantity in double, the tokens visited one by one in
 * row-major order.  The log-prob planes arrive already widened (exactly) from
 * their storage dtype to double.  Nothing is blocked, fused or reordered
 * beyond what the formulas state.
 *
 * Source: the model card "Geometric-AI Kernels" (Hugging Face page of
 * Geometric-AI/geometric-ai-kernels):
 *   - section "BNPO Loss": ratio, clipped, per_token and kl formulas, and the
 *     global token-mean  loss = sum((per_token + beta*kl)*mask) / max(sum(mask), 1);
 *   - section "GRPO Loss": per-response normalisation
 *     loss = mean_r( sum_t((per_token + beta*kl)*mask) / max(sum_t(mask), 1) );
 *   - section "Reverse KL": KL(student || teacher) between the softmaxes of two
 *     (rows, vocab) logit slabs, kl_row = sum_v p_v (log p_v - log q_v),
 *     loss = (mask * kl_row).sum() / mask.sum() (unclamped), and the analytic
 *     gradient p_v (log p_v - log q_v - kl_row) * mask[r] / mask.sum(); the
 *     same normalisation for the per-token estimator below.
 *
 * Readings of points the card leaves open:
 *   - per_token = -A * min(ratio, clip(ratio, 1-eps, 1+eps_high)) literally;
 *     when ratio equals its clipped value the unclipped branch is taken, so
 *     d per_token / d lp = -A*ratio unless clipping lowered ratio to 1+eps_high.
 *     The *_ppo functions take the sign-aware PPO form
 *     -min(A*ratio, A*clip(ratio, 1-eps, 1+eps_high)) instead (the card calls
 *     per_token "PPO-clipped"); ties again take the unclipped branch.
 *   - masked slots are selected out: they add nothing, their gradient is +0 and
 *     their log-probs are never read.  Any nonzero mask byte means "valid".
 *   - GRPO averages over all bs rows; a fully masked row adds 0 and still counts.
 *   - Reverse-KL on per-token log-probs is the card's per-token KL estimator
 *     exp(x) - x - 1 with x = teacher - student, averaged over valid tokens
 *     with the unclamped 1/N, so an all-masked batch gives 0/0 = NaN loss and
 *     a +0 gradient.
 *
 * Selective log-probabilities (the step upstream of the loss, page "Add SM100
 * CuTe DSL GRPO fast path", section "Summary"): for each token i, the logits
 * z_i = hidden_i . weight^T (+ bias) over the vocabulary (temperature 1), and
 * logp_i = z_i[target_i] - log(sum_v exp(z_i[v])).  The backward for an
 * upstream gradient g_i = d loss / d logp_i: dz_i = g_i (onehot(target_i) -
 * softmax(z_i)), d hidden_i = dz_i . weight, d weight = sum_i dz_i^T hidden_i,
 * d bias = sum_i dz_i.
 *
 * Parity pins for every function here live in tests/test_oracle*.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define RLPL_ORACLE_VERSION 4

int rlpl_oracle_version(void) { return RLPL_ORACLE_VERSION; }

/* PPO-clipped ratio term of one token ("BNPO Loss": ratio, clipped, per_token).
 * Returns per_token; *slope receives d per_token / d lp (d ratio / d lp = ratio). */
static double clipped_ratio_term(double lp, double old, double adv, double lo, double hi,
                                 double *slope)
{
    double ratio = exp(lp - old);
    double clipped = ratio;
    if (clipped < lo) clipped = lo;
    if (clipped > hi) clipped = hi;
    double chosen, dchosen;
    if (ratio <= clipped) {
        chosen = ratio;          /* min picks the unclipped ratio (ties included) */
        dchosen = ratio;
    } else {
        chosen = clipped;        /* only when clipping lowered ratio to hi, a constant */
        dchosen = 0.0;
    }
    *slope = -adv * dchosen;
    return -adv * chosen;
}

/* Sign-aware PPO ratio term of one token: per_token = -min(A*ratio, A*clipped),
 * the standard PPO clipped objective that the card's "PPO-clipped" names (for
 * A >= 0 it equals the literal form above; for A < 0 the lower bound 1-eps
 * is the one that clips).  Ties take the unclipped branch.  *slope receives
 * d per_token / d lp. */
static double ppo_ratio_term(double lp, double old, double adv, double lo, double hi,
                             double *slope)
{
    double ratio = exp(lp - old);
    double clipped = ratio;
    if (clipped < lo) clipped = lo;
    if (clipped > hi) clipped = hi;
    double unclipped_obj = adv * ratio, clipped_obj = adv * clipped;
    if (unclipped_obj <= clipped_obj) {
        *slope = -adv * ratio;   /* the unclipped objective is the minimum (ties included) */
        return -unclipped_obj;
    }
    *slope = 0.0;                /* the clipped objective is a constant in lp */
    return -clipped_obj;
}

/* k3 KL estimator of one token ("BNPO Loss": kl), x = ref - lp.
 * Returns kl; *slope receives d kl / d lp = -(exp(x) - 1). */
static double k3_kl(double lp, double ref, double *slope)
{
    double x = ref - lp;
    double e = exp(x);
    *slope = -(e - 1.0);
    return e - x - 1.0;
}

/* Per-token loss contribution (per_token + beta*kl) and its derivative in lp;
 * sign_aware selects the sign-aware PPO ratio term. */
static double token_term(const double *lp, const double *old, const double *ref,
                         double adv, int64_t i, double beta, double lo, double hi,
                         int sign_aware, double *slope)
{
    double dpol;
    double term = sign_aware ? ppo_ratio_term(lp[i], old[i], adv, lo, hi, &dpol)
                             : clipped_ratio_term(lp[i], old[i], adv, lo, hi, &dpol);
    double dkl = 0.0;
    if (beta != 0.0) {
        double kl = k3_kl(lp[i], ref[i], &dkl);
        term += beta * kl;
    }
    *slope = dpol + beta * dkl;
    return term;
}

/*
 * BNPO: loss = sum((per_token + beta*kl) * mask) / max(sum(mask), 1).
 * grad[i] = d loss / d lp[i]  (mask[i] != 0), +0 otherwise.  grad may be NULL
 * (loss only).  ref may be NULL when beta == 0.  *n_valid = sum(mask != 0).
 * Returns 0, or -1 on a NULL required pointer / bad shape.
 */
static int bnpo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                const double *ref, const double *adv, const uint8_t *mask,
                double beta, double eps, double eps_high, int sign_aware,
                double *loss, double *grad, int64_t *n_valid)
{
    if (bs < 0 || seq_len < 0 || !lp || !old || !adv || !mask || !loss || !n_valid) return -1;
    if (beta != 0.0 && !ref) return -1;
    const double lo = 1.0 - eps, hi = 1.0 + eps_high;
    int64_t n = 0;
    double sum = 0.0, slope;
    for (int64_t r = 0; r < bs; ++r)
        for (int64_t t = 0; t < seq_len; ++t) {
            int64_t i = r * seq_len + t;
            if (mask[i] == 0) continue;
            ++n;
            sum += token_term(lp, old, ref, adv[r], i, beta, lo, hi, sign_aware, &slope);
        }
    double denom = (double)n;
    if (denom < 1.0) denom = 1.0;   /* max(mask.sum(), 1) */
    *loss = sum / denom;
    *n_valid = n;
    if (grad)
        for (int64_t r = 0; r < bs; ++r)
            for (int64_t t = 0; t < seq_len; ++t) {
                int64_t i = r * seq_len + t;
                if (mask[i] == 0) { grad[i] = 0.0; continue; }
                token_term(lp, old, ref, adv[r], i, beta, lo, hi, sign_aware, &slope);
                grad[i] = slope / denom;
            }
    return 0;
}

/*
 * GRPO: loss = (1/bs) * sum_r [ sum_t((per_token + beta*kl) * mask) / max(sum_t(mask), 1) ].
 * grad[i] = d loss / d lp[i].  n_valid has bs entries (per-row counts).
 */
static int grpo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                const double *ref, const double *adv, const uint8_t *mask,
                double beta, double eps, double eps_high, int sign_aware,
                double *loss, double *grad, int64_t *n_valid)
{
    if (bs < 0 || seq_len < 0 || !lp || !old || !adv || !mask || !loss || !n_valid) return -1;
    if (beta != 0.0 && !ref) return -1;
    const double lo = 1.0 - eps, hi = 1.0 + eps_high;
    double total = 0.0, slope;
    for (int64_t r = 0; r < bs; ++r) {
        int64_t n = 0;
        double row_sum = 0.0;
        for (int64_t t = 0; t < seq_len; ++t) {
            int64_t i = r * seq_len + t;
            if (mask[i] == 0) continue;
            ++n;
            row_sum += token_term(lp, old, ref, adv[r], i, beta, lo, hi, sign_aware, &slope);
        }
        double denom = (double)n;
        if (denom < 1.0) denom = 1.0;   /* max(mask.sum(-1), 1) */
        total += row_sum / denom;
        n_valid[r] = n;
        if (grad)
            for (int64_t t = 0; t < seq_len; ++t) {
                int64_t i = r * seq_len + t;
                if (mask[i] == 0) { grad[i] = 0.0; continue; }
                token_term(lp, old, ref, adv[r], i, beta, lo, hi, sign_aware, &slope);
                grad[i] = slope / (denom * (double)bs);
            }
    }
    *loss = bs > 0 ? total / (double)bs : 0.0;   /* mean over the bs rows */
    return 0;
}

/* The card's literal per_token (-A * min(ratio, clipped)) ... */
int rlpl_oracle_bnpo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                     const double *ref, const double *adv, const uint8_t *mask,
                     double beta, double eps, double eps_high,
                     double *loss, double *grad, int64_t *n_valid)
{
    return bnpo(bs, seq_len, lp, old, ref, adv, mask, beta, eps, eps_high, 0, loss, grad, n_valid);
}

int rlpl_oracle_grpo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                     const double *ref, const double *adv, const uint8_t *mask,
                     double beta, double eps, double eps_high,
                     double *loss, double *grad, int64_t *n_valid)
{
    return grpo(bs, seq_len, lp, old, ref, adv, mask, beta, eps, eps_high, 0, loss, grad, n_valid);
}

/* ... and the sign-aware PPO per_token (-min(A*ratio, A*clipped)), same normalisations. */
int rlpl_oracle_bnpo_ppo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                         const double *ref, const double *adv, const uint8_t *mask,
                         double beta, double eps, double eps_high,
                         double *loss, double *grad, int64_t *n_valid)
{
    return bnpo(bs, seq_len, lp, old, ref, adv, mask, beta, eps, eps_high, 1, loss, grad, n_valid);
}

int rlpl_oracle_grpo_ppo(int64_t bs, int64_t seq_len, const double *lp, const double *old,
                         const double *ref, const double *adv, const uint8_t *mask,
                         double beta, double eps, double eps_high,
                         double *loss, double *grad, int64_t *n_valid)
{
    return grpo(bs, seq_len, lp, old, ref, adv, mask, beta, eps, eps_high, 1, loss, grad, n_valid);
}

/*
 * Reverse-KL on per-token log-probs: x = teacher - student,
 * loss = sum(mask * (exp(x) - x - 1)) / sum(mask)  (unclamped: 0/0 = NaN when
 * every token is masked), grad[i] = (1 - exp(x)) / sum(mask) on valid tokens,
 * +0 elsewhere.
 */
int rlpl_oracle_rkl(int64_t bs, int64_t seq_len, const double *student, const double *teacher,
                    const uint8_t *mask, double *loss, double *grad, int64_t *n_valid)
{
    if (bs < 0 || seq_len < 0 || !student || !teacher || !mask || !loss || !n_valid) return -1;
    int64_t n = 0;
    double sum = 0.0, slope;
    for (int64_t i = 0; i < bs * seq_len; ++i) {
        if (mask[i] == 0) continue;
        ++n;
        sum += k3_kl(student[i], teacher[i], &slope);
    }
    *loss = sum / (double)n;   /* not clamped: 0/0 is NaN when no token is valid */
    *n_valid = n;
    if (grad)
        for (int64_t i = 0; i < bs * seq_len; ++i) {
            if (mask[i] == 0) { grad[i] = 0.0; continue; }
            k3_kl(student[i], teacher[i], &slope);
            grad[i] = slope / (double)n;
        }
    return 0;
}

/* log(sum_v exp(x_v)) of one row, as max + log(sum exp(x_v - max)): the same
 * number, written so that no exp overflows. */
static double log_sum_exp(const double *x, int64_t n)
{
    double m = x[0];
    for (int64_t v = 1; v < n; ++v)
        if (x[v] > m) m = x[v];
    double z = 0.0;
    for (int64_t v = 0; v < n; ++v) z += exp(x[v] - m);
    return m + log(z);
}

/*
 * Reverse KL over full logit rows ("Reverse KL"): for each row r of the
 * (rows, vocab) slabs, p = softmax(student[r]), q = softmax(teacher[r]),
 * kl_r = sum_v p_v (log p_v - log q_v).  N = number of rows with a nonzero
 * mask byte; loss = sum_r mask_r kl_r / N, not clamped (0/0 = NaN when every
 * row is masked).  grad (rows*vocab, optional) = p_v (log p_v - log q_v - kl_r)
 * / N on valid rows and +0 on masked rows, whose logits are never read.
 * kl_rows (rows, optional) receives kl_r for valid rows and 0 for masked rows.
 */
int rlpl_oracle_rkl_logits(int64_t rows, int64_t vocab, const double *student,
                           const double *teacher, const uint8_t *mask, double *loss,
                           double *grad, int64_t *n_valid, double *kl_rows)
{
    if (rows < 0 || vocab < 1 || !student || !teacher || !mask || !loss || !n_valid) return -1;
    int64_t n = 0;
    for (int64_t r = 0; r < rows; ++r)
        if (mask[r] != 0) ++n;
    double sum = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const double *s = student + r * vocab, *t = teacher + r * vocab;
        double *g = grad ? grad + r * vocab : NULL;
        if (mask[r] == 0) {
            if (g)
                for (int64_t v = 0; v < vocab; ++v) g[v] = 0.0;
            if (kl_rows) kl_rows[r] = 0.0;
            continue;
        }
        const double lse_s = log_sum_exp(s, vocab), lse_t = log_sum_exp(t, vocab);
        double kl = 0.0;
        for (int64_t v = 0; v < vocab; ++v) {
            const double log_p = s[v] - lse_s, log_q = t[v] - lse_t;
            kl += exp(log_p) * (log_p - log_q);
        }
        sum += kl;
        if (kl_rows) kl_rows[r] = kl;
        if (g)
            for (int64_t v = 0; v < vocab; ++v) {
                const double log_p = s[v] - lse_s, log_q = t[v] - lse_t;
                g[v] = exp(log_p) * (log_p - log_q - kl) / (double)n;
            }
    }
    *loss = sum / (double)n;   /* not clamped: 0/0 is NaN when no row is valid */
    *n_valid = n;
    return 0;
}

/*
 * Selective log-probabilities: logp[i] = z_i[target_i] - logsumexp(z_i), with
 * z_i[v] = sum_k hidden[i][k] * weight[v][k] + (bias ? bias[v] : 0).
 * hidden (n, h), weight (vocab, h), bias (vocab) or NULL, targets (n) in
 * [0, vocab).  lse (n, optional) receives logsumexp(z_i).
 * When grad_logp is not NULL it also writes d_hidden (n, h), d_weight
 * (vocab, h) and d_bias (vocab, if bias) for the upstream gradient grad_logp
 * (each of the three outputs may be NULL).  Returns 0, or -1 on bad arguments.
 */
int rlpl_oracle_selective_logprob(int64_t n, int64_t h, int64_t vocab, const double *hidden,
                                  const double *weight, const double *bias, const int64_t *targets,
                                  double *logp, double *lse, const double *grad_logp,
                                  double *d_hidden, double *d_weight, double *d_bias)
{
    if (n < 0 || h < 1 || vocab < 1 || !hidden || !weight || !targets || !logp) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (targets[i] < 0 || targets[i] >= vocab) return -1;
    if (d_weight)
        for (int64_t j = 0; j < vocab * h; ++j) d_weight[j] = 0.0;
    if (d_bias)
        for (int64_t v = 0; v < vocab; ++v) d_bias[v] = 0.0;
    double *z = (double *)malloc((size_t)vocab * sizeof(double));
    if (!z) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double *x = hidden + i * h;
        for (int64_t v = 0; v < vocab; ++v) {
            double acc = bias ? bias[v] : 0.0;
            const double *w = weight + v * h;
            for (int64_t k = 0; k < h; ++k) acc += x[k] * w[k];
            z[v] = acc;
        }
        const double l = log_sum_exp(z, vocab);
        logp[i] = z[targets[i]] - l;
        if (lse) lse[i] = l;
        if (!grad_logp) continue;
        if (d_hidden)
            for (int64_t k = 0; k < h; ++k) d_hidden[i * h + k] = 0.0;
        for (int64_t v = 0; v < vocab; ++v) {
            const double dz = grad_logp[i] * ((v == targets[i] ? 1.0 : 0.0) - exp(z[v] - l));
            const double *w = weight + v * h;
            if (d_hidden)
                for (int64_t k = 0; k < h; ++k) d_hidden[i * h + k] += dz * w[k];
            if (d_weight)
                for (int64_t k = 0; k < h; ++k) d_weight[v * h + k] += dz * x[k];
            if (d_bias) d_bias[v] += dz;
        }
    }
    free(z);
    return 0;
}
