/*
 * Drives every entry point of the CPU oracle (oracle/rlpl_oracle.c) over
 * seeded random small problems, edge cases included (empty shapes, fully
 * masked inputs, optional outputs left NULL, rejected arguments), with every
 * buffer allocated at its exact size: built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py, any out-of-bounds
 * access, use of freed memory or undefined arithmetic aborts the run.
 * Prints "ok <calls>" and exits 0 when every call returned what its
 * arguments call for.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int rlpl_oracle_version(void);
int rlpl_oracle_bnpo(int64_t, int64_t, const double *, const double *, const double *, const double *,
                     const uint8_t *, double, double, double, double *, double *, int64_t *);
int rlpl_oracle_grpo(int64_t, int64_t, const double *, const double *, const double *, const double *,
                     const uint8_t *, double, double, double, double *, double *, int64_t *);
int rlpl_oracle_bnpo_ppo(int64_t, int64_t, const double *, const double *, const double *, const double *,
                         const uint8_t *, double, double, double, double *, double *, int64_t *);
int rlpl_oracle_grpo_ppo(int64_t, int64_t, const double *, const double *, const double *, const double *,
                         const uint8_t *, double, double, double, double *, double *, int64_t *);
int rlpl_oracle_rkl(int64_t, int64_t, const double *, const double *, const uint8_t *, double *, double *,
                    int64_t *);
int rlpl_oracle_rkl_logits(int64_t, int64_t, const double *, const double *, const uint8_t *, double *,
                           double *, int64_t *, double *);
int rlpl_oracle_selective_logprob(int64_t, int64_t, int64_t, const double *, const double *, const double *,
                                  const int64_t *, double *, double *, const double *, double *, double *,
                                  double *);

static uint64_t state = 0x9e3779b97f4a7c15ull;

static uint64_t next_u64(void) {   /* splitmix64 */
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double uniform(double lo, double hi) { return lo + (hi - lo) * (double)(next_u64() >> 11) * 0x1p-53; }
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u64() % (uint64_t)n) : 0; }

/* Exact-size allocations (at least one byte, so that a zero-size problem still
 * gets a distinct pointer whose every access is out of bounds). */
static double *doubles(int64_t n, double lo, double hi) {
    double *p = malloc(n > 0 ? (size_t)n * sizeof(double) : 1);
    for (int64_t i = 0; i < n; ++i) p[i] = uniform(lo, hi);
    return p;
}
static uint8_t *mask_of(int64_t n, double p_valid) {
    uint8_t *m = malloc(n > 0 ? (size_t)n : 1);
    for (int64_t i = 0; i < n; ++i) m[i] = uniform(0.0, 1.0) < p_valid ? (uint8_t)(1 + below(255)) : 0;
    return m;
}

static long calls = 0, failures = 0;

static void expect(int got, int want, const char *what, int64_t a, int64_t b) {
    ++calls;
    if (got != want) {
        ++failures;
        fprintf(stderr, "FAIL %s (%lld, %lld): returned %d, expected %d\n", what, (long long)a, (long long)b, got,
                want);
    }
}

typedef int (*policy_fn)(int64_t, int64_t, const double *, const double *, const double *, const double *,
                         const uint8_t *, double, double, double, double *, double *, int64_t *);

static void policy_case(int64_t bs, int64_t T, double p_valid) {
    static const policy_fn fns[4] = {rlpl_oracle_bnpo, rlpl_oracle_grpo, rlpl_oracle_bnpo_ppo, rlpl_oracle_grpo_ppo};
    static const char *names[4] = {"bnpo", "grpo", "bnpo_ppo", "grpo_ppo"};
    const int64_t n = bs * T;
    double *lp = doubles(n, -4.0, -0.01), *old = doubles(n, -4.0, -0.01), *ref = doubles(n, -4.0, -0.01);
    double *adv = doubles(bs, -2.0, 2.0), *grad = doubles(n, 0.0, 0.0);
    uint8_t *mask = mask_of(n, p_valid);
    int64_t *counts = malloc((bs > 0 ? (size_t)bs : 1) * sizeof(int64_t));
    for (int f = 0; f < 4; ++f) {
        double loss = 0.0;
        const double beta = (f & 1) ? 0.0 : 0.04;
        /* with beta 0 the reference plane is optional */
        expect(fns[f](bs, T, lp, old, beta == 0.0 ? NULL : ref, adv, mask, beta, 0.2, 0.28, &loss, grad, counts),
               0, names[f], bs, T);
        if (!isfinite(loss)) expect(1, 0, "finite loss", bs, T);
        expect(fns[f](bs, T, lp, old, ref, adv, mask, 0.04, 0.2, 0.28, &loss, NULL, counts), 0, names[f], bs, T);
        expect(fns[f](bs, T, lp, old, NULL, adv, mask, 0.04, 0.2, 0.28, &loss, grad, counts), -1, names[f], bs, T);
        expect(fns[f](bs, T, NULL, old, ref, adv, mask, 0.04, 0.2, 0.28, &loss, grad, counts), -1, names[f], bs, T);
        expect(fns[f](-1, T, lp, old, ref, adv, mask, 0.04, 0.2, 0.28, &loss, grad, counts), -1, names[f], -1, T);
    }
    free(lp); free(old); free(ref); free(adv); free(grad); free(mask); free(counts);
}

static void rkl_case(int64_t bs, int64_t T, double p_valid) {
    const int64_t n = bs * T;
    double *s = doubles(n, -6.0, -0.01), *t = doubles(n, -6.0, -0.01), *grad = doubles(n, 0.0, 0.0);
    uint8_t *mask = mask_of(n, p_valid);
    double loss = 0.0;
    int64_t count = -1;
    expect(rlpl_oracle_rkl(bs, T, s, t, mask, &loss, grad, &count), 0, "rkl", bs, T);
    if ((count > 0) != isfinite(loss)) expect(1, 0, "rkl loss finite iff a token is valid", bs, T);
    expect(rlpl_oracle_rkl(bs, T, s, t, mask, &loss, NULL, &count), 0, "rkl", bs, T);
    expect(rlpl_oracle_rkl(bs, T, s, NULL, mask, &loss, grad, &count), -1, "rkl", bs, T);
    free(s); free(t); free(grad); free(mask);
}

static void vocab_case(int64_t rows, int64_t V, double p_valid) {
    const int64_t n = rows * V;
    double *s = doubles(n, -8.0, 8.0), *t = doubles(n, -8.0, 8.0), *grad = doubles(n, 0.0, 0.0);
    double *kl = doubles(rows, 0.0, 0.0);
    uint8_t *mask = mask_of(rows, p_valid);
    double loss = 0.0;
    int64_t count = -1;
    expect(rlpl_oracle_rkl_logits(rows, V, s, t, mask, &loss, grad, &count, kl), 0, "rkl_logits", rows, V);
    expect(rlpl_oracle_rkl_logits(rows, V, s, t, mask, &loss, NULL, &count, NULL), 0, "rkl_logits", rows, V);
    expect(rlpl_oracle_rkl_logits(rows, 0, s, t, mask, &loss, grad, &count, kl), -1, "rkl_logits", rows, 0);
    free(s); free(t); free(grad); free(kl); free(mask);
}

static void logprob_case(int64_t n, int64_t h, int64_t V) {
    double *x = doubles(n * h, -1.0, 1.0), *w = doubles(V * h, -1.0, 1.0), *b = doubles(V, -0.5, 0.5);
    double *logp = doubles(n, 0.0, 0.0), *lse = doubles(n, 0.0, 0.0), *g = doubles(n, -1.0, 1.0);
    double *dx = doubles(n * h, 0.0, 0.0), *dw = doubles(V * h, 0.0, 0.0), *db = doubles(V, 0.0, 0.0);
    int64_t *tg = malloc((n > 0 ? (size_t)n : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) tg[i] = below(V);
    expect(rlpl_oracle_selective_logprob(n, h, V, x, w, b, tg, logp, lse, g, dx, dw, db), 0, "logprob", n, V);
    expect(rlpl_oracle_selective_logprob(n, h, V, x, w, NULL, tg, logp, NULL, NULL, NULL, NULL, NULL), 0,
           "logprob fwd", n, V);
    expect(rlpl_oracle_selective_logprob(n, h, V, x, w, b, tg, logp, lse, g, NULL, dw, NULL), 0, "logprob dw",
           n, V);
    if (n > 0) {
        const int64_t keep = tg[0];
        tg[0] = V;                         /* a target outside the vocabulary is rejected */
        expect(rlpl_oracle_selective_logprob(n, h, V, x, w, b, tg, logp, lse, g, dx, dw, db), -1, "logprob",
               n, V);
        tg[0] = keep;
    }
    free(x); free(w); free(b); free(logp); free(lse); free(g); free(dx); free(dw); free(db); free(tg);
}

int main(void) {
    if (rlpl_oracle_version() < 1) return 2;
    static const int64_t edges[][2] = {{0, 0}, {0, 5}, {5, 0}, {1, 1}, {1, 17}, {3, 64}, {7, 33}};
    for (size_t e = 0; e < sizeof edges / sizeof edges[0]; ++e)
        for (int k = 0; k < 3; ++k) {
            const double p = k == 0 ? 0.0 : k == 1 ? 1.0 : 0.6;
            policy_case(edges[e][0], edges[e][1], p);
            rkl_case(edges[e][0], edges[e][1], p);
        }
    for (int i = 0; i < 60; ++i) {
        policy_case(below(9), below(70), uniform(0.0, 1.0));
        rkl_case(below(9), below(70), uniform(0.0, 1.0));
        vocab_case(below(6), 1 + below(300), uniform(0.0, 1.0));
    }
    vocab_case(0, 1, 1.0);
    vocab_case(3, 1, 1.0);
    for (int i = 0; i < 12; ++i) logprob_case(below(6), 1 + below(24), 1 + below(40));
    logprob_case(0, 4, 3);
    printf("ok %ld\n", calls);
    return failures ? 1 : 0;
}
