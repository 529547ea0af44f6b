"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/rlpl_oracle.c (on the CPU),
builds it, points the oracle wrapper at it and runs every pin in
test_oracle.py: at least one pin has to fail.
"""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle
import test_oracle_logprob
import test_oracle_ppo
import test_oracle_vocab

SRC = os.path.join(os.path.dirname(oracle.__file__), "rlpl_oracle.c")

MUTANTS = {
    "ratio uses old - lp": ("double ratio = exp(lp - old);", "double ratio = exp(old - lp);"),
    "kl uses lp - ref": ("double x = ref - lp;", "double x = lp - ref;"),
    "kl drops the -1": ("return e - x - 1.0;", "return e - x;"),
    "kl slope sign": ("*slope = -(e - 1.0);", "*slope = (e - 1.0);"),
    "policy slope sign": ("*slope = -adv * dchosen;", "*slope = adv * dchosen;"),
    "policy term sign": ("return -adv * chosen;", "return adv * chosen;"),
    "slope misses chain-rule ratio": ("dchosen = ratio;", "dchosen = 1.0;"),
    "ties take the clipped branch": ("if (ratio <= clipped) {", "if (ratio < clipped) {"),
    "upper bound uses eps": ("hi = 1.0 + eps_high;", "hi = 1.0 + eps;"),
    "beta dropped": ("term += beta * kl;", "term += kl;"),
    "advantage of row 0 everywhere": (
        "sum += token_term(lp, old, ref, adv[r], i, beta, lo, hi, sign_aware, &slope);",
        "sum += token_term(lp, old, ref, adv[0], i, beta, lo, hi, sign_aware, &slope);"),
    "bnpo denominator not clamped": ("    if (denom < 1.0) denom = 1.0;   /* max(mask.sum(), 1) */\n", ""),
    "grpo grad misses 1/bs": ("grad[i] = slope / (denom * (double)bs);", "grad[i] = slope / denom;"),
    "grpo mean over valid rows": None,   # built by hand below
    "rkl grad not normalised": ("grad[i] = slope / (double)n;", "grad[i] = slope;"),
    "ppo picks the max objective": ("if (unclipped_obj <= clipped_obj) {", "if (unclipped_obj >= clipped_obj) {"),
    "ppo clipped branch has a slope": ("    *slope = 0.0;                /* the clipped objective is a constant in lp */",
                                       "    *slope = -adv * clipped;"),
    "ppo uses the literal min for every sign": ("double unclipped_obj = adv * ratio, clipped_obj = adv * clipped;",
                                                "double unclipped_obj = ratio, clipped_obj = clipped;"),
    "logprob dz sign": ("grad_logp[i] * ((v == targets[i] ? 1.0 : 0.0) - exp(z[v] - l));",
                        "grad_logp[i] * (exp(z[v] - l) - (v == targets[i] ? 1.0 : 0.0));"),
    "logprob d_weight uses the weight": ("d_weight[v * h + k] += dz * x[k];", "d_weight[v * h + k] += dz * w[k];"),
    "logprob bias ignored": ("double acc = bias ? bias[v] : 0.0;", "double acc = 0.0;"),
    "logprob gathers logit 0": ("logp[i] = z[targets[i]] - l;", "logp[i] = z[0] - l;"),
    "logprob d_hidden misses the softmax": ("const double dz = grad_logp[i] * ((v == targets[i] ? 1.0 : 0.0) - exp(z[v] - l));",
                                            "const double dz = grad_logp[i] * (v == targets[i] ? 1.0 : 0.0);"),
    "vocab forward KL instead of reverse": ("kl += exp(log_p) * (log_p - log_q);",
                                            "kl += exp(log_q) * (log_q - log_p);"),
    "vocab grad misses -kl_row": ("g[v] = exp(log_p) * (log_p - log_q - kl) / (double)n;",
                                  "g[v] = exp(log_p) * (log_p - log_q) / (double)n;"),
    "vocab grad weighted by q": ("g[v] = exp(log_p) * (log_p - log_q - kl) / (double)n;",
                                 "g[v] = exp(log_q) * (log_p - log_q - kl) / (double)n;"),
    "vocab grad sign": ("g[v] = exp(log_p) * (log_p - log_q - kl) / (double)n;",
                        "g[v] = exp(log_p) * (log_q - log_p + kl) / (double)n;"),
    "vocab mean over all rows": ("*loss = sum / (double)n;   /* not clamped: 0/0 is NaN when no row is valid */",
                                 "*loss = sum / (double)rows;"),
    "vocab counts masked rows": ("        if (mask[r] != 0) ++n;\n", "        ++n;\n"),
    "vocab teacher normaliser from student": ("lse_t = log_sum_exp(t, vocab);", "lse_t = log_sum_exp(s, vocab);"),
    "vocab log-sum-exp drops the max": ("    return m + log(z);", "    return log(z);"),
    "vocab grad row offset": ("double *g = grad ? grad + r * vocab : NULL;", "double *g = grad ? grad + r : NULL;"),
    "rkl reads masked tokens": ("        if (mask[i] == 0) continue;\n        ++n;\n        sum += k3_kl(", "        if (mask[i] == 0) { sum += 0.0 * student[i]; continue; }\n        ++n;\n        sum += k3_kl("),
}


def _pins():
    return [(name, fn) for mod in (test_oracle, test_oracle_logprob, test_oracle_ppo, test_oracle_vocab)
            for name, fn in inspect.getmembers(mod, inspect.isfunction)
            if name.startswith("test_") and "generator" not in name]


def _param_sets(fn):
    """Keyword-argument sets of a pin: the product of its parametrize marks."""
    sets = [{}]
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
        sets = [dict(s, **dict(zip(names, v))) for s in sets for v in vals]
    return sets


def _run_pins():
    failed = []
    for name, fn in _pins():
        for kw in _param_sets(fn):
            try:
                fn(**kw)
            except (AssertionError, ValueError):
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("case", sorted(MUTANTS))
def test_pins_catch_planted_mistake(case, tmp_path):
    src = open(SRC).read()
    if case == "grpo mean over valid rows":
        # divide the row total by the number of non-empty rows instead of bs
        src2 = src.replace("    double total = 0.0, slope;\n    for (int64_t r = 0; r < bs; ++r) {",
                           "    double total = 0.0, slope; int64_t nonempty = 0;\n    for (int64_t r = 0; r < bs; ++r) {")
        src2 = src2.replace("total += row_sum / denom;", "total += row_sum / denom; if (n > 0) ++nonempty;")
        src2 = src2.replace("*loss = bs > 0 ? total / (double)bs : 0.0;",
                            "*loss = nonempty > 0 ? total / (double)nonempty : 0.0;")
        assert src2 != src
    else:
        old, new = MUTANTS[case]
        assert src.count(old) >= 1, case
        src2 = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src2)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(so), str(c), "-lm"])
    oracle._use_library(str(so))
    try:
        failed = _run_pins()
    finally:
        oracle._use_library(None)
    assert failed, f"no pin caught the planted mistake: {case}"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
