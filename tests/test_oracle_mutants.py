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
        "sum += token_term(lp, old, ref, adv[r], i, beta, lo, hi, &slope);",
        "sum += token_term(lp, old, ref, adv[0], i, beta, lo, hi, &slope);"),
    "bnpo denominator not clamped": ("    if (denom < 1.0) denom = 1.0;   /* max(mask.sum(), 1) */\n", ""),
    "grpo grad misses 1/bs": ("grad[i] = slope / (denom * (double)bs);", "grad[i] = slope / denom;"),
    "grpo mean over valid rows": None,   # built by hand below
    "rkl grad not normalised": ("grad[i] = slope / (double)n;", "grad[i] = slope;"),
    "rkl reads masked tokens": ("        if (mask[i] == 0) continue;\n        ++n;\n        sum += k3_kl(", "        if (mask[i] == 0) { sum += 0.0 * student[i]; continue; }\n        ++n;\n        sum += k3_kl("),
}


def _pins():
    return [(name, fn) for name, fn in inspect.getmembers(test_oracle, inspect.isfunction)
            if name.startswith("test_") and "generator" not in name]


def _run_pins():
    failed = []
    for name, fn in _pins():
        sig = inspect.signature(fn)
        params = [[]]
        mark = getattr(fn, "pytestmark", [])
        for m in mark:
            if m.name == "parametrize":
                params = [[v] for v in m.args[1]]
        for p in params:
            try:
                fn(*p)
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
