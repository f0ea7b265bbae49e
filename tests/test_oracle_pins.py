"""The CPU oracle against its pins (runs without a GPU)."""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_FAST_PINS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


def test_brute_force_bf16():
    P.check_brute_force(seed=30, dtype="bf16")


def test_uniform_routing_statistics():
    P.check_uniform_routing()


def test_parameter_counts_match_pages():
    P.check_parameter_counts()


# Plausible mistakes, each planted in a copy of the oracle's C source.  Every
# one must make at least one pin fail; a mutant that passes all pins would
# mean the pins cannot see that class of error.
MUTANTS = {
    "silu_on_w3_branch": ("a[j] = silu(a[j]) * b[j];", "a[j] = a[j] * silu(b[j]);"),
    "softmax_sign": ("gates[j] = exp(l[ids[j]] - lmax);", "gates[j] = exp(lmax - l[ids[j]]);"),
    "ties_to_high_index": ("if (best < 0 || v > best_v) {", "if (best < 0 || v >= best_v) {"),
    "picks_smallest": ("if (best < 0 || v > best_v) {", "if (best < 0 || v < best_v) {"),
    "router_transposed": ("elem(w_router, dtype, i * E + e)", "elem(w_router, dtype, e * d + i)"),
    "router_drops_term": ("for (int64_t i = 0; i < d; ++i) {\n        double xi = elem(x, dtype, t * d + i);\n        for (int64_t e = 0;",
                          "for (int64_t i = 1; i < d; ++i) {\n        double xi = elem(x, dtype, t * d + i);\n        for (int64_t e = 0;"),
    "w2_transposed": ("elem(w2, dtype, w2_base + j * d + c)", "elem(w2, dtype, w2_base + c * f + j)"),
    "w1_transposed": ("a[j] += xi * elem(w1, dtype, w13_base + i * f + j);", "a[j] += xi * elem(w1, dtype, w13_base + j * d + i);"),
    "gates_unnormalised": ("gates[j] /= z;", "gates[j] /= 1.0;"),
    "overwrites_not_sums": ("o[c] += g[j] * ye[c];", "o[c] = g[j] * ye[c];"),
    "bias_subtracted": ("l[e] += (double)bias[e];", "l[e] -= (double)bias[e];"),
    "rmsnorm_no_eps": ("ss / (double)d + eps", "ss / (double)d"),
    "ungated_sum": ("o[c] += g[j] * ye[c];", "o[c] += ye[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new, 1)
    cfile = tmp_path / "mutant.c"
    cfile.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-I", os.path.dirname(oracle.__file__), str(cfile), "-o", str(so), "-lm"],
                   check=True)
    mutant = oracle.configure(ctypes.CDLL(str(so)))
    saved = oracle._load()
    oracle._lib = mutant
    failures = []
    try:
        for check in P.ALL_FAST_PINS:
            try:
                check()
            except AssertionError:
                failures.append(check.__name__)
    finally:
        oracle._lib = saved
    assert failures, "no pin caught mutant " + name
