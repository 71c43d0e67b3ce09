"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies the oracle's C source, applies one plausible slip (a dropped
term, a wrong sign, a wrong index, a swapped order), builds the copy with gcc
into a temporary directory and runs every pin against it.  At least one pin
must fail.  The real oracle is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle_pins
from oracle import Oracle
from oracle import build_oracle

MUTANTS = {
    "y_reads_old_state": (
        "S[n] = a * S[n] + d * Bt_[n] * xv;\n                            acc += S[n] * Ct_[n];",
        "acc += S[n] * Ct_[n];\n                            S[n] = a * S[n] + d * Bt_[n] * xv;"),
    "scan_drops_skip_D": ("y[((b * L + t) * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);",
                          "y[((b * L + t) * H + h) * P + p] = acc;"),
    "scan_decay_sign": ("const double a = exp(d * A[h]);\n                        double acc",
                        "const double a = exp(-d * A[h]);\n                        double acc"),
    "scan_group_index": ("const int g = h / heads_per_group;\n                    for (int n = 0; n < N; ++n)\n"
                         "                        S[n] = init",
                         "const int g = h % G;\n                    for (int n = 0; n < N; ++n)\n"
                         "                        S[n] = init"),
    "scan_drops_dt_on_B": ("S[n] = a * S[n] + d * Bt_[n] * xv;", "S[n] = a * S[n] + Bt_[n] * xv;"),
    "scan_B_C_swapped": ("acc += S[n] * Ct_[n];", "acc += S[n] * Bt_[n];"),
    "scan_init_transposed": ("S[n] = init ? init[(((b * H) + h) * P + p) * N + n] : 0.0;",
                             "S[n] = init ? init[(((b * H) + h) * N + n) * P + p] : 0.0;"),
    "scan_dt_index": ("const double d = dt[(b * L + t) * H + h];",
                      "const double d = dt[(b * L + t) * H + (h + 1) % H];"),
    "conv_taps_reversed": ("acc += w[c * K + k] * conv_ext(u, s_in, L, CD, K, b, t - (K - 1) + k, c);",
                           "acc += w[c * K + (K - 1 - k)] * conv_ext(u, s_in, L, CD, K, b, t - (K - 1) + k, c);"),
    "conv_halo_off_by_one": ("return s_in[(b * CD + c) * K + (K + tau)];",
                             "return s_in[(b * CD + c) * K + (K - 1 + tau)];"),
    "conv_drops_bias": ("double acc = bias ? bias[c] : 0.0;\n                for",
                        "double acc = 0.0;\n                for"),
    "conv_state_window_shift": ("conv_ext(u, s_in, L, CD, K, b, L - K + k, c);",
                                "conv_ext(u, s_in, L, CD, K, b, L - K + k - 1, c);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "update_roll_wrong_way": ("for (int k = 0; k + 1 < K; ++k) sc[k] = sc[k + 1];\n            sc[K - 1] = u[b * CD + c];",
                              "for (int k = K - 1; k > 0; --k) sc[k] = sc[k - 1];\n            sc[0] = u[b * CD + c];"),
    "state_update_reads_old_state": (
        "S[n] = a * S[n] + d * Bv[n] * xv;\n                    acc += S[n] * Cv[n];",
        "acc += S[n] * Cv[n];\n                    S[n] = a * S[n] + d * Bv[n] * xv;"),
    "state_update_group_index": ("const int g = h / heads_per_group;\n                const double d = dt[b * H + h];",
                                 "const int g = h % G;\n                const double d = dt[b * H + h];"),
}


@pytest.fixture(scope="module")
def src():
    with open(build_oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(src, name):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        csrc = os.path.join(d, "mut.c")
        lib = os.path.join(d, "libmut.so")
        with open(csrc, "w") as f:
            f.write(mutated)
        build_oracle.build(csrc, lib)
        orc = Oracle(lib)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(orc)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmodified_copy_passes(src):
    """Control: the same build route with no mutation passes every pin."""
    with tempfile.TemporaryDirectory() as d:
        csrc = os.path.join(d, "same.c")
        lib = os.path.join(d, "libsame.so")
        with open(csrc, "w") as f:
            f.write(src)
        build_oracle.build(csrc, lib)
        orc = Oracle(lib)
        for pin in oracle_pins.ALL_PINS:
            pin(orc)
