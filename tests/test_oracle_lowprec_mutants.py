"""Planted mistakes in the oracle's element-to-random-number mapping of the 16-bit state forms must
be caught by the pins of test_oracle_lowprec.py (CPU only).

Each case copies oracle/oracle.py as text, applies one plausible slip and loads the copy as a module
of the oracle package; the pins then run against it.  The real oracle is never modified.
"""
import importlib.util
import os
import sys

import pytest

import test_oracle_lowprec as pins
from oracle import build_oracle

SRC = os.path.join(os.path.dirname(build_oracle.__file__), "oracle.py")
ANCHOR = "e = s * H * P * N + np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)"
MUTANTS = {
    "counter_from_batch_position": "e = b * H * P * N + np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)",
    "counter_one_block_off": "e = s * H * P * N + 8 + np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)",
    "counter_ignores_slot": "e = np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)",
    "counter_head_major_pool": "e = s * P * N + np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)",
}
PINS = [pins.test_lp_codes_follow_the_slot_not_the_batch_position, pins.test_lp_codes_depend_on_the_flat_pool_index,
        pins.test_lp_codes_absolute_index_on_a_tiny_pool]


def load_variant(name, text):
    spec = importlib.util.spec_from_loader("oracle._variant_" + name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    exec(compile(text, SRC + ":" + name, "exec"), mod.__dict__)
    return mod.Oracle(build_oracle.LIB)


@pytest.fixture(scope="module")
def src():
    if not os.path.exists(build_oracle.LIB):
        build_oracle.build()
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mapping_mutant_is_caught(src, name):
    assert src.count(ANCHOR) == 1
    orc = load_variant(name, src.replace(ANCHOR, MUTANTS[name]))
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"


def test_unmodified_copy_passes(src):
    orc = load_variant("same", src)
    for pin in PINS:
        pin(orc)
