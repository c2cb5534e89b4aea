"""Pins for the CPU oracle (no GPU).

The pin functions live in tests/oracle_pins.py.  The last tests plant
plausible mistakes in copies of the oracle's C source and assert that the
pins catch every one of them.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import parity_error
from oracle_pins import ALL_PINS, MUTANTS, _run_pins, pin_worked_2x2
from roofline_driven_optimisation_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


# ---------------------------------------------------------------------------
# the tests
# ---------------------------------------------------------------------------

def test_worked_2x2(orc, golden):
    pin_worked_2x2(orc, golden("worked_2x2.txt"))


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_argument_errors(orc):
    lib = orc.lib
    assert lib.oracle_gemm_f32(-1, 1, 1, 1.0, 0.0, None, None, None, None, None) != 0
    assert lib.oracle_gemm_f32(1, 1, 1, 1.0, 0.0, None, None, None, None, None) != 0
    # an empty output with K = 0 needs no pointer at all
    assert lib.oracle_gemm_f32(0, 4, 0, 1.0, 0.0, None, None, None, None, None) == 0
    # B is still required when K*N > 0, even with M = 0
    assert lib.oracle_gemm_f32(0, 4, 4, 1.0, 0.0, None, None, None, None, None) != 0
    with pytest.raises(ValueError):
        orc.gemm_entries(np.ones((2, 2), np.float32), np.ones((2, 2), np.float32), [2], [0])
    with pytest.raises(ValueError):
        orc.gemm(np.ones((2, 3), np.float32), np.ones((2, 2), np.float32))


def test_parity_error_helper():
    ref = np.array([1.0, 2.0])
    den = np.array([1.0, 1.0])
    assert parity_error(np.array([1.0, 2.5], np.float32), ref, den) == 0.5
    assert parity_error(np.array([np.nan, 2.0], np.float32), ref, den) == float("inf")


def test_bf16_rounding_matches_torch():
    """Our round-to-nearest-even bf16 conversion equals torch's cast."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.normal(size=100000).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -1.0 - 2 ** -8, 65504.0, 1e-40, 0.0, -0.0],
                 dtype=np.float32),
        # exact ties at the bf16 midpoint: both tie directions
        (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32),
    ])
    ours = f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail at least one pin
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[mutant]
    assert src.count(old) >= 1, "mutation anchor not found: %r" % old
    cfile = tmp_path / ("oracle_%s.c" % mutant)
    cfile.write_text(src.replace(old, new, 1))
    lib = oracle.compile_library(str(cfile), str(tmp_path / ("lib_%s.so" % mutant)))
    proc, failures = _pins_in_child(lib)
    if failures is None:
        # only a crash by signal (e.g. an out-of-bounds read) counts as caught
        assert proc.returncode < 0, proc.stdout + proc.stderr
        return
    assert failures, "planted mistake %r passed every pin" % mutant


def _pins_in_child(lib):
    """Run every pin against ``lib`` in a fresh interpreter (a mutant may
    crash, and libgomp does not survive fork())."""
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; "
            "oracle_pins.main(%r, %r)" % (HERE, ROOT, lib, os.path.join(HERE, "golden", "worked_2x2.txt")))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, env=env)
    line = [l for l in proc.stdout.splitlines() if l.startswith("PIN_FAILURES ")]
    if not line:
        return proc, None
    return proc, json.loads(line[-1][len("PIN_FAILURES "):])


def test_child_harness_runs_clean_oracle():
    """The child harness itself works: the real oracle passes every pin there."""
    proc, failures = _pins_in_child(oracle.build(force=False))
    assert proc.returncode == 0, proc.stderr
    assert failures == []


def test_unmutated_passes_all(golden):
    assert _run_pins(oracle.default(), golden("worked_2x2.txt")) == []
