"""Stored expected values stay what the oracle computes: the benchmark's guard
file (tests/golden/decode_32k_step_seed0.txt, written by
tests/golden/make_decode_32k_step.py from the oracle alone) is regenerated and
compared."""
import importlib.util
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(path):
    return np.array([list(map(float, line.split())) for line in open(path)
                     if line.strip() and not line.startswith("#")], dtype=np.float64)


def test_decode_step_guard_file_matches_the_oracle(tmp_path):
    stored = _read(os.path.join(GOLDEN, "decode_32k_step_seed0.txt"))
    assert stored.shape == (32, 128)
    spec = importlib.util.spec_from_file_location("make_decode_32k_step",
                                                  os.path.join(GOLDEN, "make_decode_32k_step.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    m.OUT = str(tmp_path / "fresh.txt")
    m.main()
    np.testing.assert_allclose(_read(m.OUT), stored, rtol=2e-9, atol=1e-12)
