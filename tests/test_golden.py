"""Regression lock of the oracle on the 16x16 workload (see tests/golden)."""
import os

import numpy as np

import oracle
import workloads as wl

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_regression_lock():
    cfg = wl.CONFIGS["c0"]
    inp = wl.layer_inputs(cfg, "f32")
    y = oracle.spectral_conv2d(inp["x64"], inp["w64"], *cfg.modes)
    rows = [l.split() for l in open(os.path.join(HERE, "c0_oracle_samples.txt"))
            if not l.startswith("#")]
    assert rows
    for r in rows:
        b, o, h, w = map(int, r[:4])
        assert abs(y[b, o, h, w] - float(r[4])) <= 1e-14 * max(1.0, abs(float(r[4])))
