"""Writes c0_oracle_samples.txt from the oracle (regression lock).

Calls only oracle/ and workloads/. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

SAMPLES = [(0, 0, 0, 0), (0, 1, 5, 7), (1, 3, 15, 15), (1, 2, 8, 0), (0, 3, 3, 12)]


def main():
    cfg = wl.CONFIGS["c0"]
    inp = wl.layer_inputs(cfg, "f32")
    y = oracle.spectral_conv2d(inp["x64"], inp["w64"], *cfg.modes)
    with open(os.path.join(HERE, "c0_oracle_samples.txt"), "w") as f:
        f.write("# oracle y[b, o, h, w] on the 16x16 fp32 workload, seed 0 (regression lock)\n")
        for (b, o, h, w) in SAMPLES:
            f.write(f"{b} {o} {h} {w} {y[b, o, h, w]:.17e}\n")


if __name__ == "__main__":
    main()
