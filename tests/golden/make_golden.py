"""Writes config0_oracle_y.txt: sampled oracle outputs of the tiny fp32 workload.

Calls only the oracle and the input generator. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssmgen  # noqa: E402

cfg = ssmgen.CONFIGS[0]
y = oracle.scan_inputs(ssmgen.make_inputs(cfg), cfg)
out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config0_oracle_y.txt")
with open(out, "w") as f:
    f.write("# oracle y of the tiny fp32 workload (batch 1, 64 channels, N 16, L 256)\n")
    f.write("# written by tests/golden/make_golden.py; columns: b d t y (float.hex)\n")
    for d in (0, 1, 31, 63):
        for t in (0, 1, 2, 127, 255):
            f.write(f"0 {d} {t} {float(y[0, d, t]).hex()}\n")
print("wrote", out)
