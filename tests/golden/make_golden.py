"""Writes the stored oracle outputs under tests/golden/.

Calls only the fp64 oracle and the seeded input generators; run it again
only when a change to the oracle's arithmetic is justified by the pages.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import fm_synth as S  # noqa: E402
import oracle as O  # noqa: E402


def tiny_actions():
    cfg = S.workload("tiny_fp32")
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    return O.denoise(cfg, W, k, v, S.make_noise(cfg), S.make_state(cfg))


def main():
    y = tiny_actions()
    path = os.path.join(HERE, "tiny_fp32_actions.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle actions (x at t=0) of the tiny fp32 workload:\n")
        f.write("# d=64, 2 layers, 4x16 heads, MLP 256, chunk 8 + state token, prefix 32,\n")
        f.write("# 10 Euler steps, seed 0.  Written by tests/golden/make_golden.py.\n")
        np.savetxt(f, y.reshape(-1, y.shape[-1]), fmt="%.17g")
    print("wrote", path)


if __name__ == "__main__":
    main()
