"""Regression guard: the oracle still produces the stored tiny-workload actions."""
import os

import numpy as np

import fm_synth as S
import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_actions_unchanged():
    cfg = S.workload("tiny_fp32")
    ref = np.loadtxt(os.path.join(HERE, "tiny_fp32_actions.txt")).reshape(1, cfg.chunk, cfg.action_dim)
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    got = O.denoise(cfg, W, k, v, S.make_noise(cfg), S.make_state(cfg))
    assert np.max(np.abs(got - ref)) < 1e-12
