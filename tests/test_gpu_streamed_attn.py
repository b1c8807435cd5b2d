"""GPU parity of the streamed attention kernel (fm_config.attn_kernel =
FM_ATTN_STREAMED): workgroups of 128 query rows of one (robot, kv head),
32-key chunks of K and V through LDS, an online softmax per row, key ranges
merged by the last workgroup to arrive.  Every case runs the whole loop
through the C ABI with the kernel forced and compares with the fp64 oracle
at the bars of the other bf16 / fp8 tests; ring contexts must still equal a
full-cache recompute bit for bit.
"""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check, run_denoiser, small_cfg

pytestmark = pytest.mark.gpu


def _inputs(cfg):
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    return W, k, v, S.make_noise(cfg), S.make_state(cfg)


@pytest.mark.parametrize("kw", [
    dict(),                                                   # 56 query rows: one group, two waves past the rows
    dict(head_dim=32),
    dict(head_dim=128, prefix_static=300, prefix_len=300),    # two key ranges
    dict(head_dim=256, n_q_heads=2, prefix_static=600, prefix_len=200),  # four ranges, the last two fully masked
    dict(batch=5, chunk=20, n_q_heads=4, n_kv_heads=2, prefix_static=150, prefix_len=150),  # two kv heads
    dict(prefix_static=1100, prefix_len=1100, chunk=9),       # more than 1024 keys, four ranges of 9 chunks
    dict(batch=3, chunk=7, state_dim=0, prefix_static=0, prefix_len=0),  # no prefix: one chunk of suffix keys
    dict(batch=12, chunk=30, prefix_static=150, prefix_len=150),  # 372 rows: the batched GEMMs around it
    dict(batch=20, chunk=60, n_q_heads=8, head_dim=32, prefix_static=100, prefix_len=100),  # 12 query groups
    dict(state_causal=True),                                  # block-causal state row
    dict(state_causal=True, head_dim=128, prefix_static=300, prefix_len=260),  # block-causal with key ranges
    dict(norm="ada", time_dim=32, state_dim=0),
    dict(rope_theta=10000.0, prefix_static=300, prefix_len=280),
])
def test_streamed_small(kw):
    cfg = small_cfg(attn_kernel="streamed", **kw)
    announce(f"streamed {kw}")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    check(f"streamed {kw}", got, O.denoise(cfg, W, k, v, x0, st), 1e-2, 3e-2)


def test_streamed_fp8_weights():
    cfg = small_cfg(attn_kernel="streamed", weight_dtype="fp8", head_dim=128, prefix_static=300, prefix_len=300)
    announce("streamed fp8 weights")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    check("streamed fp8 weights", got, O.denoise(cfg, W, k, v, x0, st), 5e-2)


def test_streamed_w8a8_writes_the_o_operand():
    # W8A8: the streamed kernel stores the O projection's fp8 operand
    cfg = S.workload("tiny_fp32").replace(
        name="streamed_w8a8", seed=17, d_model=256, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=64,
        d_mlp=512, time_dim=256, chunk=13, state_dim=32, batch=20, prefix_static=300, prefix_len=290,
        weight_dtype="fp8", act_dtype="bf16", w8a8=True, attn_kernel="streamed")
    announce("streamed w8a8")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    check("streamed w8a8", got, O.denoise(cfg, W, k, v, x0, st), 5e-2)


def test_streamed_runs_are_bitwise_repeatable_with_key_ranges():
    cfg = small_cfg(attn_kernel="streamed", head_dim=256, n_q_heads=2, prefix_static=600, prefix_len=590)
    W, k, v, x0, st = _inputs(cfg)
    a, b, c = run_denoiser(cfg, W, k, v, x0, st, repeat=3)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_streamed_and_register_kernels_agree():
    W = k = v = None
    outs = {}
    for kern in ("register", "streamed"):
        cfg = small_cfg(attn_kernel=kern, head_dim=128, prefix_static=300, prefix_len=300, batch=3)
        if W is None:
            W, k, v, x0, st = _inputs(cfg)
        outs[kern] = run_denoiser(cfg, W, k, v, x0, st)[0]
    check("streamed vs register", outs["streamed"], outs["register"].astype(np.float64), 1e-2, 3e-2)


def test_streamed_ring_equals_recompute_with_key_ranges():
    from test_gpu_parity import _ring_run
    cfg = small_cfg(name="small_ring_streamed", attn_kernel="streamed", head_dim=128, prefix_static=20,
                    frame_tokens=192, n_frames=3, prefix_len=596)
    _ring_run(cfg, ticks=5, oracle_ticks={4})


def test_streamed_full_pi0_1view():
    cfg = S.workload("pi0_1view").replace(attn_kernel="streamed")
    announce("pi0_1view streamed: generating")
    W, k, v, x0, st = _inputs(cfg)
    announce("pi0_1view streamed: gpu")
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    announce("pi0_1view streamed: oracle")
    check("pi0_1view streamed", got, O.denoise(cfg, W, k, v, x0, st), 1e-2, 3e-2)
