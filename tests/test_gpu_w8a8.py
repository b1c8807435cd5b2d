"""GPU parity of the W8A8 path (fp8 weights with block-quantised activations
on gfx950's block-scaled fp8 MFMA) against the oracle's W8A8 reading: every
weight GEMM's activation operand quantised in runs of 32 consecutive k with
a power-of-two scale per run, the norm-fed GEMMs on h * gain with 1/rms and
the Ada shift applied after the product.

Bar: rel-L2 <= 5e-2, the fp8 bar of the other fp8 tests.  The GPU quantises
activations it computed in fp32 and rounded to bf16, the oracle the exact
fp64 values, so codes near a rounding boundary can differ by one E4M3 step;
the comparison is over the same dequantised weights.
"""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check, run_denoiser

pytestmark = pytest.mark.gpu

FP8_BAR = 5e-2


def _small(**kw):
    # 20 robots x 14 suffix rows = 280 rows: ragged 64- and 128-row tiles;
    # K of 256 / 128 / 512: two, one and four 128-k stages
    base = S.workload("tiny_fp32").replace(
        name="small_w8a8", seed=17, d_model=256, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=64,
        d_mlp=512, time_dim=256, chunk=13, state_dim=32, batch=20, prefix_static=45, prefix_len=45,
        weight_dtype="fp8", act_dtype="bf16", w8a8=True)
    return base.replace(**kw)


def _inputs(cfg):
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    return W, k, v, S.make_noise(cfg), S.make_state(cfg)


@pytest.mark.parametrize("name,kw", [
    ("rms with state", dict()),
    ("ada, no state", dict(norm="ada", time_dim=64, state_dim=0, batch=22)),          # 286 rows
    ("longer k", dict(d_model=512, time_dim=512, d_mlp=1024, n_q_heads=4, head_dim=64, batch=19)),
    ("many tiles", dict(batch=40, chunk=20, prefix_static=70, prefix_len=61)),          # 840 rows
])
def test_w8a8_small_against_oracle(name, kw):
    cfg = _small(**kw)
    announce(f"w8a8 {name}: {kw}")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    ref = O.denoise(cfg, W, k, v, x0, st)
    check(f"w8a8 {name}", got, ref, FP8_BAR)


def test_w8a8_differs_from_w8a16_by_activation_rounding_only():
    # the same weights through both fp8 paths: close, and not identical
    cfg = _small()
    W, k, v, x0, st = _inputs(cfg)
    a = run_denoiser(cfg, W, k, v, x0, st)[0]
    b = run_denoiser(cfg.replace(w8a8=False), W, k, v, x0, st)[0]
    rel = O.rel_l2(a, b)
    announce(f"w8a8 vs w8a16 rel_l2 {rel:.3e}")
    assert 1e-4 < rel < FP8_BAR


def test_w8a8_runs_are_bitwise_repeatable():
    cfg = _small()
    W, k, v, x0, st = _inputs(cfg)
    outs = run_denoiser(cfg, W, k, v, x0, st, repeat=3)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_w8a8_pi0_shape_two_layers():
    # the Pi0 expert's widths (K = 1024, 2048, 4096) with 6 robots (306 rows)
    cfg = S.workload("pi0_1view").replace(name="pi0_w8a8_2l", n_layers=2, batch=6, weight_dtype="fp8",
                                          w8a8=True)
    announce("w8a8 pi0 shape, 2 layers, 6 robots")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    ref = O.denoise(cfg, W, k, v, x0, st)
    check("w8a8 pi0 2 layers", got, ref, FP8_BAR)


def test_w8a8_pi05_ada_b16_sampled_robots():
    # the batched-robot workload at full size, first and last robot
    cfg = S.workload("pi05_ada_b16").replace(weight_dtype="fp8", w8a8=True)
    announce("w8a8 pi05_ada_b16: generating")
    W, k, v, x0, st = _inputs(cfg)
    announce("w8a8 pi05_ada_b16: gpu")
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    robots = [0, cfg.batch - 1]
    ref = O.denoise(cfg, W, k, v, x0, st, robots=robots)
    check("w8a8 pi05_ada_b16 robots 0, 15", got[robots], ref, FP8_BAR)


def _draw_w8a8(seed):
    """A batched W8A8 configuration of 256-1024 rows: widths in multiples of
    128, one or two 128-k stages per layer GEMM and more, ragged row tiles."""
    g = np.random.default_rng(7000 + seed)
    hd = int(g.choice([64, 128]))
    hkv = int(g.choice([1, 2]))
    hq = hkv * int(g.choice([1, 2, 4]))
    while (hq * hd) % 128 or ((hq + 2 * hkv) * hd) % 128:
        hq += hkv
    state = int(g.choice([0, 32]))
    chunk = int(g.integers(16, 64))
    per = chunk + (state > 0)
    d = int(g.choice([128, 256, 512]))
    kw = dict(seed=seed, head_dim=hd, n_kv_heads=hkv, n_q_heads=hq, d_model=d, time_dim=d,
              d_mlp=int(g.choice([256, 384, 512])), n_layers=int(g.integers(1, 3)), chunk=chunk,
              batch=int(g.integers(-(-256 // per), 1024 // per + 1)), state_dim=state,
              n_steps=int(g.integers(1, 5)), sampler=str(g.choice(["euler", "heun", "ab2"])))
    cap = int(g.integers(0, 300))
    kw.update(prefix_static=cap, prefix_len=int(g.integers(0, cap + 1)))
    if g.random() < 0.4:
        kw.update(norm="ada", time_dim=32)
    if state and g.random() < 0.3:
        kw["state_causal"] = True
    if g.random() < 0.3:
        kw["rope_theta"] = 10000.0
    elif g.random() < 0.3:
        kw["kv_fp8"] = True
    return _small(name=f"w8a8sweep{seed}", **kw)


@pytest.mark.parametrize("seed", range(12))
def test_w8a8_rows_sweep(seed):
    cfg = _draw_w8a8(seed)
    rows = cfg.batch * cfg.suffix
    assert 256 <= rows <= 1024
    announce(f"w8a8 sweep {seed}: {rows} rows, batch {cfg.batch}, d {cfg.d_model}, mlp {cfg.d_mlp}, "
             f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}, layers {cfg.n_layers}, {cfg.norm}, "
             f"{cfg.sampler}, causal {cfg.state_causal}, rope {cfg.rope_theta}, kv8 {cfg.kv_fp8}")
    W, k, v, x0, st = _inputs(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    check(f"w8a8 sweep {seed}", got, O.denoise(cfg, W, k, v, x0, st), FP8_BAR)
