"""GPU parity over a seeded sweep of small configurations: shapes, head
layouts, prefix lengths, samplers, schedules and options drawn together, so
that combinations no hand-written case names are exercised too.  Each case is
compared with the fp64 oracle at the bar of its dtype (bf16: rel-L2 1e-2,
max-abs 3e-2; fp32: 1e-4)."""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check, run_denoiser, small_cfg

pytestmark = pytest.mark.gpu


def _draw(seed):
    g = np.random.default_rng(1000 + seed)
    hd = int(g.choice([32, 64, 128, 256]))
    hkv = int(g.choice([1, 2]))
    hq = hkv * int(g.choice([1, 2, 4, 8]))
    while (hq * hd) % 32 or hq * hd > 2048:
        hq //= 2
    kw = dict(seed=seed, head_dim=hd, n_kv_heads=hkv, n_q_heads=max(hq, hkv),
              d_model=int(g.choice([64, 128, 192, 256])), d_mlp=int(g.choice([128, 256, 384])),
              n_layers=int(g.integers(1, 4)), chunk=int(g.integers(1, 40)), batch=int(g.integers(1, 13)),
              state_dim=int(g.choice([0, 32])), n_steps=int(g.integers(1, 7)),
              action_dim=int(g.choice([16, 32])))
    kw["time_dim"] = kw["d_model"]
    ring = g.random() < 0.25
    if ring:
        kw.update(prefix_static=int(g.integers(0, 40)), frame_tokens=32, n_frames=int(g.integers(1, 4)))
        kw["prefix_len"] = kw["prefix_static"] + kw["frame_tokens"] * kw["n_frames"]
    else:
        cap = int(g.integers(0, 400))
        kw.update(prefix_static=cap, prefix_len=int(g.integers(0, cap + 1)))
    if g.random() < 0.3:
        kw.update(norm="ada", time_dim=int(g.choice([16, 32])))
    kw["sampler"] = str(g.choice(["euler", "heun", "ab2"]))
    if g.random() < 0.3 and kw["n_steps"] > 1:
        u = np.linspace(0, 1, kw["n_steps"] + 1)
        kw["t_schedule"] = tuple(float(np.float32(x)) for x in (1 - u) / (1 + 2 * u))  # shifted, ends 1 -> 0
    if kw["state_dim"] and g.random() < 0.4:
        kw["state_causal"] = True
    keys = (kw["prefix_static"] + 31) // 32 * 32 + kw.get("frame_tokens", 0) * kw.get("n_frames", 0) + \
        (kw["chunk"] + (kw["state_dim"] > 0) + 31) // 32 * 32
    if g.random() < 0.25 and keys <= 1024:
        kw["kv_fp8"] = True
    if not ring and g.random() < 0.3:
        kw["rope_theta"] = float(g.choice([100.0, 10000.0]))
    if g.random() < 0.15 and not kw.get("kv_fp8") and kw["d_model"] % 64 == 0 and kw["d_mlp"] % 64 == 0 \
            and (kw["n_q_heads"] * hd) % 64 == 0:
        kw["weight_dtype"] = "fp8"
    return small_cfg(name=f"sweep{seed}", **kw)


@pytest.mark.parametrize("seed", range(64))
def test_sweep(seed):
    cfg = _draw(seed)
    desc = {k: getattr(cfg, k) for k in ("batch", "chunk", "state_dim", "d_model", "n_layers", "n_q_heads", "n_kv_heads",
                                         "head_dim", "d_mlp", "prefix_static", "prefix_len", "n_frames", "norm",
                                         "sampler", "n_steps", "state_causal", "kv_fp8", "weight_dtype", "rope_theta")}
    desc["schedule"] = cfg.t_schedule is not None
    announce(f"sweep {seed}: {desc}")
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    tol = 5e-2 if cfg.weight_dtype == "fp8" else 1e-2
    check(f"sweep {seed}", got, O.denoise(cfg, W, k, v, x0, st), tol, None if cfg.weight_dtype == "fp8" else 3e-2)


def _draw_rows(seed):
    """Batched configurations of 256-1024 rows: the LDS-staged GEMMs (mid and
    large tile plans, ragged last row tiles), bf16 or fp8 weights."""
    g = np.random.default_rng(3000 + seed)
    hd = int(g.choice([64, 128, 256]))
    hkv = int(g.choice([1, 2]))
    hq = hkv * int(g.choice([1, 2, 4]))
    while hq * hd > 1024:
        hq //= 2
    state = int(g.choice([0, 32]))
    chunk = int(g.integers(24, 64))
    per = chunk + (state > 0)
    kw = dict(seed=seed, head_dim=hd, n_kv_heads=hkv, n_q_heads=max(hq, hkv), d_model=int(g.choice([128, 256])),
              d_mlp=int(g.choice([256, 320, 512])), n_layers=int(g.integers(1, 3)), chunk=chunk,
              batch=int(g.integers(-(-256 // per), 17)), state_dim=state, n_steps=int(g.integers(1, 5)),
              action_dim=32)
    kw["time_dim"] = kw["d_model"]
    cap = int(g.integers(0, 300))
    kw.update(prefix_static=cap, prefix_len=int(g.integers(0, cap + 1)))
    if g.random() < 0.3:
        kw.update(norm="ada", time_dim=32)
    kw["sampler"] = str(g.choice(["euler", "heun", "ab2"]))
    if state and g.random() < 0.3:
        kw["state_causal"] = True
    if g.random() < 0.3:
        kw["rope_theta"] = 10000.0
    if g.random() < 0.5:
        kw["weight_dtype"] = "fp8"
    elif g.random() < 0.3:
        kw["kv_fp8"] = True
    return small_cfg(name=f"rowsweep{seed}", **kw)


@pytest.mark.parametrize("seed", range(24))
def test_rows_sweep(seed):
    cfg = _draw_rows(seed)
    rows = cfg.batch * (cfg.chunk + (cfg.state_dim > 0))
    assert 256 <= rows <= 1024
    announce(f"rows sweep {seed}: {rows} rows, batch {cfg.batch}, d {cfg.d_model}, mlp {cfg.d_mlp}, "
             f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}, {cfg.weight_dtype}, kv8 {cfg.kv_fp8}, "
             f"{cfg.norm}, {cfg.sampler}, causal {cfg.state_causal}, rope {cfg.rope_theta}")
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    got = run_denoiser(cfg, W, k, v, x0, st)[0]
    fp8 = cfg.weight_dtype == "fp8"
    check(f"rows sweep {seed}", got, O.denoise(cfg, W, k, v, x0, st), 5e-2 if fp8 else 1e-2, None if fp8 else 3e-2)


def _draw_encoder(seed):
    g = np.random.default_rng(5000 + seed)
    hd = int(g.choice([32, 64, 128, 256]))
    hkv = int(g.choice([1, 2]))
    kw = dict(seed=seed, head_dim=hd, n_kv_heads=hkv, n_q_heads=hkv * int(g.choice([1, 2, 4])),
              d_model=int(g.choice([64, 128, 256])), d_mlp=int(g.choice([128, 256])), n_layers=int(g.integers(1, 4)))
    kw["time_dim"] = kw["d_model"]
    if g.random() < 0.3:
        kw["rope_theta"] = 10000.0
    if g.random() < 0.2 and (kw["n_q_heads"] * hd) % 64 == 0:
        kw["weight_dtype"] = "fp8"
    return small_cfg(name=f"encsweep{seed}", **kw), int(g.integers(1, 300)), int(g.integers(1, 5))


@pytest.mark.parametrize("seed", range(16))
def test_encoder_sweep(seed):
    import torch
    import flow_matching_denoising_euler_amd as fm
    cfg, n_tok, n_seq = _draw_encoder(seed)
    cfg = cfg.replace(batch=n_seq)
    announce(f"encoder sweep {seed}: {n_seq} x {n_tok} tokens, d {cfg.d_model}, {cfg.n_layers} layers, "
             f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}, {cfg.weight_dtype}, rope {cfg.rope_theta}")
    Wp, tokens = S.make_prefix_stack(cfg, n_tok)
    enc = fm.Encoder(cfg, Wp, n_tokens=n_tok, n_seqs=n_seq)
    try:
        k, v = enc.encode(tokens)
        torch.cuda.synchronize()
        k, v = k.float().cpu().numpy(), v.float().cpu().numpy()
    finally:
        enc.close()
    W64 = O.effective_weights(cfg, {"layers": Wp["layers"]})
    kr, vr = zip(*[O.prefix_stack_kv(cfg, W64, tokens[b]) for b in range(n_seq)])
    tol = 5e-2 if cfg.weight_dtype == "fp8" else 1e-2
    for name, got, ref in (("K", k, np.stack(kr)), ("V", v, np.stack(vr))):
        rel = O.rel_l2(got, ref)
        announce(f"  {name}: rel_l2 {rel:.3e}")
        assert np.all(np.isfinite(got)) and rel <= tol, (name, rel)
