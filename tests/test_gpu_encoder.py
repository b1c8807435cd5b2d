"""GPU parity of the prefix encoder (fm_encoder_create / fm_encode_prefix)
against the oracle's prefix stack, and the encoder feeding the denoiser.

Tolerances: fp32 rel-L2 <= 1e-4; bf16 K/V rel-L2 <= 1e-2 and max-abs <=
1e-2 of the largest reference magnitude (the outputs are themselves bf16,
whose rounding is relative); fp8 weights rel-L2 <= 5e-2 against the oracle
on the same dequantised weights.  Denoised actions keep the loop's bars.
"""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check, small_cfg

pytestmark = pytest.mark.gpu


def _prefix_weights(cfg, Wp):
    """The prefix stack as the encoder uses it: fp8 matrices dequantised."""
    return O.effective_weights(cfg, {"layers": Wp["layers"]})


def _oracle_kv(cfg, Wp, tokens):
    """[seqs][layers][T][Hkv][Dh] K and V, one oracle prefix stack per sequence."""
    W64 = _prefix_weights(cfg, Wp)
    ks, vs = zip(*[O.prefix_stack_kv(cfg, W64, tokens[b]) for b in range(tokens.shape[0])])
    return np.stack(ks), np.stack(vs)


def _encode(cfg, Wp, tokens):
    import torch
    import flow_matching_denoising_euler_amd as fm
    enc = fm.Encoder(cfg, Wp, n_tokens=tokens.shape[1], n_seqs=tokens.shape[0])
    try:
        k, v = enc.encode(tokens)
        torch.cuda.synchronize()
        return k.float().cpu().numpy(), v.float().cpu().numpy()
    finally:
        enc.close()


def _check_kv(name, got, ref, dtype):
    rel = O.rel_l2(got, ref)
    mab = O.max_abs(got, ref)
    scale = float(np.max(np.abs(ref)))
    announce(f"{name}: rel_l2 {rel:.3e} max_abs {mab:.3e} (max |ref| {scale:.2f})")
    assert np.all(np.isfinite(got)), name
    tol = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}[dtype]
    assert rel <= tol, (name, rel)
    if dtype == "bf16":
        assert mab <= 1e-2 * scale, (name, mab, scale)


def _wdtype(cfg):
    return "f32" if cfg.act_dtype == "f32" else ("fp8" if cfg.weight_dtype == "fp8" else "bf16")


# --- K/V of the stack, element by element ----------------------------------------
@pytest.mark.parametrize("name,kw,n_tokens,n_seqs", [
    ("fp32", None, 40, 2),                                               # ragged tokens, 2 sequences
    ("bf16", dict(), 45, 2),                                             # one row tile
    ("bf16 2 kv heads", dict(n_q_heads=4, n_kv_heads=2, n_layers=3), 100, 3),  # 300 rows: large-M GEMMs
    ("bf16 head_dim 256", dict(n_q_heads=2, head_dim=256, d_mlp=512), 256, 1),  # one 256-token frame
    ("bf16 head_dim 128, long", dict(head_dim=128), 1000, 1),          # 1000 tokens, largest key tile
    ("fp8", dict(weight_dtype="fp8"), 64, 2),
    ("fp8 300 rows", dict(weight_dtype="fp8"), 150, 2),                 # fp8 weights, LDS-staged GEMMs, mid tiles
    ("fp8 600 rows", dict(weight_dtype="fp8", n_q_heads=4, n_kv_heads=2), 300, 2),  # large tiles
])
def test_encoder_kv_small(name, kw, n_tokens, n_seqs):
    cfg = S.workload("tiny_fp32") if kw is None else small_cfg(**kw)
    cfg = cfg.replace(batch=n_seqs)
    announce(f"encoder {name}: {n_seqs} x {n_tokens} tokens")
    Wp, tokens = S.make_prefix_stack(cfg, n_tokens)
    k, v = _encode(cfg, Wp, tokens)
    kr, vr = _oracle_kv(cfg, Wp, tokens)
    assert k.shape == kr.shape == (n_seqs, cfg.n_layers, n_tokens, cfg.n_kv_heads, cfg.head_dim)
    _check_kv(f"encoder {name} K", k, kr, _wdtype(cfg))
    _check_kv(f"encoder {name} V", v, vr, _wdtype(cfg))


def test_encoder_first_layer_kv_is_one_projection():
    # layer 0's K and V depend on the tokens through one norm and one GEMM, so
    # every element is within the bf16 rounding of the GEMM operand (a sum of
    # d terms, each off by at most 2^-9 relative: a few 2^-9 rms) plus the
    # rounding of the output itself (2^-9 relative)
    cfg = small_cfg(batch=2)
    Wp, tokens = S.make_prefix_stack(cfg, 77)
    k, v = _encode(cfg, Wp, tokens)
    kr, vr = _oracle_kv(cfg, Wp, tokens)
    announce("encoder layer 0")
    for got, ref in ((k[:, 0], kr[:, 0]), (v[:, 0], vr[:, 0])):
        rms = float(np.sqrt(np.mean(ref ** 2)))
        assert np.all(np.abs(got - ref) <= 2 ** -6 * rms + 2 ** -8 * np.abs(ref))


def test_encoder_sequences_are_independent_and_deterministic():
    cfg = small_cfg(batch=3)
    Wp, tokens = S.make_prefix_stack(cfg, 50)
    announce("encoder independence")
    k, v = _encode(cfg, Wp, tokens)
    k2, v2 = _encode(cfg, Wp, tokens)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)
    k1, v1 = _encode(cfg.replace(batch=1), Wp, tokens[1:2].copy())
    assert np.array_equal(k[1:2], k1) and np.array_equal(v[1:2], v1)


def test_full_pi0_frame():
    # one 256-token frame through the Pi0-shaped stack (18 layers, width 1024)
    cfg = S.workload("pi0_1view").replace(batch=1)
    announce("encoder pi0 frame 256 tokens")
    Wp, tokens = S.make_prefix_stack(cfg, 256)
    k, v = _encode(cfg, Wp, tokens)
    kr, vr = _oracle_kv(cfg, Wp, tokens)
    _check_kv("pi0 frame K", k, kr, "bf16")
    _check_kv("pi0 frame V", v, vr, "bf16")


def test_full_pi0_stream_fp8_frame():
    cfg = S.workload("stream_fp8").replace(batch=1)
    announce("encoder pi0 fp8 frame 256 tokens")
    Wp, tokens = S.make_prefix_stack(cfg, 256)
    k, v = _encode(cfg, Wp, tokens)
    kr, vr = _oracle_kv(cfg, Wp, tokens)
    _check_kv("pi0 fp8 frame K", k, kr, "fp8")
    _check_kv("pi0 fp8 frame V", v, vr, "fp8")


# --- the encoder feeding the loop ---------------------------------------------------
def _run_with_encoded_prefix(cfg, W, Wp, tokens, x0, st):
    import torch
    import flow_matching_denoising_euler_amd as fm
    enc = fm.Encoder(cfg, Wp, n_tokens=tokens.shape[1], n_seqs=cfg.batch)
    den = fm.Denoiser(cfg, W)
    try:
        k, v = enc.encode(tokens)  # device buffers straight into the loop's prefix
        for b in range(cfg.batch):
            fm.fm_set_prefix_kv(den.ctx, b, k[b], v[b], tokens.shape[1])
        out = den.denoise(x0, st).cpu().numpy()
        torch.cuda.synchronize()
        return out
    finally:
        den.close()
        enc.close()


@pytest.mark.parametrize("name,kw", [("fp32", None), ("bf16", dict(prefix_static=45, prefix_len=45)),
                                     ("bf16 ada", dict(norm="ada", time_dim=32, state_dim=0)),
                                     ("bf16 rope", dict(rope_theta=10000.0)),
                                     ("bf16 rope fp8 cache", dict(rope_theta=500.0, kv_fp8=True)),
                                     # 2 x 300 prefix tokens: the encoder's GEMMs on the LDS-staged kernel
                                     # with fp8 weights (large plan), rotated K
                                     ("fp8 weights 600 rows rope", dict(weight_dtype="fp8", prefix_static=300,
                                                                        prefix_len=300, rope_theta=10000.0))])
def test_encoded_prefix_equals_joint_recompute(name, kw):
    # the cached-prefix loop fed by the GPU encoder against the oracle that
    # recomputes [prefix tokens | suffix] as one sequence at every step
    cfg = S.workload("tiny_fp32") if kw is None else small_cfg(**kw)
    W = S.make_weights(cfg)
    Wp, tokens = S.make_prefix_stack(cfg, cfg.prefix_static)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    announce(f"encoder -> loop {name}")
    got = _run_with_encoded_prefix(cfg, W, Wp, tokens, x0, st)
    # the joint recompute runs on the weights both contexts use: with fp8
    # weights the encoder's stack holds the dequantised E4M3 matrices too
    ref = O.denoise_joint(cfg, W, _prefix_weights(cfg, Wp), tokens, x0, st)
    if cfg.act_dtype == "f32":
        check(f"encoder -> loop {name}", got, ref, 1e-4)
    elif cfg.kv_fp8:  # the joint recompute holds no fp8 cache: the fp8 bar
        check(f"encoder -> loop {name}", got, ref, 5e-2)
    else:  # bf16, and fp8 weights against the same dequantised weights
        check(f"encoder -> loop {name}", got, ref, 1e-2, 3e-2)


def test_encoded_frames_stream_through_the_ring():
    # static prompt and frames encoded separately (a frame's K/V depends on the
    # frame alone), set, then one new frame encoded and appended per tick
    import torch
    import flow_matching_denoising_euler_amd as fm
    cfg = small_cfg(name="enc_ring", prefix_static=20, frame_tokens=32, n_frames=3, prefix_len=116, batch=1)
    W = S.make_weights(cfg)
    Wp, _ = S.make_prefix_stack(cfg, 1)
    g = np.random.default_rng(11)
    tok = lambda n: S.round_bf16(g.standard_normal((1, n, cfg.d_model))).astype(np.float32)
    prompt = tok(20)
    frames = [tok(32) for _ in range(5)]
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    announce("encoder ring: 3 frames, then 2 appends")
    penc = fm.Encoder(cfg, Wp, n_tokens=20, n_seqs=1)
    fenc = fm.Encoder(cfg, Wp, n_tokens=32, n_seqs=1)
    den = fm.Denoiser(cfg, W)
    try:
        kp, vp = penc.encode(prompt)
        kf, vf = zip(*[tuple(t.clone() for t in fenc.encode(f)) for f in frames[:3]])
        k0 = torch.cat([kp[0]] + [x[0] for x in kf], dim=1).contiguous()
        v0 = torch.cat([vp[0]] + [x[0] for x in vf], dim=1).contiguous()
        fm.fm_set_prefix_kv(den.ctx, 0, k0, v0, k0.shape[1])
        outs = [den.denoise(x0, st).cpu().numpy()]
        for f in frames[3:]:
            k, v = fenc.encode(f)
            fm.fm_append_prefix_kv(den.ctx, 0, k[0], v[0])
            outs.append(den.denoise(x0, st).cpu().numpy())
        torch.cuda.synchronize()
    finally:
        den.close()
        fenc.close()
        penc.close()
    W64 = _prefix_weights(cfg, Wp)
    okv = lambda t: O.prefix_stack_kv(cfg, W64, t[0])
    pk_, pv_ = okv(prompt)
    fkv = [okv(f) for f in frames]
    for tick, out in enumerate(outs):
        win = fkv[tick:tick + 3]
        kr = np.concatenate([pk_] + [k for k, _ in win], axis=1)[None]
        vr = np.concatenate([pv_] + [v for _, v in win], axis=1)[None]
        check(f"encoder ring tick {tick}", out, O.denoise(cfg, W, kr, vr, x0, st), 1e-2, 3e-2)


# --- the async pipeline: encode on its own stream, hand off on the device -----------
def _ring_inputs(batch=1):
    cfg = small_cfg(name="enc_pipe", prefix_static=20, frame_tokens=32, n_frames=3, prefix_len=116, batch=batch)
    W = S.make_weights(cfg)
    Wp, _ = S.make_prefix_stack(cfg, 1)
    g = np.random.default_rng(12)
    tok = lambda n: S.round_bf16(g.standard_normal((batch, n, cfg.d_model))).astype(np.float32)
    return cfg, W, Wp, tok(20), [tok(32) for _ in range(7)]


def _pipeline(cfg, W, Wp, prompt, frames, two_streams):
    """Set [prompt | frames 0..2], then per tick t: denoise, and encode frame
    t + 3 and append it.  two_streams: the encode runs on its own stream,
    overlapping the denoise, and reaches the ring through fm_append_encoded;
    otherwise everything is serial on one stream through caller buffers."""
    import torch
    import flow_matching_denoising_euler_amd as fm
    sD = torch.cuda.Stream()
    sE = torch.cuda.Stream() if two_streams else sD
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    outs = []
    with torch.cuda.stream(sD):
        den = fm.Denoiser(cfg, W, stream=sD)
        penc = fm.Encoder(cfg, Wp, n_tokens=20, n_seqs=cfg.batch, stream=sD)
    with torch.cuda.stream(sE):
        fenc = fm.Encoder(cfg, Wp, n_tokens=32, n_seqs=cfg.batch, stream=sE)
        ftok = [torch.from_numpy(f).cuda() for f in frames]
    torch.cuda.synchronize()
    try:
        with torch.cuda.stream(sE):
            kf, vf = zip(*[fenc.encode(f) for f in ftok[:3]])
        torch.cuda.synchronize()
        with torch.cuda.stream(sD):
            kp, vp = penc.encode(prompt)
            for b in range(cfg.batch):
                k0 = torch.cat([kp[b]] + [x[b] for x in kf], dim=1).contiguous()
                v0 = torch.cat([vp[b]] + [x[b] for x in vf], dim=1).contiguous()
                fm.fm_set_prefix_kv(den.ctx, b, k0, v0, k0.shape[1])
            noise = torch.from_numpy(x0).cuda()
            state = None if st is None else den._act(st)
            torch.cuda.synchronize()
        keep = []
        for t in range(len(frames) - 3):
            with torch.cuda.stream(sE):
                if two_streams:
                    fenc.encode_in_place(ftok[t + 3])
                else:
                    keep.append(fenc.encode(ftok[t + 3]))
            with torch.cuda.stream(sD):
                out = torch.empty_like(noise)
                fm.fm_denoise(den.ctx, noise, state, out)
                outs.append(out)
                for b in range(cfg.batch):
                    if two_streams:
                        den.append_encoded(b, fenc, b)
                    else:
                        fm.fm_append_prefix_kv(den.ctx, b, keep[-1][0][b], keep[-1][1][b])
        torch.cuda.synchronize()
        return [o.cpu().numpy() for o in outs], x0, st
    finally:
        den.close()
        fenc.close()
        penc.close()


def test_pipeline_equals_serial_bitwise_and_oracle():
    cfg, W, Wp, prompt, frames = _ring_inputs(batch=2)
    announce("async pipeline: 4 ticks, two robots")
    pipe, x0, st = _pipeline(cfg, W, Wp, prompt, frames, two_streams=True)
    ser, _, _ = _pipeline(cfg, W, Wp, prompt, frames, two_streams=False)
    for t, (a, b) in enumerate(zip(pipe, ser)):
        assert np.array_equal(a, b), f"tick {t}: pipelined != serial"
    # tick t denoises with frames t .. t + 2
    W64 = _prefix_weights(cfg, Wp)
    for t in (0, 3):
        kr, vr = [], []
        for b in range(cfg.batch):
            parts = [O.prefix_stack_kv(cfg, W64, x[b]) for x in [prompt] + frames[t:t + 3]]
            kr.append(np.concatenate([p[0] for p in parts], axis=1))
            vr.append(np.concatenate([p[1] for p in parts], axis=1))
        check(f"pipeline tick {t}", pipe[t], O.denoise(cfg, W, np.stack(kr), np.stack(vr), x0, st), 1e-2, 3e-2)


def test_append_encoded_rejects_mismatches():
    import flow_matching_denoising_euler_amd as fm
    from flow_matching_denoising_euler_amd import _abi
    cfg, W, Wp, prompt, frames = _ring_inputs()
    announce("fm_append_encoded errors")
    den = fm.Denoiser(cfg, W)
    enc = fm.Encoder(cfg, Wp, n_tokens=32)
    bad = fm.Encoder(cfg, Wp, n_tokens=20)
    plain = fm.Denoiser(small_cfg(), S.make_weights(small_cfg()))
    try:
        L = fm.lib()
        k0 = np.zeros((cfg.n_layers, 116, cfg.n_kv_heads, cfg.head_dim), np.float32)
        keep = den.set_prefix_kv(0, k0, k0)
        assert L.fm_append_encoded(den.ctx, 0, enc.ctx, 0) == _abi.FM_ERR_STATE  # nothing encoded yet
        enc.encode_in_place(frames[0])
        bad.encode_in_place(prompt)
        assert L.fm_append_encoded(den.ctx, 0, bad.ctx, 0) == _abi.FM_ERR_SHAPE  # 20 tokens, frames of 32
        assert L.fm_append_encoded(den.ctx, 0, enc.ctx, 1) == _abi.FM_ERR_ARG    # one sequence
        assert L.fm_append_encoded(den.ctx, 1, enc.ctx, 0) == _abi.FM_ERR_ARG    # one robot
        assert L.fm_append_encoded(den.ctx, 0, den.ctx, 0) == _abi.FM_ERR_ARG    # not an encoder
        assert L.fm_append_encoded(plain.ctx, 0, enc.ctx, 0) == _abi.FM_ERR_STATE  # no ring
        assert L.fm_append_encoded(den.ctx, 0, enc.ctx, 0) == _abi.FM_OK
        import torch
        torch.cuda.synchronize()
        del keep
    finally:
        for c in (den, enc, bad, plain):
            c.close()
