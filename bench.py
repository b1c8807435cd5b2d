#!/usr/bin/env python3
"""Denoise-loop benchmark on one MI355X.

One step = one fm_denoise call: the whole Euler loop (10 steps of the action
expert) for one action chunk of every robot, with weights, prefix K/V, noise
and state already resident in HBM.  Prints one JSON line on stdout.

The roofline object describes the dominant kernel of the loop, timed live
with HIP events on the context's stream (torch's current stream) through
fm_launch_phase; `frac` = achieved / MI355X spec peak.  The loop's own
fraction of its roofline (algorithmic bytes or flops per chunk over the spec
peak, against the measured ms per chunk) is reported as `loop_roofline`.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E spec
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA spec
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector spec
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA spec

METRIC = "denoise-loop ms per action chunk (10 steps) + % of roofline, Pi0-like bs=1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg, info):
    """Per-chunk algorithmic bytes (weights streamed once per velocity
    evaluation plus the prefix K/V read once per evaluation) and flops (2*M
    per matrix parameter plus attention), the figures the roofline is priced
    on.  Euler evaluates once per step, Heun twice."""
    d, L, F, Hq, Hkv, Dh = cfg.d_model, cfg.n_layers, cfg.d_mlp, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    S = cfg.suffix
    M = cfg.batch * S
    mat = L * (d * (Hq + 2 * Hkv) * Dh + d * Hq * Dh + 3 * d * F) + 2 * cfg.action_dim * d
    T = cfg.prefix_len
    attn = 4 * cfg.batch * L * S * Hq * Dh * (T + S)
    evals = cfg.n_steps * (2 if cfg.sampler == "heun" else 1)
    flops = evals * (2 * M * mat + attn)
    byts = evals * (info.weight_bytes_per_step + info.kv_bytes_per_step)
    return byts, flops


def kernel_source_sha():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "flow_matching_denoising_euler_amd", "csrc"))):
        with open(os.path.join(ROOT, "flow_matching_denoising_euler_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, phase):
    """HBM bytes per launch of `phase` from the committed PMC summary of
    `workload` (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's
    readings), if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_sha") != kernel_source_sha():
        return None
    if "phases" in t:
        return t["phases"].get(phase, {}).get("traffic_bytes")
    return t.get("traffic_bytes") if t.get("phase") == phase else None


PHASE_NAMES = ["QKV GEMM (norm1 folded)", "attention", "O GEMM + residual", "gate/up GEMM + GELU gate",
               "down GEMM + residual", "tail (final norm, head, update, next embedding)"]


def dtype_of(cfg):
    """The arithmetic the layer GEMMs compute in."""
    if getattr(cfg, "w8a8", False):
        return "fp8-e4m3 weights and GEMM activations (32-element power-of-two blocks), fp32 accumulate"
    return {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations"}[cfg.weight_dtype]


def phase_work(cfg, info, ph):
    """Algorithmic bytes and flops of one launch of phase `ph`: its weight
    matrix streamed once (fp8: codes and per-column scales), the prefix K/V
    of one layer read once (attention), and 2 flops per multiply-add."""
    d, L, F, Hq, Hkv, Dh, A = (cfg.d_model, cfg.n_layers, cfg.d_mlp, cfg.n_q_heads, cfg.n_kv_heads,
                               cfg.head_dim, cfg.action_dim)
    M = cfg.batch * cfg.suffix
    es = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]
    sc = 4 if cfg.weight_dtype == "fp8" else 0  # fp32 scale per output column
    eg = 4 if cfg.act_dtype == "f32" else 2
    nq = (Hq + 2 * Hkv) * Dh
    if ph == 0:
        return nq * d * es + nq * sc, 2 * M * d * nq
    if ph == 1:
        T = cfg.prefix_len
        return info.kv_bytes_per_step // L, 4 * cfg.batch * cfg.suffix * Hq * Dh * (T + cfg.suffix)
    if ph == 2:
        return d * Hq * Dh * es + d * sc, 2 * M * Hq * Dh * d
    if ph == 3:
        return 2 * F * d * es + 2 * F * sc, 2 * M * d * 2 * F
    if ph == 4:
        return d * F * es + d * sc, 2 * M * F * d
    return (2 * A * d + d) * eg, 2 * 2 * cfg.batch * cfg.chunk * d * A


def roofline_of(byts, flops, us, peak_f):
    """The roofline a launch of `byts` / `flops` in `us` sits under: the
    binding one of HBM (8 TB/s) and the MFMA peak of its dtype."""
    t_b, t_f = byts / (HBM_PEAK_GBS * 1e9), flops / (peak_f * 1e12)
    if t_f > t_b:
        a = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": peak_f, "unit": "TFLOP/s", "frac": round(a / peak_f, 4)}
    a = byts / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4)}


def phase_table(fm, den, cfg, info, stream, persistent, chunk_ms):
    """Average duration of every phase kernel, timed with HIP events on the
    context's stream over back-to-back launches through fm_launch_phase
    (cycling layers and steps), its launches per chunk, and its roofline."""
    import torch
    peak_f = BF16_PEAK_TFLOPS if cfg.act_dtype == "bf16" else FP32_PEAK_TFLOPS
    evals = cfg.n_steps * (2 if cfg.sampler == "heun" else 1)
    out = {}
    if persistent:  # the whole loop is one kernel: its work is the chunk's
        reps = 10
        fm.fm_launch_phase(den.ctx, 0, 0, fm._abi.FM_PHASE_LOOP)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fm.fm_launch_phase(den.ctx, 0, 0, fm._abi.FM_PHASE_LOOP)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        byts, flops = algorithmic(cfg, info)
        out["persistent loop kernel"] = {"per_launch": {"bytes": int(byts), "flops": int(flops), "avg_us": round(us, 3)},
                                         "launches_per_chunk": 1, "per_chunk_ms": round(us / 1e3, 4),
                                         "roofline": roofline_of(byts, flops, us, peak_f)}
        return out
    for ph in range(6):
        reps = 4 * cfg.n_layers if ph < 5 else 4 * cfg.n_steps
        fm.fm_launch_phase(den.ctx, 0, 0, ph)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fm.fm_launch_phase(den.ctx, i % cfg.n_steps, i % cfg.n_layers, ph)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        byts, flops = phase_work(cfg, info, ph)
        n = evals * cfg.n_layers if ph < 5 else evals
        pk = FP8_PEAK_TFLOPS if cfg.w8a8 and ph in (0, 2, 3, 4) else peak_f
        out[PHASE_NAMES[ph]] = {"per_launch": {"bytes": int(byts), "flops": int(flops), "avg_us": round(us, 3)},
                                "launches_per_chunk": n, "per_chunk_ms": round(us * n / 1e3, 4),
                                "roofline": roofline_of(byts, flops, us, pk)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, W, k, v, x0, st, runs=3):
    """The fp64 oracle as it stands, on this host's cores, on a bounded sample:
    one warmup, then the median of `runs` single-robot chunks (all robots are
    independent, so a batch costs batch x one robot); and on one thread the
    median of `runs` single velocity evaluations, scaled to the chunk's
    evaluations (the loop's cost is linear in them)."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    W64 = O.effective_weights(cfg, W)
    stb = lambda b: None if st is None else st[b]

    def chunk(b):
        t0 = time.perf_counter()
        O.denoise_robot(cfg, W64, k[b], v[b], x0[b], stb(b))
        return time.perf_counter() - t0

    def one_eval(b):
        t0 = time.perf_counter()
        O.expert_velocity(cfg, W64, np.asarray(x0[b], np.float64), 1.0, k[b], v[b], stb(b))
        return time.perf_counter() - t0

    chunk(0)  # warmup
    times = [chunk(i % cfg.batch) for i in range(runs)]
    evals = cfg.n_steps * (2 if cfg.sampler == "heun" else 1)
    with threadpool_limits(1):
        one_eval(0)
        t1 = [one_eval(i % cfg.batch) for i in range(runs)]
    per_robot_ms = statistics.median(times) * 1e3
    return {"value": round(per_robot_ms * cfg.batch, 2), "unit": "ms per action chunk (all robots)",
            "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"fp64 NumPy oracle: 1 warmup + median of {runs} single-robot chunks of {cfg.name} "
                      f"({evals} velocity evaluations each) on {threads} threads, scaled x{cfg.batch} robots",
            "one_thread": {"value": round(statistics.median(t1) * 1e3 * evals * cfg.batch, 2),
                           "unit": "ms per action chunk (all robots)", "cores": 1,
                           "sample": f"median of {runs} single velocity evaluations on 1 thread after 1 warmup, "
                                     f"scaled x{evals} evaluations x{cfg.batch} robots"}}


def encode_bench(args, cfg):
    """The prefix encoder alone: ms per fm_encode_prefix call (output left in
    the encoder), and the dominant kernel against its roofline.  Its GEMMs
    have M = batch x frame_tokens rows; at 256 rows and bf16 the arithmetic
    intensity (2 x 256 / 2 = 256 flop/B) is below the ridge (312), so the
    encode is priced on its weight stream."""
    import numpy as np
    import torch

    import fm_synth as S
    import flow_matching_denoising_euler_amd as fm

    torch.cuda.set_device(0)
    n_tok = cfg.frame_tokens or 256
    log(f"bench: prefix stack of {cfg.name}, {cfg.batch} x {n_tok} tokens")
    Wp, tokens = S.make_prefix_stack(cfg, n_tok)
    stream = torch.cuda.current_stream()
    enc = fm.Encoder(cfg, Wp, n_tokens=n_tok, n_seqs=cfg.batch, stream=stream)
    tok = torch.from_numpy(tokens).cuda()
    for _ in range(args.warmup):
        enc.encode_in_place(tok)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        enc.encode_in_place(tok)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    info = enc.info()
    byts = info.weight_bytes_per_step + info.kv_bytes_per_step
    achieved = byts / (ms * 1e-3) / 1e9
    d, L, F, Hq, Hkv, Dh = cfg.d_model, cfg.n_layers, cfg.d_mlp, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    M = cfg.batch * n_tok
    flops = 2 * M * (L * d * (Hq + 2 * Hkv) * Dh + (L - 1) * (d * Hq * Dh + 3 * d * F)) + \
        4 * cfg.batch * (L - 1) * n_tok * Hq * Dh * n_tok
    log(f"bench: encode {ms:.4f} ms -> {achieved:.1f} GB/s of weights + K/V, {flops / ms / 1e9:.1f} TFLOP/s")
    line = {
        "metric": "prefix encoder ms per call (frames through the expert-shaped stack)",
        "value": round(ms, 4), "unit": "ms per encode", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_of(cfg),
        "data": "synthetic (seeded prefix-stack weights, N(0,1) tokens)",
        "config": {"workload": cfg.name, "sequences": cfg.batch, "tokens": n_tok, "d_model": d, "layers": L,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole encode (weights streamed once, K/V written once)",
                     "per_launch": {"bytes": byts, "flops": flops, "avg_us": round(ms * 1e3, 3)}},
        "mfma_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
    }
    enc.close()
    print(json.dumps(line), flush=True)


def pipeline_bench(args, cfg):
    """Ticks of the streaming loop with the frame encoder in it.  serial: on
    one stream, encode frame t (256 tokens through the Pi0-shaped stack) ->
    append -> denoise.  pipelined: the encoder on its own stream encodes frame
    t + 1 while tick t denoises; the tick ends with the device-side hand-off
    (fm_append_encoded).  Both run K timed ticks after W warmup ticks."""
    import numpy as np
    import torch

    import fm_synth as S
    import flow_matching_denoising_euler_amd as fm

    if cfg.n_frames <= 0:
        print("bench.py --pipeline needs a streaming workload (one with a frame ring)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log(f"bench: generating {cfg.name} and its prefix stack")
    W = S.make_weights(cfg)
    Wp, _ = S.make_prefix_stack(cfg.replace(batch=1), 1)
    k, v = S.make_prefix(cfg)
    g = np.random.default_rng(cfg.seed + 100)
    ftok = [torch.from_numpy(S.round_bf16(g.standard_normal((cfg.batch, cfg.frame_tokens, cfg.d_model)))).cuda()
            for _ in range(4)]
    x0 = torch.from_numpy(S.make_noise(cfg)).cuda()
    st = S.make_state(cfg)
    res = {}
    for mode in ("serial", "pipelined"):
        sD = torch.cuda.Stream()
        sE = torch.cuda.Stream() if mode == "pipelined" else sD
        with torch.cuda.stream(sD):
            den = fm.Denoiser(cfg, W, stream=sD)
            keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
            state = None if st is None else den._act(st)
            out = torch.empty_like(x0)
        with torch.cuda.stream(sE):
            enc = fm.Encoder(cfg, Wp, n_tokens=cfg.frame_tokens, n_seqs=cfg.batch, stream=sE)
        torch.cuda.synchronize()

        def tick(i):
            with torch.cuda.stream(sE):
                enc.encode_in_place(ftok[i % 4])
            with torch.cuda.stream(sD):
                if mode == "serial":  # the new frame first, then the denoise that sees it
                    for b in range(cfg.batch):
                        den.append_encoded(b, enc, b)
                    fm.fm_denoise(den.ctx, x0, state, out)
                else:  # denoise with the frames so far while the encoder runs, then hand off
                    fm.fm_denoise(den.ctx, x0, state, out)
                    for b in range(cfg.batch):
                        den.append_encoded(b, enc, b)

        for i in range(args.warmup):
            tick(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(sD)
        for i in range(args.steps):
            tick(i)
        t1.record(sD)
        torch.cuda.synchronize()
        res[mode] = t0.elapsed_time(t1) / args.steps
        # the parts alone, on the same contexts
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(sE):
            e0.record(sE)
            for i in range(20):
                enc.encode_in_place(ftok[i % 4])
            e1.record(sE)
        torch.cuda.synchronize()
        res["encode_ms"] = e0.elapsed_time(e1) / 20
        with torch.cuda.stream(sD):
            e0.record(sD)
            for i in range(20):
                fm.fm_denoise(den.ctx, x0, state, out)
            e1.record(sD)
        torch.cuda.synchronize()
        res["denoise_ms"] = e0.elapsed_time(e1) / 20
        assert torch.isfinite(out).all().item(), "non-finite actions"
        log(f"bench: {mode} {res[mode]:.4f} ms/tick (encode {res['encode_ms']:.4f}, denoise {res['denoise_ms']:.4f})")
        enc.close()
        den.close()
        del keep
    line = {
        "metric": "streaming tick ms (encode the new 256-token frame + append + denoise), async pipeline",
        "value": round(res["pipelined"], 4),
        "unit": "ms per tick",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["pipelined"], 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_of(cfg),
        "data": "synthetic (seeded weights for the expert and the prefix stack, N(0,1) frame tokens)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "frame_tokens": cfg.frame_tokens,
                   "n_frames": cfg.n_frames, "prefix_tokens": cfg.prefix_len, "n_steps": cfg.n_steps,
                   "parallelism": "single GPU, two streams"},
        "serial_ms_per_tick": round(res["serial"], 4),
        "encode_ms": round(res["encode_ms"], 4),
        "denoise_ms": round(res["denoise_ms"], 4),
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; a streaming workload: all of its ticks)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pi0_1view")
    ap.add_argument("--sampler", choices=("euler", "heun", "ab2"), default=None,
                    help="override the workload's sampler (Heun: two velocity evaluations per step)")
    ap.add_argument("--n-steps", type=int, default=None, help="override the workload's step count")
    ap.add_argument("--kv-fp8", action="store_true", help="hold the prefix K/V cache in fp8 E4M3 (per token and kv head scales)")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="quantise the per-layer matrices to fp8 E4M3 (per output row scales; bf16 activations)")
    ap.add_argument("--w8a8", action="store_true",
                    help="fp8 weights and fp8 GEMM activations (32-element power-of-two blocks, block-scaled MFMA)")
    ap.add_argument("--exec-mode", type=int, default=0)
    ap.add_argument("--attn-kernel", choices=("auto", "register", "streamed"), default="auto",
                    help="attention kernel (auto: the register kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 256 MiB device copy (reference for PMC byte counters)")
    ap.add_argument("--pipeline", action="store_true",
                    help="streaming workloads: time whole ticks (encode the new frame through the prefix "
                         "encoder, append it, denoise), serial on one stream and as the two-stream async "
                         "pipeline; prints that line instead")
    ap.add_argument("--encode", action="store_true",
                    help="time the prefix encoder instead: one call encodes `batch` frames of frame_tokens "
                         "(256 if the workload has no ring) through the expert-shaped stack; prints that line")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU; the denoise loop shards by robot with no "
              "exchange, so there is no multi-GPU figure to measure (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fm_synth as S
    import flow_matching_denoising_euler_amd as fm

    cfg = S.workload(args.workload)
    base_weights = cfg.weight_dtype
    if args.fp8_weights:
        if cfg.act_dtype != "bf16":
            raise SystemExit("--fp8-weights needs a workload with bf16 activations")
        cfg = cfg.replace(weight_dtype="fp8")
    if args.w8a8:
        if cfg.act_dtype != "bf16":
            raise SystemExit("--w8a8 needs a workload with bf16 activations")
        cfg = cfg.replace(weight_dtype="fp8", w8a8=True)
    if args.steps is None:
        args.steps = cfg.ticks if cfg.ticks > 0 and not (args.pipeline or args.encode) else 200
    if args.pipeline:
        return pipeline_bench(args, cfg)
    if args.encode:
        return encode_bench(args, cfg)
    if args.sampler is not None:
        cfg = cfg.replace(sampler=args.sampler)
    if args.n_steps is not None:
        cfg = cfg.replace(n_steps=args.n_steps)
    if args.kv_fp8:
        cfg = cfg.replace(kv_fp8=True)
    if args.attn_kernel != "auto":
        cfg = cfg.replace(attn_kernel=args.attn_kernel)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    log(f"bench: generating {cfg.name}")
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0 = S.make_noise(cfg)
    st = S.make_state(cfg)
    stream = torch.cuda.current_stream()
    den = fm.Denoiser(cfg, W, stream=stream, exec_mode=args.exec_mode)
    keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
    noise_d = torch.from_numpy(x0).to(dev)
    state_d = None if st is None else torch.from_numpy(st).to(dev, torch.bfloat16 if cfg.act_dtype == "bf16"
                                                              else torch.float32)
    out = torch.empty_like(noise_d)
    info = den.info()
    streaming = cfg.ticks > 0
    frames = []
    if streaming:  # a pool of pre-generated frames, resident in HBM
        for t in range(4):
            kf, vf = S.make_frame(cfg, t)
            frames.append([(den._act(kf[b]), den._act(vf[b])) for b in range(cfg.batch)])
        noises = [torch.from_numpy(S.make_tick_noise(cfg, t)).to(dev) for t in range(4)]

    def one(i):
        if streaming:
            for b in range(cfg.batch):
                fm.fm_append_prefix_kv(den.ctx, b, *frames[i % 4][b])
            fm.fm_denoise(den.ctx, noises[i % 4], state_d, out)
        else:
            fm.fm_denoise(den.ctx, noise_d, state_d, out)

    log(f"bench: warmup {args.warmup}")
    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item(), "non-finite actions"
    # timed region: exactly K steps, synchronised on both sides
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        one(i)
        ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = total_ms / args.steps
    pct = lambda p: per[min(len(per) - 1, int(p * len(per)))]
    log(f"bench: {ms:.4f} ms/chunk (p10 {pct(.1):.4f} p50 {pct(.5):.4f} p90 {pct(.9):.4f} p99 {pct(.99):.4f})")

    byts, flops = algorithmic(cfg, info)
    es = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]
    peak_f = BF16_PEAK_TFLOPS if cfg.act_dtype == "bf16" else FP32_PEAK_TFLOPS  # fp8 weights run bf16 MFMA
    t_flops = flops / (peak_f * 1e12)
    if cfg.w8a8:  # the layer GEMMs run on the fp8 MFMA: their flops at the fp8 peak
        evals = cfg.n_steps * (2 if cfg.sampler == "heun" else 1)
        gemm = sum(phase_work(cfg, info, ph)[1] for ph in (0, 2, 3, 4)) * evals * cfg.n_layers
        t_flops = gemm / (FP8_PEAK_TFLOPS * 1e12) + (flops - gemm) / (peak_f * 1e12)
    mfma_bound = t_flops > byts / (HBM_PEAK_GBS * 1e9)
    loop_roof_ms = (t_flops if mfma_bound else byts / (HBM_PEAK_GBS * 1e9)) * 1e3
    phases = phase_table(fm, den, cfg, info, stream, persistent=int(info.exec_mode) == fm.FM_EXEC_PERSISTENT,
                         chunk_ms=ms)
    dom = max(phases, key=lambda n: phases[n]["per_chunk_ms"])
    roof = dict(phases[dom]["roofline"])
    roof["kernel"] = dom
    roof["per_launch"] = phases[dom]["per_launch"]
    # committed counters: per workload, and per weight dtype where it was overridden
    variant = cfg.name + ("_w8a8" if cfg.w8a8 else ("" if cfg.weight_dtype == base_weights
                                                     else f"_{cfg.weight_dtype}_weights"))
    roof["traffic"] = load_traffic(variant, dom)
    # a second phase within 5% of the dominant one (the two trade places from
    # run to run): its roofline too
    second = sorted(phases, key=lambda n: phases[n]["per_chunk_ms"])[-2]
    roof_alt = None
    if phases[second]["per_chunk_ms"] >= 0.95 * phases[dom]["per_chunk_ms"]:
        roof_alt = dict(phases[second]["roofline"])
        roof_alt["kernel"] = second
        roof_alt["per_launch"] = phases[second]["per_launch"]
        roof_alt["traffic"] = load_traffic(variant, second)
    log(f"bench: dominant kernel {dom}: {phases[dom]['per_launch']['avg_us']:.2f} us x "
        f"{phases[dom]['launches_per_chunk']} = {phases[dom]['per_chunk_ms']:.3f} ms/chunk, "
        f"{roof['achieved']} {roof['unit']} ({roof['frac'] * 100:.2f}% of peak)")

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on the host")
        cpu = cpu_baseline(cfg, W, k, v, x0, st)
        log(f"bench: oracle {cpu['value']:.1f} ms/chunk on {cpu['cores']} threads, "
            f"{cpu['one_thread']['value']:.1f} on one ({cpu['cpu_model']})")

    line = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms per action chunk" + (" (16 robots)" if cfg.batch > 1 else "") + (" incl. frame append" if streaming else ""),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(cfg),
        "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) prefix K/V and noise)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "chunk": cfg.chunk, "state_tokens": cfg.has_state,
                   "prefix_tokens": cfg.prefix_len, "n_steps": cfg.n_steps, "sampler": cfg.sampler,
                   "kv_cache": "fp8-e4m3" if cfg.kv_fp8 else cfg.act_dtype,
                   "weights": cfg.weight_dtype + (" (w8a8)" if cfg.w8a8 else ""),
                   "d_model": cfg.d_model,
                   "layers": cfg.n_layers, "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}",
                   "d_mlp": cfg.d_mlp, "norm": cfg.norm, "exec_mode": int(info.exec_mode),
                   "attention": "streamed" if cfg.attn_kernel == "streamed" else "register",
                   "parallelism": "single GPU"},
        "chunks_per_s": round(1000.0 / ms * cfg.batch, 2),
        "latency_ms": {"p10": round(pct(.1), 4), "p50": round(statistics.median(per), 4),
                       "p90": round(pct(.9), 4), "p99": round(pct(.99), 4), "max": round(per[-1], 4),
                       "per": "tick (append + denoise)" if streaming else "chunk"},
        "roofline": roof,
        "roofline_runner_up": roof_alt,
        "loop_roofline": {"bound": "mfma" if mfma_bound else "hbm", "roofline_ms": round(loop_roof_ms, 4),
                          "frac": round(loop_roof_ms / ms, 4),
                          "algorithmic_bytes_per_chunk": byts, "algorithmic_flops_per_chunk": flops},
        "phases": {n: {kk: vv for kk, vv in p.items() if kk != "roofline"} | {"frac": p["roofline"]["frac"],
                                                                                "bound": p["roofline"]["bound"]}
                   for n, p in phases.items()},
        "cpu_baseline": cpu,
    }
    den.close()
    del keep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
