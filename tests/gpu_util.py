"""Helpers shared by the GPU tests: run a workload through the C ABI."""
import numpy as np

import fm_synth as S


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


def run_denoiser(cfg, W, k, v, noise, state, exec_mode=0, repeat=1):
    """Create a context, load every robot's prefix, denoise `repeat` times.
    Returns a list of numpy action arrays (one per repeat)."""
    import torch
    import flow_matching_denoising_euler_amd as fm
    den = fm.Denoiser(cfg, W, exec_mode=exec_mode)
    try:
        keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
        outs = [den.denoise(noise, state).cpu().numpy() for _ in range(repeat)]
        torch.cuda.synchronize()
        del keep
        return outs
    finally:
        den.close()


def small_cfg(**kw):
    """A small bf16 Pi0-shaped expert (GQA, one KV head) with ragged sizes."""
    base = S.workload("tiny_fp32").replace(
        name="small_bf16", seed=7, d_model=128, n_layers=2, n_q_heads=4, n_kv_heads=1, head_dim=64,
        d_mlp=256, time_dim=128, chunk=13, state_dim=32, batch=2, prefix_static=45, prefix_len=45,
        weight_dtype="bf16", act_dtype="bf16")
    return base.replace(**kw)


def check(name, got, ref, tol_rel, tol_abs=None):
    import oracle as O
    rel = O.rel_l2(got, ref)
    mab = O.max_abs(got, ref)
    mae = np.mean(np.abs(np.asarray(got, np.float64) - ref), axis=tuple(range(ref.ndim - 1)))
    announce(f"{name}: rel_l2 {rel:.3e} max_abs {mab:.3e} worst-dim MAE {mae.max():.3e}")
    assert np.all(np.isfinite(got)), name
    assert rel <= tol_rel, (name, rel)
    if tol_abs is not None:
        assert mab <= tol_abs, (name, mab)
