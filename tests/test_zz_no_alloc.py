"""fm_denoise_noalloc (the loop's scratch in the library's static per-GPU
array, nothing allocated) against fm_denoise on the same context: two calls
in a row, the second on a context with a smaller input, each equal to
fm_denoise bit for bit (same kernels, same order) and within the bf16 bar
of the oracle."""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check, small_cfg

pytestmark = pytest.mark.gpu


def _run_both(cfg):
    import torch
    import flow_matching_denoising_euler_amd as fm
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    den = fm.Denoiser(cfg, W)
    try:
        keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
        n = torch.from_numpy(x0).cuda()
        s = None if st is None else den._act(st)
        out_a, out_b = torch.empty_like(n), torch.empty_like(n)
        fm.fm_denoise(den.ctx, n, s, out_a)
        fm.fm_denoise_noalloc(den.ctx, n, s, out_b)
        torch.cuda.synchronize()
        del keep
        return out_a.cpu().numpy(), out_b.cpu().numpy(), O.denoise(cfg, W, k, v, x0, st)
    finally:
        den.close()


def test_noalloc_matches_denoise_two_calls_second_smaller():
    # first call: 3 robots with split-K residual GEMMs and a key-split
    # attention (both use the scratch); second: one robot, fewer rows and keys
    big = small_cfg(name="noalloc_big", batch=3, chunk=20, head_dim=128, prefix_static=600, prefix_len=500)
    small = small_cfg(name="noalloc_small", batch=1, chunk=9, head_dim=128, prefix_static=520, prefix_len=300)
    for cfg in (big, small):
        announce(f"noalloc {cfg.name}: batch {cfg.batch} chunk {cfg.chunk} prefix {cfg.prefix_len}")
        a, b, ref = _run_both(cfg)
        assert np.array_equal(a, b), f"{cfg.name}: fm_denoise_noalloc != fm_denoise"
        check(f"noalloc {cfg.name}", b, ref, 1e-2, 3e-2)
