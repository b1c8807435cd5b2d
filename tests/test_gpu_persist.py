"""GPU parity of the persistent loop kernel (FM_EXEC_PERSISTENT): the whole
denoise loop of a batch-1-sized context as one kernel with grid barriers.

It runs the same phase bodies and work items as the per-phase graph, so the
two execution modes must agree bit for bit; each case is also checked
against the fp64 oracle (bf16 bar rel-L2 <= 1e-2 and max-abs <= 3e-2; fp8
weights rel-L2 <= 5e-2 on the same dequantised weights).  The cases cover
every attention instantiation (16-key blocks per wave 1..4 without a key
split, the key split), fp8 weights, a frame ring, Heun, Adams-Bashforth,
AdaRMSNorm, a caller schedule and two robots.
"""
import numpy as np
import pytest

import fm_synth as S
import oracle as O
from gpu_util import announce, check

pytestmark = pytest.mark.gpu

# the Pi0-shaped expert (full width) with two layers, so the oracle stays fast
PI0_2L = S.workload("pi0_1view").replace(name="pi0_2layers", n_layers=2)


def _run(cfg, W, k, v, x0, st, exec_mode):
    import torch
    import flow_matching_denoising_euler_amd as fm
    den = fm.Denoiser(cfg, W, exec_mode=exec_mode)
    try:
        mode = int(den.info().exec_mode)
        keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
        out = den.denoise(x0, st).cpu().numpy()
        torch.cuda.synchronize()
        del keep
        return out, mode
    finally:
        den.close()


@pytest.mark.parametrize("name,kw", [
    ("1view", dict()),                                                    # 352 keys: 3 key blocks per wave
    ("short prefix", dict(prefix_static=45, prefix_len=45, chunk=13)),    # 1 block per wave
    ("prefix 100", dict(prefix_static=100, prefix_len=100)),              # 2 blocks per wave
    ("prefix 420", dict(prefix_static=420, prefix_len=420)),              # 4 blocks per wave
    ("3 views", dict(prefix_static=768, prefix_len=768, chunk=63)),       # key split
    ("valid < capacity", dict(prefix_static=700, prefix_len=333)),        # key split, masked tail
    ("2 robots", dict(batch=2, chunk=20, prefix_static=150, prefix_len=150)),
    ("fp8 weights", dict(weight_dtype="fp8")),
    ("fp8 ring", dict(weight_dtype="fp8", prefix_static=20, frame_tokens=256, n_frames=3, prefix_len=788)),
    ("heun 3 steps", dict(sampler="heun", n_steps=3)),
    ("ab2", dict(sampler="ab2")),
    ("shifted schedule", dict(t_schedule=tuple(float(np.float32(3 * u / (1 + 2 * u))) for u in
                                               np.linspace(1.0, 0.0, 11)))),
    ("ada", dict(norm="ada", time_dim=256, state_dim=0)),
])
def test_persistent_equals_graph_and_oracle(name, kw):
    import flow_matching_denoising_euler_amd as fm
    cfg = PI0_2L.replace(**kw)
    announce(f"persistent {name}: {kw}")
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    got_p, mode_p = _run(cfg, W, k, v, x0, st, fm.FM_EXEC_PERSISTENT)
    got_g, mode_g = _run(cfg, W, k, v, x0, st, fm.FM_EXEC_GRAPH)
    assert (mode_p, mode_g) == (fm.FM_EXEC_PERSISTENT, fm.FM_EXEC_GRAPH)
    assert np.all(np.isfinite(got_p)), name
    assert np.array_equal(got_p, got_g), f"{name}: persistent != graph"
    ref = O.denoise(cfg, W, k, v, x0, st)
    if cfg.weight_dtype == "fp8":
        check(f"persistent {name}", got_p, ref, 5e-2)
    else:
        check(f"persistent {name}", got_p, ref, 1e-2, 3e-2)


def test_persistent_covers_the_pi0_workloads():
    import flow_matching_denoising_euler_amd as fm
    for name in ("pi0_1view", "pi0_3view", "stream_fp8"):
        cfg = S.workload(name).replace(n_layers=1)  # the plan does not depend on the layer count
        W = S.make_weights(cfg)
        for mode, want in ((fm.FM_EXEC_PERSISTENT, fm.FM_EXEC_PERSISTENT), (fm.FM_EXEC_AUTO, fm.FM_EXEC_GRAPH)):
            den = fm.Denoiser(cfg, W, exec_mode=mode)
            try:
                assert int(den.info().exec_mode) == want, (name, mode)
            finally:
                den.close()


def test_persistent_is_rejected_where_it_does_not_apply():
    import flow_matching_denoising_euler_amd as fm
    cfg = PI0_2L.replace(state_causal=True)
    with pytest.raises(fm.FMError, match="persistent loop"):
        fm.Denoiser(cfg, S.make_weights(cfg), exec_mode=fm.FM_EXEC_PERSISTENT)
    # the graph runs it
    den = fm.Denoiser(cfg, S.make_weights(cfg))
    try:
        assert int(den.info().exec_mode) == fm.FM_EXEC_GRAPH
    finally:
        den.close()


def test_persistent_runs_are_bitwise_repeatable():
    import torch
    import flow_matching_denoising_euler_amd as fm
    cfg = PI0_2L
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    den = fm.Denoiser(cfg, W, exec_mode=fm.FM_EXEC_PERSISTENT)
    try:
        keep = [den.set_prefix_kv(b, k[b], v[b]) for b in range(cfg.batch)]
        outs = [den.denoise(x0, st).cpu().numpy() for _ in range(3)]
        torch.cuda.synchronize()
        del keep
    finally:
        den.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
