"""Pins of the fp64 oracle against facts it does not compute itself: closed
forms, special cases that reduce to a simpler formula, invariants the pages
state, brute force on tiny inputs and the OCP fp8 code table.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or scale, a transposed operand) fails at least one test.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import fm_synth as S
import oracle as O

TINY = S.workload("tiny_fp32")


def _tiny(**kw):
    return TINY.replace(**kw)


def _inputs(cfg):
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    return W, k, v, S.make_noise(cfg), S.make_state(cfg)


# --- P1: the integrator and its schedule -----------------------------------
def test_time_grid_is_left_endpoints_from_one():
    ts, dt = O.time_grid(10)
    assert np.all(dt == -0.1)
    assert np.allclose(ts, [1.0, 0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.3, 0.2, 0.1], atol=0, rtol=1e-15)
    assert ts[0] == 1.0


def test_euler_linear_field_closed_form():
    # v = lam * x  =>  x_N = (1 + dt*lam)^N x0 = (1 - lam/N)^N x0
    x0 = np.array([1.5, -2.0, 0.25])
    for lam, n in ((0.7, 10), (-1.3, 8), (2.0, 1)):
        got = O.euler(lambda x, t: lam * x, x0, n)
        assert np.allclose(got, (1 - lam / n) ** n * x0, rtol=1e-14, atol=0)


def test_euler_time_field_displacement():
    # v = t: displacement sum_k dt*t_k = -(N+1)/(2N) = -0.55 at N=10 (a right
    # end point scheme would give -0.45, the midpoint rule -0.5).
    got = O.euler(lambda x, t: np.full_like(x, t), np.zeros(1), 10)
    assert abs(got[0] - (-0.55)) < 1e-15
    got = O.euler(lambda x, t: np.full_like(x, t), np.zeros(1), 4)
    assert abs(got[0] - (-5 / 8)) < 1e-15


def test_schedule_of_exact_uniform_times_equals_default():
    # k/8 is exact in fp32 and fp64: the explicit schedule is the default one
    ts, dt = O.time_grid(8, [1.0 - k / 8 for k in range(9)])
    t0, d0 = O.time_grid(8)
    assert np.array_equal(ts, t0) and np.array_equal(dt, d0)


def test_euler_linear_field_nonuniform_closed_form():
    # v = lam * x  =>  x_N = prod_k (1 + lam dt_k) x0
    s = [1.0, 0.875, 0.625, 0.5, 0.25, 0.0]
    x0 = np.array([1.5, -2.0, 0.25])
    for lam in (0.7, -1.3):
        got = O.euler(lambda x, t: lam * x, x0, 5, s)
        assert np.allclose(got, np.prod([1 + lam * (b - a) for a, b in zip(s[:-1], s[1:])]) * x0, rtol=1e-14, atol=0)


def test_euler_time_field_nonuniform_left_sum():
    # v = t: displacement sum_k t_k (t_(k+1) - t_k) = 1(-1/4) + 3/4(-1/4) + 1/2(-1/2) = -11/16
    got = O.euler(lambda x, t: np.full_like(x, t), np.zeros(1), 3, [1.0, 0.75, 0.5, 0.0])
    assert got[0] == -11 / 16


def test_heun_linear_field_closed_form():
    # v = lam * x: one Heun step multiplies by 1 + lam dt + (lam dt)^2 / 2
    s = [1.0, 0.875, 0.625, 0.5, 0.25, 0.0]
    x0 = np.array([1.5, -2.0, 0.25])
    for lam in (0.7, -1.3):
        f = np.prod([1 + lam * (b - a) + (lam * (b - a)) ** 2 / 2 for a, b in zip(s[:-1], s[1:])])
        assert np.allclose(O.heun(lambda x, t: lam * x, x0, 5, s), f * x0, rtol=1e-14, atol=0)
        f = (1 - lam / 10 + (lam / 10) ** 2 / 2) ** 10
        assert np.allclose(O.heun(lambda x, t: lam * x, x0, 10), f * x0, rtol=1e-14, atol=0)


def test_heun_is_exact_for_a_velocity_linear_in_t():
    # v = a + b t: the trapezoidal rule integrates it exactly, x_N = x_0 - a - b/2
    for sched, n in ((None, 10), ([1.0, 0.75, 0.5, 0.0], 3), (None, 1)):
        got = O.heun(lambda x, t: np.full_like(x, 0.3 - 1.7 * t), np.zeros(1), n, sched)
        assert abs(got[0] - (-0.3 + 1.7 / 2)) < 1e-15


def test_ab2_linear_in_t_field_errs_only_in_its_euler_start():
    # v = a + b t: every two-step Adams-Bashforth step after the first
    # integrates the line through its last two velocities, which is v itself,
    # exactly; the first (Euler) step misses b h_0^2 / 2.  So x_N = x_0 + the
    # integral of v from 1 to 0 (= -a - b/2) - b h_0^2 / 2, on uniform and
    # non-uniform schedules (the latter test the ratio of step sizes; their
    # times are exact in fp32, the precision the schedule is taken in).
    a, b = 0.3, -1.7
    for sched, n in ((None, 10), ([1.0, 0.75, 0.5, 0.0], 3), ([1.0, 0.875, 0.625, 0.5625, 0.1875, 0.0], 5), (None, 1)):
        h0 = (sched[1] - sched[0]) if sched else -1.0 / n
        got = O.ab2(lambda x, t: np.full_like(x, a + b * t), np.zeros(1), n, sched)
        assert abs(got[0] - (-a - b / 2 - b * h0 ** 2 / 2)) < 1e-14, (sched, n)


def test_ab2_is_second_order():
    # v = lam x from x(1) = 1: the error at t = 0 falls 4x per halving of the
    # step (a first-order slip, e.g. a wrong coefficient, gives 2x)
    lam = 1.3
    exact = np.exp(-lam)
    errs = [abs(O.ab2(lambda x, t: lam * x, np.ones(1), n)[0] - exact) for n in (40, 80, 160)]
    for e1, e2 in zip(errs, errs[1:]):
        assert 3.6 < e1 / e2 < 4.4, errs


def test_ab2_uses_one_evaluation_per_step_at_the_left_ends():
    seen = []
    O.ab2(lambda x, t: (seen.append(t), np.zeros_like(x))[1], np.zeros(1), 4)
    assert seen == [1.0, 0.75, 0.5, 0.25]


def test_heun_uses_the_right_end_times():
    seen = []
    O.heun(lambda x, t: (seen.append(t), np.zeros_like(x))[1], np.zeros(1), 4)
    assert seen == [1.0, 0.75, 0.75, 0.5, 0.5, 0.25, 0.25, 0.0]


def test_schedule_validation():
    for bad in ([1.0, 0.5, 0.5, 0.0], [0.9, 0.5, 0.2, 0.0], [1.0, 0.5, 0.2, 0.1], [1.0, 0.0]):
        with pytest.raises(ValueError):
            O.time_grid(3, bad)


def test_schedule_enters_the_model_through_t():
    # a schedule moves both where v is evaluated and the step sizes: the
    # tiny loop with a non-uniform schedule differs from the uniform one,
    # and equals an Euler loop written out here with the same velocity
    cfg = TINY.replace(n_steps=4, t_schedule=(1.0, 0.75, 0.5, 0.25, 0.0))
    W, k, v, x0, st = _inputs(cfg)
    W64 = O.effective_weights(cfg, W)
    ref = np.asarray(x0[0], np.float64).copy()
    for t, dt in ((1.0, -0.25), (0.75, -0.25), (0.5, -0.25), (0.25, -0.25)):
        ref = ref + dt * O.expert_velocity(cfg, W64, ref, t, k[0], v[0], st[0])
    got = O.denoise(cfg, W, k, v, x0, st)[0]
    assert np.array_equal(got, ref)
    skew = cfg.replace(t_schedule=(1.0, 0.9, 0.6, 0.3, 0.0))
    assert not np.allclose(O.denoise(skew, W, k, v, x0, st)[0], got, rtol=1e-6, atol=0)


# --- P2 / P3: output plumbing of the head ------------------------------------
def test_zero_head_leaves_noise_bitwise():
    cfg = TINY
    W, k, v, x0, st = _inputs(cfg)
    W["w_out"][:] = 0
    W["b_out"][:] = 0
    assert np.array_equal(O.denoise(cfg, W, k, v, x0, st), x0.astype(np.float64))


def test_bias_only_head_integrates_constant_velocity_exactly():
    # N = 8 (dt = -1/8) with dyadic b and x0: every update is exact, so
    # x_N = x0 + N*dt*b = x0 - b bitwise.
    cfg = _tiny(n_steps=8)
    W, k, v, _, st = _inputs(cfg)
    g = np.random.default_rng(5)
    b = g.integers(-64, 64, size=cfg.action_dim) / 16.0
    x0 = (g.integers(-128, 128, size=(1, cfg.chunk, cfg.action_dim)) / 32.0)
    W["w_out"][:] = 0
    W["b_out"] = b.astype(np.float32)
    got = O.denoise(cfg, W, k, v, x0, st)
    assert np.array_equal(got, x0 - b)
    # N = 10: dt is inexact, the error stays within a few ulp
    cfg = TINY
    got = O.denoise(cfg, W, k, v, x0, st)
    assert np.max(np.abs(got - (x0 - b))) < 20 * np.finfo(float).eps * 8


# --- P4: time-only velocity reduces to a short closed form -------------------
def test_time_only_velocity_matches_closed_form():
    cfg = TINY
    W, k, v, x0, st = _inputs(cfg)
    W["w_in"][:] = 0
    for L in W["layers"]:
        L["wo"][:] = 0
        L["wd"][:] = 0
    got = O.denoise(cfg, W, k, v, x0, st)[0]
    d = cfg.d_model
    expect = x0[0].astype(np.float64).copy()
    for kstep in range(cfg.n_steps):
        t = 1.0 - kstep / cfg.n_steps
        tau = [math.sin(t * 10000.0 ** (-j / (d // 2))) for j in range(d // 2)] + \
              [math.cos(t * 10000.0 ** (-j / (d // 2))) for j in range(d // 2)]
        h = [float(W["b_in"][i]) + tau[i] for i in range(d)]
        r = 1.0 / math.sqrt(math.fsum(a * a for a in h) / d + cfg.rms_eps)
        u = [h[i] * r * float(W["norm_f"][i]) for i in range(d)]
        vel = [math.fsum(u[i] * float(W["w_out"][a, i]) for i in range(d)) + float(W["b_out"][a])
               for a in range(cfg.action_dim)]
        expect = expect + (-1.0 / cfg.n_steps) * np.array(vel)[None, :]
    assert np.max(np.abs(got - expect)) < 1e-12


# --- P5 / P6: attention ---------------------------------------------------------
def test_attention_scale_is_inverse_sqrt_head_dim():
    # Dh = 4: q.k1 = 2 ln 3 -> scaled score ln 3 against 0: weights 3:1.
    q = np.array([[[2 * math.log(3), 0, 0, 0]]])
    k = np.array([[[1.0, 0, 0, 0]], [[0.0, 0, 0, 0]]])
    v = np.array([[[4.0, 0, 8, 1]], [[0.0, 4, 0, 1]]])
    out = O.attention(q, k, v)[0, 0]
    assert np.allclose(out, (3 * v[0, 0] + v[1, 0]) / 4, rtol=0, atol=1e-14)


def test_attention_equal_scores_give_mean_and_dominant_key_wins():
    g = np.random.default_rng(1)
    v = g.standard_normal((6, 1, 3))
    q = g.standard_normal((2, 1, 3))
    k = np.zeros((6, 1, 3))
    assert np.allclose(O.attention(q, k, v)[:, 0], v[:, 0].mean(0), atol=1e-14)
    k = g.standard_normal((6, 1, 3)) * 0.01
    k[4, 0] = q[0, 0] * 400.0
    assert np.allclose(O.attention(q[:1], k, v)[0, 0], v[4, 0], atol=1e-12)


def test_attention_brute_force_tiny():
    g = np.random.default_rng(2)
    Sq, T, Dh, Hq, Hkv = 4, 6, 3, 2, 1
    q = g.standard_normal((Sq, Hq, Dh))
    k = g.standard_normal((T, Hkv, Dh))
    v = g.standard_normal((T, Hkv, Dh))
    got = O.attention(q, k, v)
    for h in range(Hq):
        for i in range(Sq):
            sc = [math.fsum(q[i, h, c] * k[j, 0, c] for c in range(Dh)) / math.sqrt(Dh)
                  for j in range(T)]
            w = [math.exp(s) for s in sc]
            z = math.fsum(w)
            for c in range(Dh):
                ref = math.fsum(w[j] * v[j, 0, c] for j in range(T)) / z
                assert abs(got[i, h, c] - ref) < 1e-13
    p = O.softmax_rows(g.standard_normal((5, 7)) * 30)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)


def test_attention_key_permutation_and_split_lse_combine():
    g = np.random.default_rng(3)
    q = g.standard_normal((5, 4, 8))
    k = g.standard_normal((11, 2, 8))
    v = g.standard_normal((11, 2, 8))
    full = O.attention(q, k, v)
    perm = g.permutation(11)
    assert np.allclose(O.attention(q, k[perm], v[perm]), full, atol=1e-14)
    # split the keys in two, combine the halves by their log-sum-exp
    for cut in (1, 5, 10):
        parts = []
        for sl in (slice(0, cut), slice(cut, 11)):
            o = O.attention(q, k[sl], v[sl])
            lse = np.zeros((5, 4))
            for h in range(4):
                s = q[:, h] @ k[sl, h // 2].T / math.sqrt(8)
                lse[:, h] = np.log(np.exp(s).sum(1))
            parts.append((o, lse))
        m = np.maximum(parts[0][1], parts[1][1])
        w0, w1 = np.exp(parts[0][1] - m), np.exp(parts[1][1] - m)
        comb = (parts[0][0] * w0[..., None] + parts[1][0] * w1[..., None]) / (w0 + w1)[..., None]
        assert np.allclose(comb, full, atol=1e-13)


# --- P10: grouped-query head mapping -----------------------------------------
def test_gqa_equals_mha_with_repeated_kv():
    g = np.random.default_rng(4)
    q = g.standard_normal((3, 4, 8))
    k = g.standard_normal((7, 2, 8))
    v = g.standard_normal((7, 2, 8))
    # query heads 0,1 -> kv head 0; 2,3 -> kv head 1
    rep = O.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1))
    assert np.allclose(O.attention(q, k, v), rep, atol=1e-14)
    k1, v1 = k[:, :1], v[:, :1]
    assert np.allclose(O.attention(q, k1, v1), O.attention(q, np.repeat(k1, 4, 1), np.repeat(v1, 4, 1)),
                       atol=1e-14)


def test_gqa_model_equals_mha_model_with_tiled_kv_weights():
    cfg1 = _tiny(n_kv_heads=1)
    W, _, _, x0, st = _inputs(cfg1)
    k, v = S.make_prefix(cfg1)
    cfgm = _tiny(n_kv_heads=4)
    Wm = {kk: vv for kk, vv in W.items()}
    Wm["layers"] = [dict(L, wk=np.tile(L["wk"], (4, 1)), wv=np.tile(L["wv"], (4, 1)))
                    for L in W["layers"]]
    a = O.denoise(cfg1, W, k, v, x0, st)
    b = O.denoise(cfgm, Wm, np.repeat(k, 4, axis=3), np.repeat(v, 4, axis=3), x0, st)
    assert O.rel_l2(a, b) < 1e-13


# --- P11: norms, GELU, SiLU, sinusoid -------------------------------------------
def test_rmsnorm_closed_forms():
    h = np.array([[3.0, 4.0]])
    assert np.allclose(O.rmsnorm(h, np.ones(2), 0.0), h / math.sqrt(12.5), atol=1e-15)
    c, eps = 0.37, 1e-6
    g = np.array([1.0, 2.0, -0.5, 3.0])
    assert np.allclose(O.rmsnorm(np.full((1, 4), c), g, eps), c / math.sqrt(c * c + eps) * g, atol=1e-15)
    x = np.random.default_rng(0).standard_normal((3, 16))
    assert np.allclose(O.rmsnorm(5.0 * x, np.ones(16), 0.0), O.rmsnorm(x, np.ones(16), 0.0), atol=1e-14)


def test_gelu_is_exact_erf_form():
    assert O.gelu(np.array([0.0]))[0] == 0.0
    # Phi(1) of the standard normal distribution
    assert abs(O.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    x = np.linspace(-6, 6, 97)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-14)
    assert abs(O.gelu(np.array([1.0]))[0] - math.tanh(1.0)) > 1e-2  # not some other curve
    # the tanh approximation differs by ~1e-4 at x = 1.5: the exact form is used
    tanh_approx = 0.5 * 1.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * (1.5 + 0.044715 * 1.5 ** 3)))
    assert abs(O.gelu(np.array([1.5]))[0] - 1.5 * 0.5 * (1 + math.erf(1.5 / math.sqrt(2)))) < 1e-15
    assert abs(O.gelu(np.array([1.5]))[0] - tanh_approx) > 1e-5


def test_silu_values():
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_sinusoid_values():
    assert np.array_equal(O.sinusoid(0.0, 8), [0, 0, 0, 0, 1, 1, 1, 1])
    got = O.sinusoid(1.0, 4)  # w = [1, 10000^(-1/2)] = [1, 0.01]
    assert np.allclose(got, [math.sin(1), math.sin(0.01), math.cos(1), math.cos(0.01)], atol=1e-16)


# --- P7: cached timestep-invariant prefix equals joint recompute ----------------
@pytest.mark.parametrize("kind", ["rms_mha", "rms_gqa", "ada", "state_causal", "rope"])
def test_cached_prefix_equals_joint_recompute(kind):
    cfg = {"rms_mha": TINY, "rms_gqa": _tiny(n_kv_heads=1, batch=2),
           "ada": _tiny(norm="ada", time_dim=16, state_dim=0),
           "state_causal": _tiny(n_kv_heads=1, state_causal=True),
           "rope": _tiny(n_kv_heads=2, rope_theta=10000.0, batch=2)}[kind]
    W = S.make_weights(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    Wp, tokens = S.make_prefix_stack(cfg, 32)
    ks, vs = zip(*[O.prefix_stack_kv(cfg, Wp, tokens[b]) for b in range(cfg.batch)])
    cached = O.denoise(cfg, W, np.stack(ks), np.stack(vs), x0, st)
    joint = O.denoise_joint(cfg, W, Wp, tokens, x0, st)
    assert O.rel_l2(cached, joint) < 1e-12


# --- rotary position embedding ------------------------------------------------------
def test_rope_pairs_and_direction():
    # Dh = 4: pairs (0, 2) and (1, 3) turn by p and p * theta^(-1/2), counterclockwise
    th, p = 100.0, 0.7
    e0, e1 = np.array([[[1.0, 0, 0, 0]]]), np.array([[[0, 1.0, 0, 0]]])
    assert np.allclose(O.rope(e0, [p], th)[0, 0], [np.cos(p), 0, np.sin(p), 0], atol=1e-15)
    w = p * th ** -0.5
    assert np.allclose(O.rope(e1, [p], th)[0, 0], [0, np.cos(w), 0, np.sin(w)], atol=1e-15)
    x = np.random.default_rng(3).standard_normal((5, 2, 8))
    assert np.array_equal(O.rope(x, np.zeros(5), th), x)                       # position 0: identity
    assert np.allclose(np.linalg.norm(O.rope(x, np.arange(5) * 3.0, th), axis=-1), np.linalg.norm(x, axis=-1))


def test_rope_scores_depend_on_relative_position_only():
    g = np.random.default_rng(4)
    q, k = g.standard_normal((1, 1, 16)), g.standard_normal((1, 1, 16))
    s = lambda m, n: float(np.sum(O.rope(q, [m], 1e4) * O.rope(k, [n], 1e4)))
    for m, n, c in ((3, 1, 5), (0, 7, 11), (40, 2, -2)):
        assert abs(s(m, n) - s(m + c, n + c)) < 1e-12
    assert abs(s(3, 1) - s(4, 1)) > 1e-6


# --- block-causal state token (Pi0-style suffix) ------------------------------------
def _one_robot(cfg):
    W64 = O.effective_weights(cfg, S.make_weights(cfg))
    k, v = S.make_prefix(cfg)
    return W64, k[0], v[0], S.make_noise(cfg)[0], S.make_state(cfg)[0]


@pytest.mark.parametrize("norm", ["rms", "ada"])
def test_block_causal_state_is_a_cached_prefix_token(norm):
    # Under the block-causal suffix the state token sees only the prefix and
    # itself, so it can be run alone and its per-layer K/V appended to the
    # prefix: the action tokens of an expert without a state token then give
    # the same velocity.  Without the mask they do not.
    cfg = _tiny(state_causal=True, norm=norm, time_dim=16 if norm == "ada" else TINY.time_dim)
    W64, kp, vp, x, s0 = _one_robot(cfg)
    t = 0.37
    vel = O.expert_velocity(cfg, W64, x, t, kp, vp, s0)
    _, ks, vs = O.expert_velocity(cfg, W64, x[:0], t, kp, vp, s0, return_kv=True)  # the state token alone
    assert ks.shape[1] == 1
    kp2, vp2 = np.concatenate([kp, ks], axis=1), np.concatenate([vp, vs], axis=1)
    vel2 = O.expert_velocity(cfg.replace(state_dim=0, state_causal=False), W64, x, t, kp2, vp2, None)
    assert np.allclose(vel, vel2, rtol=1e-12, atol=1e-12)
    full = O.expert_velocity(cfg.replace(state_causal=False), W64, x, t, kp, vp, s0)
    assert O.rel_l2(full, vel2) > 1e-4


def test_block_causal_state_kv_ignores_x_and_t():
    cfg = _tiny(state_causal=True)
    W64, kp, vp, x, s0 = _one_robot(cfg)
    _, k1, v1 = O.expert_velocity(cfg, W64, x, 0.9, kp, vp, s0, return_kv=True)
    _, k2, v2 = O.expert_velocity(cfg, W64, -3.0 * x, 0.1, kp, vp, s0, return_kv=True)
    assert np.array_equal(k1[:, 0], k2[:, 0]) and np.array_equal(v1[:, 0], v2[:, 0])  # the state row
    assert not np.allclose(k1[:, 1:], k2[:, 1:])                                      # action rows


# --- P8: ring buffer in logical order ---------------------------------------------
def test_ring_logical_order_after_appends():
    ns, nf, F = 2, 3, 3
    r = O.PrefixRing(ns, nf, F)
    base = np.arange(1 * (ns + F * nf)).reshape(1, -1)
    r.set(base)
    assert np.array_equal(r.logical(), base)
    frames = [np.full((1, nf), 100 + i) for i in range(7)]
    for i, f in enumerate(frames):
        r.append(f)
        last = ([base[:, ns + j * nf: ns + (j + 1) * nf] for j in range(F)] + frames[:i + 1])[-F:]
        assert np.array_equal(r.logical(), np.concatenate([base[:, :ns]] + last, axis=1))


# --- P9: AdaRMSNorm special values -------------------------------------------------
def _ada_cfg():
    return _tiny(norm="ada", time_dim=16)


def test_ada_identity_modulation_reduces_to_rms_expert():
    cfg_a = _ada_cfg()
    cfg_r = TINY
    Wa = S.make_weights(cfg_a)
    k, v = S.make_prefix(cfg_a)
    x0, st = S.make_noise(cfg_a), S.make_state(cfg_a)
    d = cfg_a.d_model
    ident = np.concatenate([np.zeros(d), np.zeros(d), np.ones(d)])
    for L in Wa["layers"]:
        for n in ("norm1", "norm2"):
            L[n + "_w"][:] = 0
            L[n + "_b"] = ident.copy()
    Wa["norm_f_w"][:] = 0
    Wa["norm_f_b"] = ident.copy()
    t = 0.7
    Wr = {kk: vv for kk, vv in Wa.items() if not kk.startswith(("norm_f", "w_time", "b_time"))}
    Wr["b_in"] = Wa["b_in"] - O.sinusoid(t, d)  # cancel the additive time feature at t
    Wr["norm_f"] = np.ones(d)
    Wr["layers"] = [dict(wq=L["wq"], wk=L["wk"], wv=L["wv"], wo=L["wo"], wg=L["wg"], wu=L["wu"],
                         wd=L["wd"], norm1=np.ones(d), norm2=np.ones(d)) for L in Wa["layers"]]
    Wa64, Wr64 = O.effective_weights(cfg_a, Wa), O.effective_weights(cfg_r, Wr)
    va = O.expert_velocity(cfg_a, Wa64, x0[0], t, k[0], v[0], st[0])
    vr = O.expert_velocity(cfg_r, Wr64, x0[0], t, k[0], v[0], st[0])
    assert O.rel_l2(va, vr) < 1e-14


def test_ada_gamma_minus_one_and_alpha_zero():
    # alpha = 0 turns every block into the identity, gamma_f = -1 makes the
    # final norm output beta_f: the velocity is beta_f W_out^T + b_out for
    # every x and t, so x_N = x0 - (beta_f W_out^T + b_out).
    cfg = _ada_cfg()
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    d = cfg.d_model
    beta_f = np.random.default_rng(9).standard_normal(d)
    for L in W["layers"]:
        for n in ("norm1", "norm2"):
            L[n + "_w"][:] = 0
            L[n + "_b"] = np.concatenate([np.zeros(d), np.zeros(d), np.zeros(d)])
    W["norm_f_w"][:] = 0
    W["norm_f_b"] = np.concatenate([-np.ones(d), beta_f, np.zeros(d)])
    vel = beta_f @ W["w_out"].astype(np.float64).T + W["b_out"]
    got = O.denoise(cfg, W, k, v, x0, st)
    assert np.max(np.abs(got - (x0 - vel))) < 1e-13


# --- P9b: the AdaRMSNorm time MLP, written out in scalars ----------------------------
def _silu_s(z):
    return z / (1.0 + math.exp(-z))


def _tau_s(t, dim):
    half = dim // 2
    w = [10000.0 ** (-j / half) for j in range(half)]
    return [math.sin(t * wj) for wj in w] + [math.cos(t * wj) for wj in w]


def _mv_s(W, x, b=None):
    """y_o = sum_i W[o][i] x[i] (+ b_o), exactly rounded sums."""
    W = np.asarray(W, np.float64)
    return [math.fsum(float(W[o, i]) * x[i] for i in range(len(x))) + (0.0 if b is None else float(b[o]))
            for o in range(W.shape[0])]


def _time_c_s(W, t, time_dim):
    # c = SiLU(W_t tau(t) + b_t): the flow-phase embedding every norm reads
    return [_silu_s(z) for z in _mv_s(W["w_time"], _tau_s(t, time_dim), W["b_time"])]


def test_ada_modulation_matches_scalar_time_mlp():
    # every norm's (gamma, beta, alpha) = split3(W_n c + b_n) with
    # c = SiLU(W_t tau_time_dim(t) + b_t), per layer (norm1, norm2) then final
    cfg = _ada_cfg()
    W = S.make_weights(cfg)
    d = cfg.d_model
    for t in (1.0, 0.3):
        per_layer, fin = O.ada_modulation(cfg, O.effective_weights(cfg, W), t)
        c = _time_c_s(W, t, cfg.time_dim)
        want = [[_mv_s(L[n + "_w"], c, L[n + "_b"]) for n in ("norm1", "norm2")] for L in W["layers"]]
        for li, (m1, m2) in enumerate(per_layer):
            for got, ref in ((m1, want[li][0]), (m2, want[li][1])):
                for part in range(3):
                    assert np.max(np.abs(got[part] - np.array(ref[part * d:(part + 1) * d]))) < 1e-12
        ref_f = _mv_s(W["norm_f_w"], c, W["norm_f_b"])
        for part in range(3):
            assert np.max(np.abs(fin[part] - np.array(ref_f[part * d:(part + 1) * d]))) < 1e-12


def test_ada_time_mlp_through_the_final_norm_closed_form():
    # Every block is the identity (all per-layer modulations zero, so alpha =
    # 0); the final norm is modulated by the flow phase: v = (rms(h0) (1 +
    # gamma_f(t)) + beta_f(t)) W_out^T + b_out with h0 = x W_in^T + b_in.  The
    # whole loop is rewritten here in scalars; a dropped SiLU, tau(1 - t), a
    # swapped (gamma, beta) split or a missing (1 + .) all change x_N.
    cfg = _ada_cfg()
    W = S.make_weights(cfg)
    k, v = S.make_prefix(cfg)
    x0, st = S.make_noise(cfg), S.make_state(cfg)
    d, A = cfg.d_model, cfg.action_dim
    for L in W["layers"]:
        for n in ("norm1", "norm2"):
            L[n + "_w"][:] = 0
            L[n + "_b"][:] = 0
    got = O.denoise(cfg, W, k, v, x0, st)[0]
    x = [[float(a) for a in row] for row in x0[0]]
    for kstep in range(cfg.n_steps):
        t = 1.0 - kstep / cfg.n_steps
        m = _mv_s(W["norm_f_w"], _time_c_s(W, t, cfg.time_dim), W["norm_f_b"])
        gam, bet = m[:d], m[d:2 * d]
        new = []
        for row in x:
            h = _mv_s(W["w_in"], row, W["b_in"])
            r = 1.0 / math.sqrt(math.fsum(a * a for a in h) / d + cfg.rms_eps)
            u = [h[i] * r * (1.0 + gam[i]) + bet[i] for i in range(d)]
            vel = _mv_s(W["w_out"], u, W["b_out"])
            new.append([row[a] + (-1.0 / cfg.n_steps) * vel[a] for a in range(A)])
        x = new
    assert np.max(np.abs(got - np.array(x))) < 1e-11


def test_ada_constant_modulation_is_rms_expert_with_gains_and_gates():
    # W_n = 0, b_n = [g - 1 | 0 | a]: each norm is an RMSNorm with gain g and
    # its residual branch is gated by a, which equals scaling the output rows
    # of W_o (norm1's gate) or W_d (norm2's gate).  Distinct gains and gates per
    # layer and per norm tell norm1 from norm2 and the two gates apart.
    cfg_a = _ada_cfg()
    cfg_r = TINY
    Wa = S.make_weights(cfg_a)
    k, v = S.make_prefix(cfg_a)
    x0, st = S.make_noise(cfg_a), S.make_state(cfg_a)
    d = cfg_a.d_model
    g = np.random.default_rng(21)
    gains = {}
    for li, L in enumerate(Wa["layers"]):
        for n in ("norm1", "norm2"):
            gain, gate = 1.0 + 0.3 * g.standard_normal(d), 0.5 + g.random(d)
            gains[(li, n)] = (gain, gate)
            L[n + "_w"][:] = 0
            L[n + "_b"] = np.concatenate([gain - 1.0, np.zeros(d), gate])
    gain_f = 1.0 + 0.3 * g.standard_normal(d)
    Wa["norm_f_w"][:] = 0
    Wa["norm_f_b"] = np.concatenate([gain_f - 1.0, np.zeros(d), g.random(d)])
    t = 0.4
    Wr = {kk: vv for kk, vv in Wa.items() if not kk.startswith(("norm_f", "w_time", "b_time"))}
    Wr["b_in"] = Wa["b_in"] - O.sinusoid(t, d)  # cancel the additive time feature at t
    Wr["norm_f"] = gain_f
    Wr["layers"] = []
    for li, L in enumerate(Wa["layers"]):
        (g1, a1), (g2, a2) = gains[(li, "norm1")], gains[(li, "norm2")]
        Wr["layers"].append(dict(wq=L["wq"], wk=L["wk"], wv=L["wv"], wg=L["wg"], wu=L["wu"],
                                 wo=a1[:, None] * L["wo"].astype(np.float64),
                                 wd=a2[:, None] * L["wd"].astype(np.float64), norm1=g1, norm2=g2))
    Wa64, Wr64 = O.effective_weights(cfg_a, Wa), O.effective_weights(cfg_r, Wr)
    va = O.expert_velocity(cfg_a, Wa64, x0[0], t, k[0], v[0], st[0])
    vr = O.expert_velocity(cfg_r, Wr64, x0[0], t, k[0], v[0], st[0])
    assert O.rel_l2(va, vr) < 1e-13
    # the gates matter: equal gates give a different velocity
    Wr["layers"][0]["wo"] = Wa["layers"][0]["wo"]
    vr2 = O.expert_velocity(cfg_r, O.effective_weights(cfg_r, Wr), x0[0], t, k[0], v[0], st[0])
    assert O.rel_l2(va, vr2) > 1e-4


# --- P7b: the prefix stack, element by element ------------------------------------------
def _prefix_stack_scalar(cfg, Wp, tokens, theta=0.0):
    """The prefix encoder written out with scalar loops: per layer RMSNorm ->
    q, k, v -> (rotary positions) -> attention over the sequence -> O +
    residual -> RMSNorm -> GELU(gate) * up -> down + residual.  Returns the
    per-layer K and V (K unrotated)."""
    d, hq, hkv, dh = cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    T = tokens.shape[0]
    h = [[float(a) for a in row] for row in tokens]

    def rms(row, gain):
        r = 1.0 / math.sqrt(math.fsum(a * a for a in row) / d + cfg.rms_eps)
        return [row[i] * r * float(gain[i]) for i in range(d)]

    def rot(vec, pos):
        if not theta:
            return vec
        half = dh // 2
        out = list(vec)
        for i in range(half):
            a = pos * theta ** (-2.0 * i / dh)
            out[i] = vec[i] * math.cos(a) - vec[i + half] * math.sin(a)
            out[i + half] = vec[i + half] * math.cos(a) + vec[i] * math.sin(a)
        return out

    def gelu_s(z):
        return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))

    Ks, Vs = [], []
    for L in Wp["layers"]:
        u = [rms(h[t], L["norm1"]) for t in range(T)]
        q = [_mv_s(L["wq"], u[t]) for t in range(T)]
        k = [_mv_s(L["wk"], u[t]) for t in range(T)]
        v = [_mv_s(L["wv"], u[t]) for t in range(T)]
        Ks.append([[k[t][j * dh:(j + 1) * dh] for j in range(hkv)] for t in range(T)])
        Vs.append([[v[t][j * dh:(j + 1) * dh] for j in range(hkv)] for t in range(T)])
        o = [[0.0] * (hq * dh) for _ in range(T)]
        for t in range(T):
            for hh in range(hq):
                j = hh * hkv // hq
                qv = rot(q[t][hh * dh:(hh + 1) * dh], t)
                s = [math.fsum(a * b for a, b in zip(qv, rot(k[p][j * dh:(j + 1) * dh], p))) / math.sqrt(dh)
                     for p in range(T)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                z = math.fsum(e)
                for c in range(dh):
                    o[t][hh * dh + c] = math.fsum(e[p] / z * v[p][j * dh + c] for p in range(T))
        for t in range(T):
            att = _mv_s(L["wo"], o[t])
            h[t] = [h[t][i] + att[i] for i in range(d)]
            u2 = rms(h[t], L["norm2"])
            gte, up = _mv_s(L["wg"], u2), _mv_s(L["wu"], u2)
            mlp = _mv_s(L["wd"], [gelu_s(a) * b for a, b in zip(gte, up)])
            h[t] = [h[t][i] + mlp[i] for i in range(d)]
    return np.array(Ks), np.array(Vs)


@pytest.mark.parametrize("theta", [0.0, 100.0])
def test_prefix_stack_matches_scalar_loops(theta):
    # three layers, so that the first layer's attention + MLP body reaches the
    # K/V of the later ones (norm2 in place of norm1, a dropped residual or the
    # GELU on the wrong branch all change them); GQA with two query heads per
    # kv head
    cfg = _tiny(d_model=8, n_layers=3, n_q_heads=4, n_kv_heads=2, head_dim=4, d_mlp=12,
                rope_theta=theta)
    Wp, tokens = S.make_prefix_stack(cfg, 3)
    k, v = O.prefix_stack_kv(cfg, Wp, tokens[0])
    ks, vs = _prefix_stack_scalar(cfg, Wp, tokens[0], theta)
    assert k.shape == ks.shape == (3, 3, 2, 4)
    assert np.max(np.abs(k - ks)) < 1e-12 and np.max(np.abs(v - vs)) < 1e-12
    assert np.max(np.abs(k[2] - k[1])) > 1e-3  # the layers differ


# --- P12: robots are independent ------------------------------------------------
def test_batch_independence():
    cfg = _tiny(batch=3)
    W, k, v, x0, st = _inputs(cfg)
    full = O.denoise(cfg, W, k, v, x0, st)
    for b in range(3):
        one = O.denoise(cfg.replace(batch=1), W, k[b:b + 1], v[b:b + 1], x0[b:b + 1], st[b:b + 1])
        assert np.array_equal(one[0], full[b])
    assert O.rel_l2(full[0], full[1]) > 0.1


# --- P13: OCP E4M3FN codes -----------------------------------------------------------
def test_e4m3_code_table():
    # Values of the OCP 8-bit floating point (OFP8) E4M3 format.
    vals = O.e4m3_values()
    assert vals[0x00] == 0.0 and vals[0x01] == 2.0 ** -9 and vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x38] == 1.0 and vals[0x39] == 1.125
    assert vals[0x7E] == 448.0 and math.isnan(vals[0x7F]) and math.isnan(vals[0xFF])
    assert vals[0xB8] == -1.0 and vals[0xFE] == -448.0
    finite = vals[:127]
    assert np.all(np.diff(finite) > 0)


def test_e4m3_encode_rounding_and_saturation():
    vals = O.e4m3_values()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(O.e4m3_encode(vals[codes].astype(np.float32)), codes)
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             2.0 ** -10 * 1.0001: 0x01, 500.0: 0x7E, 464.0: 0x7E, 1e30: 0x7E,
             -1e9: 0xFE, -2.0 ** -11: 0x80, 240.0: 0x77, 232.0: 0x76, 248.0: 0x78}
    for x, c in cases.items():
        assert O.e4m3_encode(np.float32(x))[()] == c, (x, hex(c))


def test_e4m3_per_channel_quantisation_error_bound():
    g = np.random.default_rng(11)
    w = (g.standard_normal((64, 200)) * np.exp(g.standard_normal((64, 1)))).astype(np.float32)
    w[3] = 0
    codes, s = O.quantize_e4m3_per_channel(w)
    assert s[3] == 1.0 and np.all(codes[3] == 0)
    deq = O.e4m3_decode(codes) * s[:, None].astype(np.float64)
    q = np.abs(w.astype(np.float64) / s[:, None])
    # half a unit in the last place of the E4M3 grid at |q| (ulp 2^(e-3), min 2^-9)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_ulp = 0.5 * 2.0 ** (e - 3) * s[:, None] * (1 + 1e-6)
    assert np.all(np.abs(deq - w) <= half_ulp + 1e-30)
    assert np.all(np.max(np.abs(O.e4m3_decode(codes[[0, 1, 2]])), axis=1) == 448.0)


def test_fp8_prefix_cache_rows():
    # each (token, kv head) row of a [layers][T][Hkv][Dh] cache has its own
    # scale: a row of E4M3 values with max |x| = 448 is kept exactly, and any
    # row scaled by a power of two comes back scaled by the same power
    g = np.random.default_rng(13)
    vals = O.e4m3_values()
    ok = np.isfinite(vals) & (np.abs(vals) <= 448)
    rows = g.choice(vals[ok], size=(2, 5, 3, 32)).astype(np.float32)
    rows[..., 0] = 448.0
    assert np.array_equal(O.prefix_kv_e4m3(rows), rows)
    scaled = rows * np.float32(2.0) ** g.integers(-6, 6, size=(2, 5, 3, 1)).astype(np.float32)
    assert np.array_equal(O.prefix_kv_e4m3(scaled), scaled)
    # a generic cache: every element within half an E4M3 step of its row's grid
    x = (g.standard_normal((2, 7, 1, 64)) * np.exp(g.standard_normal((2, 7, 1, 1)))).astype(np.float32)
    deq = O.prefix_kv_e4m3(x)
    amax = np.max(np.abs(x), axis=-1, keepdims=True).astype(np.float64)
    assert np.all(np.abs(deq - x) <= amax / 448 * 2.0 ** -4 * np.maximum(np.abs(x) / amax * 448, 2.0 ** -6) * 1.01 + 1e-30)


def test_fp8_prefix_cache_changes_the_loop_only_through_the_prefix():
    cfg = _tiny(act_dtype="bf16", weight_dtype="bf16")
    W, k, v, x0, st = _inputs(cfg)
    a = O.denoise(cfg.replace(kv_fp8=True), W, k, v, x0, st)
    b = O.denoise(cfg, W, O.prefix_kv_e4m3(k), O.prefix_kv_e4m3(v), x0, st)
    assert np.array_equal(a, b)
    c = O.denoise(cfg, W, k, v, x0, st)
    assert 1e-5 < O.rel_l2(a, c) < 5e-2


def test_fp8_workload_uses_dequantised_matrices_only():
    cfg = _tiny(weight_dtype="fp8", act_dtype="bf16")
    W = S.make_weights(cfg)
    E = O.effective_weights(cfg, W)
    codes, s = O.quantize_e4m3_per_channel(W["layers"][0]["wg"])
    assert np.array_equal(E["layers"][0]["wg"], O.e4m3_decode(codes) * s[:, None].astype(np.float64))
    assert np.array_equal(E["w_in"], W["w_in"].astype(np.float64))
    assert np.array_equal(E["layers"][1]["norm1"], W["layers"][1]["norm1"].astype(np.float64))


# --- P14: W8A8 activations, 32-element blocks with power-of-two scales -----------------
def _pow2(x: int) -> Fraction:
    return Fraction(2) ** x


def test_mx_block_exponent_is_the_smallest_non_saturating_power():
    # X is the smallest integer with amax <= 448 2^X (checked in exact
    # rationals), floored at -126
    g = np.random.default_rng(21)
    amax = np.concatenate([np.exp(g.uniform(-80, 80, 400)),
                           448.0 * 2.0 ** np.arange(-20, 21), 448.0 * 2.0 ** np.arange(-20, 21) * (1 + 2.0 ** -40),
                           224.0 * 2.0 ** np.arange(-5, 6), [1.0, 1.75, 1.7500001, 2.0]])
    for a in amax:
        X = O.mx_block_exponent(a)
        fa = Fraction(float(a))
        assert fa <= 448 * _pow2(X), (a, X)
        assert X == -126 or fa > 448 * _pow2(X - 1), (a, X)
    assert O.mx_block_exponent(448.0) == 0 and O.mx_block_exponent(448.0 * (1 + 2.0 ** -40)) == 1
    assert O.mx_block_exponent(449.0) == 1 and O.mx_block_exponent(224.0) == -1
    assert O.mx_block_exponent(1.0) == -8 and O.mx_block_exponent(1.8) == -7
    assert O.mx_block_exponent(0.0) == -126 and O.mx_block_exponent(2.0 ** -140) == -126
    assert O.mx_block_exponent(448.0 * 2.0 ** -126) == -126 and O.mx_block_exponent(448.0 * 2.0 ** -125) == -125


def test_mx_identity_on_grid_values():
    # blocks of E4M3 values times 2^X whose largest magnitude lies in
    # (224, 448] come back unchanged, with that X and those codes
    g = np.random.default_rng(22)
    vals = O.e4m3_values()
    finite = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] != 0], np.uint8)
    top = np.array([c for c in finite if 224 < abs(vals[c]) <= 448], np.uint8)
    codes = g.choice(finite, size=(6, 128)).astype(np.uint8)
    codes[:, ::32] = g.choice(top, size=(6, 4))          # one top-binade value per block
    X = g.integers(-40, 40, size=(6, 4))
    a = O.e4m3_decode(codes).reshape(6, 4, 32) * np.exp2(X.astype(np.float64))[..., None]
    a = a.reshape(6, 128)
    c2, X2 = O.mx_quantize_e4m3(a)
    assert np.array_equal(X2, X) and np.array_equal(c2, codes)
    assert np.array_equal(O.mx_fake_quant(a), a)


def test_mx_half_step_error_bound_rounding_and_no_saturation():
    g = np.random.default_rng(23)
    a = g.standard_normal((40, 256)) * np.exp(g.uniform(-30, 30, (40, 8))).repeat(32, axis=1)
    a[3, 64:96] = 0.0                                     # an all-zero block
    codes, X = O.mx_quantize_e4m3(a)
    deq = O.mx_dequantize(codes, X)
    scale = np.exp2(X.astype(np.float64)).repeat(32, axis=1)
    q = np.abs(a) / scale
    assert np.all(q <= 448.0)                             # never beyond the E4M3 range
    blk = np.max(q.reshape(40, 8, 32), axis=-1)
    assert np.all((blk > 224.0) | (blk == 0.0))           # and no wasted binade
    assert X[3, 2] == -126 and np.all(codes[3, 64:96] == 0)
    # half a step of the E4M3 grid at |q| (2^(e-3) for normal q, 2^-9 below 2^-6)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    assert np.all(np.abs(deq - a) <= 0.5 * 2.0 ** (e - 3) * scale)
    # exact ties go to the even code: a block with max 448 (X = 0)
    ties = np.zeros(32)
    ties[:6] = [448.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -0.5625 * 2.0 ** -6]
    c, Xt = O.mx_quantize_e4m3(ties)
    assert Xt[0] == 0
    assert list(c[:6]) == [0x7E, 0x38, 0x3A, 0x00, 0x02, 0x84]
    # a block whose max would saturate under a floor(log2) rule is scaled one binade up
    c, Xs = O.mx_quantize_e4m3(np.full(32, 500.0))
    assert Xs[0] == 1 and np.all(O.e4m3_decode(c) == 256.0)


def test_mx_blocks_are_32_wide_and_independent():
    g = np.random.default_rng(24)
    a = g.standard_normal((3, 96))
    c0, X0 = O.mx_quantize_e4m3(a)
    b = a.copy()
    b[1, 40] = 1e6                                         # only row 1, block 1 changes
    c1, X1 = O.mx_quantize_e4m3(b)
    same = np.ones((3, 96), bool)
    same[1, 32:64] = False
    assert np.array_equal(c0[same], c1[same])
    assert X1[1, 1] != X0[1, 1] and np.array_equal(np.delete(X1.ravel(), 4), np.delete(X0.ravel(), 4))
    with pytest.raises(ValueError):
        O.mx_quantize_e4m3(np.ones((2, 48)))


@pytest.mark.parametrize("norm", ["rms", "ada"])
def test_w8a8_split_form_is_norm_then_gemm(norm):
    # with the quantiser replaced by the identity, the W8A8 form
    # rstd (a W^T) + shift W^T is the plain norm-then-GEMM
    cfg = _tiny() if norm == "rms" else _ada_cfg()
    W, k, v, x0, st = _inputs(cfg)
    W64 = O.effective_weights(cfg, W)
    ref = O.expert_velocity(cfg, W64, x0[0], 0.6, k[0], v[0], st[0])
    got = O.expert_velocity(cfg, W64, x0[0], 0.6, k[0], v[0], st[0], act_quant=lambda a: a)
    assert O.rel_l2(got, ref) < 1e-13


@pytest.mark.parametrize("norm", ["rms", "ada"])
def test_w8a8_quantises_all_four_gemm_operands(norm):
    # a quantiser that zeroes its operand removes every attention and MLP
    # contribution (only the Ada shifts survive in q, k, v, gate and up), so
    # with alpha = 0 for Ada the velocity is the head on the final norm of the
    # embedding; the operands are [S][d], [S][Hq Dh], [S][d], [S][F] per layer
    cfg = _tiny() if norm == "rms" else _ada_cfg()
    W, k, v, x0, st = _inputs(cfg)
    if norm == "ada":  # keep the shifts, zero every alpha
        for L in W["layers"]:
            for n in ("norm1", "norm2"):
                L[n + "_w"][2 * cfg.d_model:] = 0
                L[n + "_b"][2 * cfg.d_model:] = 0
    W64 = O.effective_weights(cfg, W)
    shapes = []

    def zero(a):
        shapes.append(a.shape)
        return np.zeros_like(a)

    t = 0.3
    got = O.expert_velocity(cfg, W64, x0[0], t, k[0], v[0], st[0], act_quant=zero)
    S_ = cfg.suffix
    one = [(S_, cfg.d_model), (S_, cfg.n_q_heads * cfg.head_dim), (S_, cfg.d_model), (S_, cfg.d_mlp)]
    assert shapes == one * cfg.n_layers
    act = O.linear(x0[0], W64["w_in"], W64["b_in"])
    if norm == "rms":
        act = act + O.sinusoid(t, cfg.d_model)
        hf = O.rmsnorm(act, W64["norm_f"], cfg.rms_eps)
    else:
        _, (gf, bf, _) = O.ada_modulation(cfg, W64, t)
        hf = O.ada_rmsnorm(act, gf, bf, cfg.rms_eps)
    want = O.linear(hf, W64["w_out"], W64["b_out"])
    assert O.rel_l2(got, want) < 1e-13
    if norm == "rms":  # the alpha-free RMS expert: any residual contribution would show
        ref = O.expert_velocity(cfg, W64, x0[0], t, k[0], v[0], st[0])
        assert O.rel_l2(ref, want) > 1e-2


def test_w8a8_loop_is_close_to_w8a16():
    cfg = _tiny(weight_dtype="fp8", act_dtype="bf16")
    W, k, v, x0, st = _inputs(cfg)
    a = O.denoise(cfg.replace(w8a8=True), W, k, v, x0, st)
    b = O.denoise(cfg, W, k, v, x0, st)
    assert 1e-4 < O.rel_l2(a, b) < 5e-2


# --- structure: suffix rows, state token, time only on action rows --------------------
def test_state_token_reaches_actions_only_through_attention():
    cfg = TINY
    W, k, v, x0, st = _inputs(cfg)
    a = O.denoise(cfg, W, k, v, x0, st)
    b = O.denoise(cfg, W, k, v, x0, st * 0 + 3.0)
    assert O.rel_l2(a, b) > 1e-3
    for L in W["layers"]:
        L["wk"][:] = 0  # uniform attention: still reads V of the state row
    c = O.denoise(cfg, W, k, v, x0, st)
    for L in W["layers"]:
        L["wv"][:] = 0
        L["wo"][:] = 0
    d1 = O.denoise(cfg, W, k, v, x0, st)
    d2 = O.denoise(cfg, W, k, v, x0, st * 0 + 3.0)
    assert np.array_equal(d1, d2) and O.rel_l2(c, d1) > 1e-4


def test_empty_prefix_attends_within_suffix_only():
    cfg = TINY
    W, k, v, x0, st = _inputs(cfg)
    e = O.denoise(cfg, W, k[:, :, :0], v[:, :, :0], x0, st)
    assert np.all(np.isfinite(e)) and O.rel_l2(e, O.denoise(cfg, W, k, v, x0, st)) > 1e-3
