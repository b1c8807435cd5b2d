"""fp64 CPU oracle of the flow-matching action-expert Euler denoise loop.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  It is plain NumPy in float64,
written from the pages' description of the method; it shares no code,
table or constant with the GPU library.

What the method computes, and where the pages fix it
----------------------------------------------------
* A flow-matching policy turns noise into an action chunk by integrating a
  learned velocity field with explicit Euler steps, 10 of them: FlowEdge
  README, "Installation" (the flow sampler run as "euler 10"), and the
  realtime-vla write-up, "The latency table, and what it assumes" (10 flow
  steps per prediction).
* Each velocity evaluation runs the action expert over the suffix tokens
  (one state token plus the noisy action chunk).  Those tokens attend to the
  vision/prompt prefix, whose keys and values do not depend on the flow
  time, so they are computed once and reused by every step: Reflex abstract
  (Timestep-Invariance Property; full-batch-equivalent attention outputs).
* The prefix context splits into a static region (prompt), a sliding window
  of camera frames updated in O(1) per frame, and the dynamic suffix:
  Reflex abstract.
* AdaRMSNorm takes its modulation from the flow phase: Reflex abstract.
* State is a 32-vector and the noise is (chunk, 32): realtime-vla write-up,
  "Copying an inference file into your own project".
* fp8 execution of the weights: InstinctFlash README, "Load a model"
  (precision="fp8") and "Architecture" (HARDWARE layer, fp8/int8).

Readings taken where the pages are silent
-----------------------------------------
* Time runs from t=1 (noise) to t=0 (action); dt = -1/N; the velocity at
  step k is evaluated at the left end t_k = 1 - k/N, computed directly.  A
  caller may instead give the step schedule (step schedules are chosen
  separately from the model: InstinctFlash README, "Load a model"): N + 1
  times 1 = s_0 > ... > s_N = 0, step k evaluating at s_k with dt_k =
  s_(k+1) - s_k.
* Sinusoidal time features: [sin(t w_j) | cos(t w_j)], w_j = 10000^(-j/(D/2)),
  j < D/2, t unscaled.  Additive experts add the d-wide feature to the
  action tokens only (not the state token); the AdaRMSNorm expert takes
  time only through its norms.
* AdaRMSNorm: c = SiLU(W_t tau_256(t) + b_t); each norm n has its own linear
  giving (gamma, beta, alpha) = split3(W_n c + b_n); the norm output is
  rms(h) * (1 + gamma) + beta and alpha scales the residual branch it feeds.
  The final norm uses gamma and beta only.
* RMSNorm: h / sqrt(mean(h^2) + eps) * g.  GELU is the exact erf form.
* Transformer linears have no bias; the action-in, state, action-out, time
  and modulation linears do.
* Attention: scale 1/sqrt(head_dim), no mask (full to the prefix,
  bidirectional in the suffix), no positions; query head h reads KV head
  floor(h * Hkv / Hq).
* fp8 weights are OCP E4M3FN with one fp32 scale per output channel,
  s = max|w| / 448 (1 when the row is zero), codes = round-to-nearest-even
  of the fp32 quotient w / s, saturating at +-448.  The loop then uses the
  dequantised weights code * s exactly.
* W8A8 (cfg.w8a8, fp8 weights only): the activation operand of each of the
  four weight GEMMs of a layer is quantised as well, in blocks of 32
  consecutive elements along the reduction dimension of each row, with one
  power-of-two scale per block (the block layout of the OCP Microscaling
  formats, E4M3 elements with an E8M0 scale).  The block exponent X is the
  smallest integer with max|a| <= 448 * 2^X (so no element saturates),
  floored at -126; codes are the E4M3 values of a / 2^X rounded to nearest,
  ties to even.  The two norm-fed GEMMs quantise the gain-scaled residual
  a = h * g (RMSNorm gain g, or 1 + gamma for AdaRMSNorm) and apply the
  row's 1/rms factor and the Ada shift beta after the product:
  y = rstd * (Q(a) W^T) + beta W^T, which is the unquantised norm-then-GEMM
  by linearity.  The attention output and the GELU gate product are
  quantised as they are.  The final norm and the action head stay unquantised.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "time_grid", "sinusoid", "linear", "rms_inv", "rmsnorm", "ada_rmsnorm",
    "silu", "gelu", "softmax_rows", "attention", "masked_attention", "rope",
    "ada_modulation", "euler", "heun", "ab2", "integrate", "expert_velocity", "denoise", "denoise_robot",
    "e4m3_values", "e4m3_decode", "e4m3_encode", "quantize_e4m3_per_channel",
    "effective_weights", "prefix_kv_e4m3", "FP8_MATRICES", "PrefixRing", "prefix_stack_kv",
    "joint_velocity", "denoise_joint", "rel_l2", "max_abs",
    "MX_BLOCK", "mx_block_exponent", "mx_quantize_e4m3", "mx_dequantize", "mx_fake_quant",
]

F64 = np.float64


# ---------------------------------------------------------------------------
# Schedule and time features
# ---------------------------------------------------------------------------
def time_grid(n_steps: int, schedule: Optional[Sequence[float]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Euler schedule: the times t_k and steps dt_k, k = 0..N-1.  Default
    t_k = 1 - k/N and dt_k = -1/N (see module docstring: direction and
    left-endpoint evaluation are this code's reading; the step count is the
    pages' 10 flow steps).  With a schedule s (N + 1 times from 1 down to 0,
    rounded to fp32 as at the library boundary): t_k = s_k, dt_k = s_(k+1) - s_k."""
    if schedule is None:
        k = np.arange(n_steps, dtype=F64)
        return 1.0 - k / n_steps, np.full(n_steps, -1.0 / n_steps)
    s = np.asarray(schedule, dtype=np.float32).astype(F64)
    if s.shape != (n_steps + 1,) or s[0] != 1.0 or s[-1] != 0.0 or not np.all(np.diff(s) < 0):
        raise ValueError("schedule: n_steps + 1 strictly decreasing times from 1 to 0")
    return s[:-1], np.diff(s)


def sinusoid(t: float, dim: int) -> np.ndarray:
    """Sinusoidal features of a scalar time: [sin(t w) | cos(t w)]."""
    half = dim // 2
    j = np.arange(half, dtype=F64)
    w = 10000.0 ** (-j / half)
    return np.concatenate([np.sin(t * w), np.cos(t * w)])


# ---------------------------------------------------------------------------
# Primitives
# ---------------------------------------------------------------------------
def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W^T (+ b), W stored [out][in]."""
    y = np.asarray(x, F64) @ np.asarray(w, F64).T
    if b is not None:
        y = y + np.asarray(b, F64)
    return y


def rms_inv(h: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean over the last axis of h^2 + eps)."""
    return 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return h * rms_inv(h, eps) * np.asarray(g, F64)


def ada_rmsnorm(h, gamma, beta, eps: float) -> np.ndarray:
    """AdaRMSNorm (Reflex abstract): normalised h, scaled by (1 + gamma) and
    shifted by beta, both taken from the flow-phase embedding."""
    return h * rms_inv(h, eps) * (1.0 + gamma) + beta


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = x/2 (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Unmasked multi-query attention.

    q [Sq][Hq][Dh], k and v [Tk][Hkv][Dh]; query head h uses KV head
    floor(h*Hkv/Hq); scores are scaled by 1/sqrt(Dh).  Returns [Sq][Hq][Dh].
    """
    sq, hq, dh = q.shape
    hkv = k.shape[1]
    out = np.empty((sq, hq, dh), F64)
    scale = 1.0 / math.sqrt(dh)
    for h in range(hq):
        j = (h * hkv) // hq
        p = softmax_rows((q[:, h, :] @ k[:, j, :].T) * scale)
        out[:, h, :] = p @ v[:, j, :]
    return out


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary position embedding of x [n][heads][Dh] at positions [n]: with
    half = Dh / 2, the pair (i, i + half) of every head turns by the angle
    position * theta^(-2 i / Dh) (the rotate-half pairing).  A reading: the
    pages name no positional encoding; Pi0-style experts rotate q and k."""
    x = np.asarray(x, F64)
    dh = x.shape[-1]
    half = dh // 2
    ang = np.asarray(positions, F64)[:, None] * (float(theta) ** (-2.0 * np.arange(half) / dh))[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def masked_attention(q, k, v, allowed: np.ndarray) -> np.ndarray:
    """Attention with a boolean [Sq][Tk] mask (True = may attend).  Written
    separately from `attention` so that the cached-prefix path can be checked
    against a joint-sequence recompute."""
    sq, hq, dh = q.shape
    hkv = k.shape[1]
    out = np.zeros((sq, hq, dh), F64)
    for h in range(hq):
        j = (h * hkv) // hq
        s = np.einsum("qd,kd->qk", q[:, h, :], k[:, j, :]) / math.sqrt(dh)
        s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - m), 0.0)
        out[:, h, :] = np.einsum("qk,kd->qd", e / e.sum(axis=1, keepdims=True), v[:, j, :])
    return out


def rel_l2(a, ref) -> float:
    a, ref = np.asarray(a, F64), np.asarray(ref, F64)
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


def max_abs(a, ref) -> float:
    return float(np.max(np.abs(np.asarray(a, F64) - np.asarray(ref, F64))))


# ---------------------------------------------------------------------------
# fp8 E4M3FN (OCP) weights
# ---------------------------------------------------------------------------
FP8_MATRICES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def _e4m3_value(code: int) -> float:
    """Value of an OCP E4M3FN code: 1 sign, 4 exponent bits (bias 7),
    3 mantissa bits, subnormals at exponent 0, 0x7F/0xFF NaN, no infinity."""
    sgn = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sgn * m * 2.0 ** -9
    return sgn * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_values() -> np.ndarray:
    """The 256 code values, indexed by code."""
    return np.array([_e4m3_value(c) for c in range(256)], F64)


_POS = e4m3_values()[:127]  # codes 0..126: 0 .. 448, strictly increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return e4m3_values()[np.asarray(codes, np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to the even code,
    saturating at +-448; the sign bit follows the sign of x (so negative
    values that round to zero give 0x80)."""
    return _e4m3_encode_f64(np.asarray(x, np.float32).astype(F64))


def _e4m3_encode_f64(x: np.ndarray) -> np.ndarray:
    """E4M3FN codes of float64 values (nearest, ties to the even code,
    saturating at +-448), with no intermediate rounding."""
    x = np.asarray(x, F64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (mag | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


MX_BLOCK = 32
MX_MIN_EXP = -126


def mx_block_exponent(amax: float) -> int:
    """Exponent X of a block's power-of-two scale: the smallest integer with
    amax <= 448 * 2^X, floored at -126 (an all-zero block gets -126)."""
    amax = float(amax)
    if not amax > 0.0:
        return MX_MIN_EXP
    _, e = math.frexp(amax)          # amax = f 2^e, 0.5 <= f < 1
    x = e - 1 - 8                    # 448 2^x >= 256 2^x > amax / 2 ...
    while amax > 448.0 * 2.0 ** x:   # ... so at most two steps up
        x += 1
    while x - 1 >= MX_MIN_EXP and amax <= 448.0 * 2.0 ** (x - 1):
        x -= 1
    return max(x, MX_MIN_EXP)


def mx_quantize_e4m3(a) -> Tuple[np.ndarray, np.ndarray]:
    """Block quantisation of a[..., K] (K a multiple of 32): every run of 32
    consecutive elements along the last axis shares the scale 2^X of
    mx_block_exponent(max |run|); codes are E4M3 of a / 2^X (exact division,
    nearest, ties to even; never saturating, by the choice of X).  Returns
    (codes uint8 [..., K], X int32 [..., K / 32])."""
    a = np.asarray(a, F64)
    K = a.shape[-1]
    if K % MX_BLOCK:
        raise ValueError(f"reduction length {K} is not a multiple of {MX_BLOCK}")
    blocks = a.reshape(a.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    X = np.vectorize(mx_block_exponent, otypes=[np.int32])(amax) if amax.size else amax.astype(np.int32)
    codes = _e4m3_encode_f64(blocks / np.exp2(X.astype(F64))[..., None])
    return codes.reshape(a.shape), X


def mx_dequantize(codes, X) -> np.ndarray:
    """code value * 2^X of the block each element belongs to, in float64."""
    codes = np.asarray(codes, np.uint8)
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (codes.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (v * np.exp2(np.asarray(X, F64))[..., None]).reshape(codes.shape)


def mx_fake_quant(a) -> np.ndarray:
    """What a W8A8 GEMM consumes of the activation a: its block-quantised
    value, dequantised (float64)."""
    return mx_dequantize(*mx_quantize_e4m3(a))


def quantize_e4m3_per_channel(w) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel E4M3 quantisation of W[out][in]: scale
    s = max|w_row| / 448 in float32 (1 for an all-zero row), codes of the
    float32 quotient w / s.  Returns (codes uint8 [out][in], s float32 [out])."""
    w = np.asarray(w, np.float32)
    amax = np.max(np.abs(w), axis=1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (w / s[:, None]).astype(np.float32)
    return e4m3_encode(q), s


def prefix_kv_e4m3(kv) -> np.ndarray:
    """An fp8 prefix cache as the loop reads it: every (token, kv head) row
    of K or V [..][Dh] quantised like a weight row (scale = row max / 448 in
    float32, E4M3 codes of the float32 quotient), returned dequantised in
    float64 (code * scale).  The suffix K/V of each step stay unquantised."""
    kv = np.asarray(kv, np.float32)
    codes, s = quantize_e4m3_per_channel(kv.reshape(-1, kv.shape[-1]))
    return (e4m3_decode(codes) * s.astype(F64)[:, None]).reshape(kv.shape)


def effective_weights(cfg, W: dict) -> dict:
    """Weights as the loop uses them, in float64.  For an fp8 workload the
    seven per-layer matrices are replaced by their dequantised fp8 values
    (code * scale); everything else converts exactly."""
    out = {k: np.asarray(v, F64) for k, v in W.items() if k != "layers"}
    out["layers"] = []
    for L in W["layers"]:
        E = {}
        for k, v in L.items():
            if cfg.weight_dtype == "fp8" and k in FP8_MATRICES:
                codes, s = quantize_e4m3_per_channel(v)
                E[k] = e4m3_decode(codes) * s.astype(F64)[:, None]
            else:
                E[k] = np.asarray(v, F64)
        out["layers"].append(E)
    return out


# ---------------------------------------------------------------------------
# The action expert's velocity and the Euler loop
# ---------------------------------------------------------------------------
def ada_modulation(cfg, W: dict, t: float):
    """(gamma, beta, alpha) of every norm at flow time t: per layer
    [(norm1), (norm2)], then the final norm."""
    c = silu(linear(sinusoid(t, cfg.time_dim), W["w_time"], W["b_time"]))
    d = cfg.d_model

    def split(wn, bn):
        m = linear(c, wn, bn)
        return m[:d], m[d:2 * d], m[2 * d:]

    per_layer = [(split(L["norm1_w"], L["norm1_b"]), split(L["norm2_w"], L["norm2_b"]))
                 for L in W["layers"]]
    return per_layer, split(W["norm_f_w"], W["norm_f_b"])


def _norm(cfg, h, gain, mod):
    if cfg.norm == "rms":
        return rmsnorm(h, gain, cfg.rms_eps)
    gamma, beta, _ = mod
    return ada_rmsnorm(h, gamma, beta, cfg.rms_eps)


def _norm_parts(cfg, h, gain, mod):
    """The norm taken apart for a quantised GEMM: (1/rms(h) [S][1], the
    gain-scaled residual a [S][d], the shift or None), with
    norm(h) = (1/rms) a + shift."""
    if cfg.norm == "rms":
        return rms_inv(h, cfg.rms_eps), h * np.asarray(gain, F64), None
    gamma, beta, _ = mod
    return rms_inv(h, cfg.rms_eps), h * (1.0 + gamma), beta


def _norm_gemms(parts, quant, ws):
    """The GEMMs of one norm output on its quantised operand: for each W,
    (1/rms) (Q(a) W^T) (+ shift W^T)."""
    rstd, a, shift = parts
    aq = quant(a)
    out = []
    for w in ws:
        y = rstd * linear(aq, w)
        out.append(y if shift is None else y + linear(shift, w))
    return out


def expert_velocity(cfg, W: dict, x: np.ndarray, t: float, k_pre: np.ndarray,
                    v_pre: np.ndarray, state: Optional[np.ndarray], return_kv: bool = False,
                    act_quant: Optional[Callable[[np.ndarray], np.ndarray]] = None):
    """Velocity v(x, t) of one robot.

    x [chunk][A]; k_pre, v_pre [layers][T][Hkv][Dh] in logical order; state
    [state_dim] or None.  W holds float64 weights (see effective_weights).
    Returns v [chunk][A] (and, with return_kv, the suffix K and V of every
    layer, [layers][S][Hkv][Dh]).

    Suffix mask: none, or with cfg.state_causal the block-causal suffix of
    Pi0-style experts (a reading; the pages fix no suffix mask): the state
    token attends to the prefix and itself, the action tokens to everything.
    With cfg.rope_theta the suffix q and k are rotated (rope) at positions
    T + s; k_pre is then the rotated cache (see denoise).

    W8A8 (cfg.w8a8): every weight GEMM of a layer multiplies the quantised
    activation act_quant(a) (default mx_fake_quant), the norm-fed ones in
    the split form of _norm_gemms.  Passing act_quant forces that form.
    """
    if act_quant is None and getattr(cfg, "w8a8", False):
        act_quant = mx_fake_quant
    S_has = 1 if cfg.state_dim else 0
    hq, hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    act = linear(np.asarray(x, F64), W["w_in"], W["b_in"])
    if cfg.norm == "rms":
        act = act + sinusoid(t, cfg.d_model)
    if S_has:
        h = np.vstack([linear(np.asarray(state, F64), W["w_state"], W["b_state"])[None], act])
    else:
        h = act
    S = h.shape[0]
    T = np.asarray(k_pre[0]).shape[0] if len(k_pre) else 0
    causal = bool(getattr(cfg, "state_causal", False)) and S_has
    theta = float(getattr(cfg, "rope_theta", 0.0))
    if causal:
        allowed = np.ones((S, T + S), bool)
        allowed[0, T + 1:] = False
    mods, mod_f = ada_modulation(cfg, W, t) if cfg.norm == "ada" else (None, None)
    ks, vs = [], []
    for li, L in enumerate(W["layers"]):
        m1, m2 = mods[li] if mods else (None, None)
        if act_quant is None:
            u = _norm(cfg, h, L.get("norm1"), m1)
            q, k, v = linear(u, L["wq"]), linear(u, L["wk"]), linear(u, L["wv"])
        else:
            q, k, v = _norm_gemms(_norm_parts(cfg, h, L.get("norm1"), m1), act_quant,
                                  (L["wq"], L["wk"], L["wv"]))
        q, k, v = q.reshape(S, hq, dh), k.reshape(S, hkv, dh), v.reshape(S, hkv, dh)
        if theta:  # suffix row s sits at position T + s, after the prefix
            q, k = rope(q, T + np.arange(S), theta), rope(k, T + np.arange(S), theta)
        ks.append(k)
        vs.append(v)
        K = np.concatenate([np.asarray(k_pre[li], F64), k], axis=0)
        V = np.concatenate([np.asarray(v_pre[li], F64), v], axis=0)
        o = (masked_attention(q, K, V, allowed) if causal else attention(q, K, V)).reshape(S, hq * dh)
        a1 = m1[2] if m1 else 1.0
        h = h + a1 * linear(o if act_quant is None else act_quant(o), L["wo"])
        if act_quant is None:
            u = _norm(cfg, h, L.get("norm2"), m2)
            gt, up = linear(u, L["wg"]), linear(u, L["wu"])
        else:
            gt, up = _norm_gemms(_norm_parts(cfg, h, L.get("norm2"), m2), act_quant, (L["wg"], L["wu"]))
        z = gelu(gt) * up
        a2 = m2[2] if m2 else 1.0
        h = h + a2 * linear(z if act_quant is None else act_quant(z), L["wd"])
    u = _norm(cfg, h[S_has:], W.get("norm_f"), mod_f)
    out = linear(u, W["w_out"], W["b_out"])
    return (out, np.stack(ks), np.stack(vs)) if return_kv else out


def euler(velocity: Callable[[np.ndarray, float], np.ndarray], x0: np.ndarray,
          n_steps: int, schedule: Optional[Sequence[float]] = None) -> np.ndarray:
    """x_{k+1} = x_k + dt_k * v(x_k, t_k) over the schedule of time_grid."""
    ts, dts = time_grid(n_steps, schedule)
    x = np.asarray(x0, F64).copy()
    for t, dt in zip(ts, dts):
        x = x + dt * velocity(x, float(t))
    return x


def heun(velocity: Callable[[np.ndarray, float], np.ndarray], x0: np.ndarray,
         n_steps: int, schedule: Optional[Sequence[float]] = None) -> np.ndarray:
    """Heun's method (the explicit trapezoidal rule) over the same schedule:
    v1 = v(x_k, t_k); v2 = v(x_k + dt_k v1, t_(k+1)); x_(k+1) = x_k +
    dt_k (v1 + v2) / 2.  Every step, the last included, evaluates v at its
    right end t_(k+1) as well (t = 0 on the last step)."""
    ts, dts = time_grid(n_steps, schedule)
    t_next = np.append(ts[1:], 0.0)  # t_(k+1): the next grid time, 0 after the last
    x = np.asarray(x0, F64).copy()
    for t, tn, dt in zip(ts, t_next, dts):
        v1 = velocity(x, float(t))
        v2 = velocity(x + dt * v1, float(tn))
        x = x + dt * 0.5 * (v1 + v2)
    return x


def ab2(velocity: Callable[[np.ndarray, float], np.ndarray], x0: np.ndarray,
        n_steps: int, schedule: Optional[Sequence[float]] = None) -> np.ndarray:
    """The two-step Adams-Bashforth method (a linear multistep sampler, one
    evaluation per step) over the same schedule.  Step k integrates, over
    [t_k, t_(k+1)], the line through the last two velocities (t_(k-1),
    v_(k-1)) and (t_k, v_k): with h_k = dt_k and r = h_k / (2 h_(k-1)),
    x_(k+1) = x_k + h_k ((1 + r) v_k - r v_(k-1)).  The first step, with one
    velocity only, is an Euler step."""
    ts, dts = time_grid(n_steps, schedule)
    x = np.asarray(x0, F64).copy()
    v_prev, h_prev = None, None
    for t, h in zip(ts, dts):
        v = velocity(x, float(t))
        if v_prev is None:
            x = x + h * v
        else:
            r = h / (2.0 * h_prev)
            x = x + h * ((1.0 + r) * v - r * v_prev)
        v_prev, h_prev = v, h
    return x


def integrate(cfg, velocity, x0) -> np.ndarray:
    """The workload's sampler (cfg.sampler: "euler", the default, "heun" or
    "ab2")."""
    step = {"euler": euler, "heun": heun, "ab2": ab2}[getattr(cfg, "sampler", "euler")]
    return step(velocity, x0, cfg.n_steps, getattr(cfg, "t_schedule", None))


def denoise_robot(cfg, W64: dict, k_pre, v_pre, noise, state) -> np.ndarray:
    """One robot's action chunk x at t=0 from its noise at t=1."""
    return integrate(cfg, lambda x, t: expert_velocity(cfg, W64, x, t, k_pre, v_pre, state), noise)


def denoise(cfg, W: dict, k_pre, v_pre, noise, state=None,
            robots: Optional[Sequence[int]] = None) -> np.ndarray:
    """Batch of independent robots.  k_pre/v_pre [B][layers][T][Hkv][Dh],
    noise [B][chunk][A], state [B][state_dim] or None.  `robots` picks a
    subset (the result then has len(robots) rows)."""
    W64 = effective_weights(cfg, W)
    idx = range(noise.shape[0]) if robots is None else robots
    theta = float(getattr(cfg, "rope_theta", 0.0))
    if theta:  # the cache holds prefix K rotated at its token positions 0..T-1
        k_pre = [np.stack([rope(kl, np.arange(kl.shape[0]), theta) for kl in k]) for k in k_pre]
    if getattr(cfg, "kv_fp8", False):  # the prefix cache held in fp8
        k_pre, v_pre = [prefix_kv_e4m3(k) for k in k_pre], [prefix_kv_e4m3(v) for v in v_pre]
    return np.stack([denoise_robot(cfg, W64, k_pre[b], v_pre[b], noise[b],
                                   None if state is None else state[b]) for b in idx])


# ---------------------------------------------------------------------------
# Streaming prefix: static prompt + sliding window of frames (Reflex abstract)
# ---------------------------------------------------------------------------
class PrefixRing:
    """Static region plus a ring of `n_frames` frame slots.  `set` takes the
    logical order (static, then frames oldest to newest); `append` overwrites
    the oldest frame in O(1); `logical` returns the prefix in logical order."""

    def __init__(self, static_tokens: int, frame_tokens: int, n_frames: int):
        self.ns, self.nf, self.F = static_tokens, frame_tokens, n_frames
        self.static = None
        self.slots: List[np.ndarray] = []
        self.head = 0

    def set(self, kv: np.ndarray):
        """kv [layers][static + F*frame][...]."""
        self.static = kv[:, :self.ns]
        self.slots = [kv[:, self.ns + j * self.nf: self.ns + (j + 1) * self.nf]
                      for j in range(self.F)]
        self.head = 0

    def append(self, frame: np.ndarray):
        self.slots[self.head] = frame
        self.head = (self.head + 1) % self.F

    def logical(self) -> np.ndarray:
        order = [self.slots[(self.head + j) % self.F] for j in range(self.F)]
        return np.concatenate([self.static] + order, axis=1)


# ---------------------------------------------------------------------------
# Joint-sequence recompute (checks the timestep-invariant cached prefix)
# ---------------------------------------------------------------------------
def _prefix_layer_qkv(cfg, Lp, hp):
    T = hp.shape[0]
    u = rmsnorm(hp, Lp["norm1"], cfg.rms_eps)
    return (linear(u, Lp["wq"]).reshape(T, cfg.n_q_heads, cfg.head_dim),
            linear(u, Lp["wk"]).reshape(T, cfg.n_kv_heads, cfg.head_dim),
            linear(u, Lp["wv"]).reshape(T, cfg.n_kv_heads, cfg.head_dim))


def _rot(cfg, x, pos):
    theta = float(getattr(cfg, "rope_theta", 0.0))
    return rope(x, pos, theta) if theta else x


def _prefix_layer_rest(cfg, Lp, hp, o):
    hp = hp + linear(o.reshape(hp.shape[0], -1), Lp["wo"])
    u = rmsnorm(hp, Lp["norm2"], cfg.rms_eps)
    return hp + linear(gelu(linear(u, Lp["wg"])) * linear(u, Lp["wu"]), Lp["wd"])


def prefix_stack_kv(cfg, Wp: dict, tokens: np.ndarray):
    """Run a prefix encoder (own RMSNorm transformer weights; prefix tokens
    attend to the prefix only) and return its per-layer K and V,
    [layers][T][Hkv][Dh]: the cache the denoise loop reads."""
    hp = np.asarray(tokens, F64)
    Ks, Vs = [], []
    pos = np.arange(hp.shape[0])
    for Lp in Wp["layers"]:
        q, k, v = _prefix_layer_qkv(cfg, Lp, hp)
        Ks.append(k)  # unrotated: the cache input (the loop rotates it)
        Vs.append(v)
        hp = _prefix_layer_rest(cfg, Lp, hp, attention(_rot(cfg, q, pos), _rot(cfg, k, pos), v))
    return np.stack(Ks), np.stack(Vs)


def joint_velocity(cfg, W64: dict, Wp: dict, tokens, x, t, state) -> np.ndarray:
    """Velocity from a full recompute of [prefix tokens | suffix] as one
    sequence, every call.  Prefix rows use the prefix weights and see only
    prefix keys; suffix rows use the expert weights and see every key."""
    S_has = 1 if cfg.state_dim else 0
    hq, hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    hp = np.asarray(tokens, F64)
    T = hp.shape[0]
    act = linear(np.asarray(x, F64), W64["w_in"], W64["b_in"])
    if cfg.norm == "rms":
        act = act + sinusoid(t, cfg.d_model)
    hs = act if not S_has else np.vstack(
        [linear(np.asarray(state, F64), W64["w_state"], W64["b_state"])[None], act])
    S = hs.shape[0]
    allowed = np.ones((T + S, T + S), bool)
    allowed[:T, T:] = False
    if getattr(cfg, "state_causal", False) and S_has:  # see expert_velocity
        allowed[T, T + 1:] = False
    mods, mod_f = ada_modulation(cfg, W64, t) if cfg.norm == "ada" else (None, None)
    for li, (L, Lp) in enumerate(zip(W64["layers"], Wp["layers"])):
        m1, m2 = mods[li] if mods else (None, None)
        qp, kp, vp = _prefix_layer_qkv(cfg, Lp, hp)
        qp, kp = _rot(cfg, qp, np.arange(T)), _rot(cfg, kp, np.arange(T))
        u = _norm(cfg, hs, L.get("norm1"), m1)
        qs = linear(u, L["wq"]).reshape(S, hq, dh)
        ks = linear(u, L["wk"]).reshape(S, hkv, dh)
        vs = linear(u, L["wv"]).reshape(S, hkv, dh)
        qs, ks = _rot(cfg, qs, T + np.arange(S)), _rot(cfg, ks, T + np.arange(S))
        o = masked_attention(np.concatenate([qp, qs]), np.concatenate([kp, ks]),
                             np.concatenate([vp, vs]), allowed)
        hp = _prefix_layer_rest(cfg, Lp, hp, o[:T])
        a1 = m1[2] if m1 else 1.0
        hs = hs + a1 * linear(o[T:].reshape(S, hq * dh), L["wo"])
        u = _norm(cfg, hs, L.get("norm2"), m2)
        a2 = m2[2] if m2 else 1.0
        hs = hs + a2 * linear(gelu(linear(u, L["wg"])) * linear(u, L["wu"]), L["wd"])
    u = _norm(cfg, hs[S_has:], W64.get("norm_f"), mod_f)
    return linear(u, W64["w_out"], W64["b_out"])


def denoise_joint(cfg, W: dict, Wp: dict, tokens, noise, state=None) -> np.ndarray:
    """Euler loop whose every step recomputes the whole joint sequence."""
    W64 = effective_weights(cfg, W)
    Wp64 = {"layers": [{k: np.asarray(v, F64) for k, v in L.items()} for L in Wp["layers"]]}
    out = []
    for b in range(noise.shape[0]):
        st = None if state is None else state[b]
        out.append(integrate(cfg, lambda x, t: joint_velocity(cfg, W64, Wp64, tokens[b], x, t, st), noise[b]))
    return np.stack(out)
