"""Seeded synthetic inputs for the flow-matching action-expert denoise loop.

This module is the one piece shared by the fp64 oracle's callers and the GPU
library's callers.  It holds workload shapes and random draws only: no step
of the denoising method is computed here.  Every tensor is drawn in float64
from its own PCG64 stream and rounded once to the storage dtype of the
workload (float32 for the fp32 workload, bfloat16 values held in float32
arrays otherwise).

Shapes follow the pages' workloads:
  * realtime-vla write-up, "Copying an inference file into your own project":
    state is a 32-vector and the noise is (chunk, 32).
  * realtime-vla write-up, "The latency table, and what it assumes": one to
    three camera views, a 20-token or empty prompt, chunk 50 or 63, 10 flow
    steps.  A 224x224 view becomes 256 image tokens of prefix.
  * Reflex abstract: static / sliding / dynamic context regions, updated in
    O(1) per frame; AdaRMSNorm gated on flow phase.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "FMConfig", "WORKLOADS", "workload", "rng", "round_bf16", "round_to",
    "make_weights", "make_prefix", "make_noise", "make_state", "make_frame",
    "make_tick_noise", "make_prefix_stack",
]

# Stream ids of the seeded generators.
STREAM_WEIGHTS, STREAM_PREFIX, STREAM_NOISE, STREAM_STATE = 0, 1, 2, 3
STREAM_TICK0 = 4  # frame of tick i: stream 4 + 2(i + n_frames); its noise: the next one
STREAM_PREFIX_STACK = 100000  # own weights + tokens of a tiny prefix encoder


@dataclasses.dataclass(frozen=True)
class FMConfig:
    """One denoise-loop workload.  Field names match the C struct fm_config."""
    name: str
    seed: int
    d_model: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_mlp: int
    action_dim: int
    chunk: int
    state_dim: int          # 0: no state token in the suffix
    batch: int
    n_steps: int
    prefix_static: int      # static region (prompt, or the whole prefix)
    frame_tokens: int       # tokens per sliding-window frame (0: no ring)
    n_frames: int           # frames held in the sliding window (0: no ring)
    prefix_len: int         # tokens the workload loads with set_prefix_kv
    norm: str               # "rms" or "ada"
    time_dim: int           # additive: == d_model; ada: sinusoid width
    weight_dtype: str       # "f32", "bf16", "fp8"
    act_dtype: str          # "f32", "bf16"
    rms_eps: float = 1e-6
    ticks: int = 0          # streaming ticks (0: not a streaming workload)
    t_schedule: Optional[Tuple[float, ...]] = None  # n_steps + 1 times, 1 -> 0 (None: uniform)
    sampler: str = "euler"  # "euler", "heun" or "ab2"
    state_causal: bool = False  # Pi0-style suffix: the state token sees only the prefix and itself
    kv_fp8: bool = False        # prefix K/V cached as fp8 E4M3 with a scale per (token, kv head)
    rope_theta: float = 0.0     # rotary position embedding base (0: none)
    w8a8: bool = False          # fp8 weights: also quantise GEMM activations (32-element blocks, power-of-two scales)
    attn_kernel: str = "auto"   # GPU attention kernel: "auto", "register" or "streamed" (no effect on the math)

    @property
    def has_state(self) -> int:
        return 1 if self.state_dim > 0 else 0

    @property
    def suffix(self) -> int:
        return self.chunk + self.has_state

    @property
    def prefix_cap(self) -> int:
        return self.prefix_static + self.frame_tokens * self.n_frames

    def replace(self, **kw) -> "FMConfig":
        return dataclasses.replace(self, **kw)


_PI0 = dict(d_model=1024, n_layers=18, n_q_heads=8, n_kv_heads=1, head_dim=256,
            d_mlp=4096, action_dim=32, n_steps=10)

WORKLOADS: Dict[str, FMConfig] = {
    # Tiny fp32 loop that the oracle finishes in well under a second.
    "tiny_fp32": FMConfig(
        name="tiny_fp32", seed=0, d_model=64, n_layers=2, n_q_heads=4, n_kv_heads=4,
        head_dim=16, d_mlp=256, action_dim=32, chunk=8, state_dim=32, batch=1,
        n_steps=10, prefix_static=32, frame_tokens=0, n_frames=0, prefix_len=32,
        norm="rms", time_dim=64, weight_dtype="f32", act_dtype="f32"),
    # Pi0-like expert, one view (256 image tokens) + 20 prompt tokens.
    "pi0_1view": FMConfig(
        name="pi0_1view", seed=1, chunk=50, state_dim=32, batch=1,
        prefix_static=276, frame_tokens=0, n_frames=0, prefix_len=276,
        norm="rms", time_dim=1024, weight_dtype="bf16", act_dtype="bf16", **_PI0),
    # Same expert, three views, empty prompt, chunk 63.
    "pi0_3view": FMConfig(
        name="pi0_3view", seed=2, chunk=63, state_dim=32, batch=1,
        prefix_static=768, frame_tokens=0, n_frames=0, prefix_len=768,
        norm="rms", time_dim=1024, weight_dtype="bf16", act_dtype="bf16", **_PI0),
    # Pi05-style AdaRMSNorm expert, 16 independent robots, 2 views + prompt.
    "pi05_ada_b16": FMConfig(
        name="pi05_ada_b16", seed=3, chunk=50, state_dim=0, batch=16,
        prefix_static=532, frame_tokens=0, n_frames=0, prefix_len=532,
        norm="ada", time_dim=256, weight_dtype="bf16", act_dtype="bf16", **_PI0),
    # Streaming: fp8 e4m3 weights, 20-token static prompt + 3 x 256 frame ring.
    "stream_fp8": FMConfig(
        name="stream_fp8", seed=4, chunk=50, state_dim=32, batch=1,
        prefix_static=20, frame_tokens=256, n_frames=3, prefix_len=788,
        norm="rms", time_dim=1024, weight_dtype="fp8", act_dtype="bf16", ticks=1000,
        **_PI0),
}


def workload(name: str) -> FMConfig:
    return WORKLOADS[name]


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def round_bf16(a) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) through float32; returns float32."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def round_to(a, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype in ("bf16", "fp8"):  # fp8 workloads are drawn in bf16; each side quantises
        return round_bf16(a)
    raise ValueError(dtype)


def _normal(g: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    return round_to(g.standard_normal(shape) * std, dtype)


def _gain(g: np.random.Generator, n: int, dtype: str) -> np.ndarray:
    return round_to(1.0 + 0.1 * g.standard_normal(n), dtype)


def make_weights(cfg: FMConfig, stream: int = STREAM_WEIGHTS) -> dict:
    """All expert weights, nn.Linear convention W[out][in], ~N(0, 1/fan_in).

    Biases draw from the same distribution as their matrix; RMSNorm gains are
    1 + 0.1 N(0,1) so the gain path is exercised.  The transformer linears
    carry no bias.
    """
    g = rng(cfg.seed, stream)
    d, A, F = cfg.d_model, cfg.action_dim, cfg.d_mlp
    qd, kd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    wd = cfg.weight_dtype
    gd = "f32" if wd == "f32" else "bf16"   # embeddings / heads / gains never fp8
    lin = lambda o, i, dt=wd: _normal(g, (o, i), 1.0 / np.sqrt(i), dt)
    bias = lambda o, i: _normal(g, (o,), 1.0 / np.sqrt(i), gd)
    W: dict = {}
    W["w_in"] = lin(d, A, gd)
    W["b_in"] = bias(d, A)
    if cfg.state_dim:
        W["w_state"] = lin(d, cfg.state_dim, gd)
        W["b_state"] = bias(d, cfg.state_dim)
    if cfg.norm == "ada":
        W["w_time"] = lin(d, cfg.time_dim, gd)
        W["b_time"] = bias(d, cfg.time_dim)
    layers: List[dict] = []
    for _ in range(cfg.n_layers):
        L = {}
        L["wq"] = lin(qd, d)
        L["wk"] = lin(kd, d)
        L["wv"] = lin(kd, d)
        L["wo"] = lin(d, qd)
        L["wg"] = lin(F, d)
        L["wu"] = lin(F, d)
        L["wd"] = lin(d, F)
        for n in ("norm1", "norm2"):
            if cfg.norm == "rms":
                L[n] = _gain(g, d, gd)
            else:
                L[n + "_w"] = lin(3 * d, d, gd)
                L[n + "_b"] = bias(3 * d, d)
        layers.append(L)
    W["layers"] = layers
    if cfg.norm == "rms":
        W["norm_f"] = _gain(g, d, gd)
    else:
        W["norm_f_w"] = lin(3 * d, d, gd)
        W["norm_f_b"] = bias(3 * d, d)
    W["w_out"] = lin(A, d, gd)
    W["b_out"] = bias(A, d)
    return W


def make_prefix(cfg: FMConfig, n_tokens: Optional[int] = None):
    """Prefix K and V, [batch][layers][tokens][kv_heads][head_dim], ~N(0,1)."""
    n = cfg.prefix_len if n_tokens is None else n_tokens
    g = rng(cfg.seed, STREAM_PREFIX)
    shp = (cfg.batch, cfg.n_layers, n, cfg.n_kv_heads, cfg.head_dim)
    k = _normal(g, shp, 1.0, cfg.act_dtype)
    v = _normal(g, shp, 1.0, cfg.act_dtype)
    return k, v


def make_noise(cfg: FMConfig, stream: int = STREAM_NOISE) -> np.ndarray:
    """x at t=1, [batch][chunk][action_dim], ~N(0,1) in the activation dtype."""
    g = rng(cfg.seed, stream)
    return _normal(g, (cfg.batch, cfg.chunk, cfg.action_dim), 1.0, cfg.act_dtype)


def make_state(cfg: FMConfig) -> Optional[np.ndarray]:
    if not cfg.state_dim:
        return None
    g = rng(cfg.seed, STREAM_STATE)
    return _normal(g, (cfg.batch, cfg.state_dim), 1.0, cfg.act_dtype)


def make_frame(cfg: FMConfig, tick: int):
    """One new frame's K/V for tick `tick` (negative ticks fill the window
    before the first tick): [batch][layers][frame_tokens][kv_heads][head_dim]."""
    if tick < -cfg.n_frames:
        raise ValueError("tick before the window was filled")
    g = rng(cfg.seed, STREAM_TICK0 + 2 * (tick + cfg.n_frames))
    shp = (cfg.batch, cfg.n_layers, cfg.frame_tokens, cfg.n_kv_heads, cfg.head_dim)
    return _normal(g, shp, 1.0, cfg.act_dtype), _normal(g, shp, 1.0, cfg.act_dtype)


def make_tick_noise(cfg: FMConfig, tick: int) -> np.ndarray:
    """Fresh noise drawn for streaming tick `tick` (tick >= 0)."""
    return make_noise(cfg, stream=STREAM_TICK0 + 2 * (tick + cfg.n_frames) + 1)


def make_prefix_stack(cfg: FMConfig, n_tokens: int):
    """Weights and input tokens of a tiny prefix encoder with the expert's
    width and layer count (used to produce timestep-invariant prefix K/V
    from actual tokens).  Returns (weights dict like make_weights' layers,
    tokens [batch][n_tokens][d_model])."""
    g = rng(cfg.seed, STREAM_PREFIX_STACK)
    d, F = cfg.d_model, cfg.d_mlp
    qd, kd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    dt = cfg.act_dtype
    lin = lambda o, i: _normal(g, (o, i), 1.0 / np.sqrt(i), dt)
    layers = []
    for _ in range(cfg.n_layers):
        layers.append(dict(wq=lin(qd, d), wk=lin(kd, d), wv=lin(kd, d), wo=lin(d, qd),
                           wg=lin(F, d), wu=lin(F, d), wd=lin(d, F),
                           norm1=_gain(g, d, dt), norm2=_gain(g, d, dt)))
    tokens = _normal(g, (cfg.batch, n_tokens, d), 1.0, dt)
    return {"layers": layers}, tokens
