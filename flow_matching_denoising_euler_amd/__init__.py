"""MI355X (gfx950) flow-matching action-expert denoiser.

A thin Python binding over libfmdenoise.so (include/fm.h).  Every function
here only marshals arguments: torch supplies device memory and the HIP
stream, and every step of the denoise loop runs in the library's HIP
kernels.  Names match the C entry points; `Denoiser` bundles them.
"""
import ctypes
from typing import Optional

from . import _abi
from ._abi import (FM_ABI_VERSION, FM_BF16, FM_EXEC_AUTO, FM_EXEC_GRAPH, FM_EXEC_PERSISTENT,  # noqa: F401
                   FM_F32, FM_FP8_E4M3, FM_OK, STATUS_NAMES, fm_config, fm_info, fm_weights)

__all__ = ["FMError", "make_config", "fm_create", "fm_set_prefix_kv", "fm_append_prefix_kv",
           "fm_denoise", "fm_denoise_noalloc", "fm_get_info", "fm_launch_phase", "fm_destroy", "fm_last_error", "fm_quantize_e4m3",
           "fm_encoder_create", "fm_encode_prefix", "fm_append_encoded", "Denoiser", "Encoder", "lib"]

lib = _abi.lib


class FMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _stream_obj(stream, device):
    """The torch stream object of `stream` (None: the current stream of
    `device`; an int: an external hipStream_t handle)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def stream_enter(ctx_stream, cur_stream):
    """Before a library call on a context bound to `ctx_stream`: if the
    caller's current stream differs, the context's stream waits for the
    work already queued on it (the host-to-device copies and casts of the
    call's inputs)."""
    if cur_stream != ctx_stream:
        ctx_stream.wait_stream(cur_stream)


def stream_leave(ctx_stream, cur_stream, temps):
    """After the call: tensors made on `cur_stream` and read by the library
    on `ctx_stream` are recorded on it (the caching allocator then keeps
    their memory until that stream's work is done), and the caller's stream
    waits for the library's results."""
    if cur_stream != ctx_stream:
        for t in temps:
            if t is not None:
                t.record_stream(ctx_stream)
        cur_stream.wait_stream(ctx_stream)


_DT = {"f32": _abi.FM_F32, "bf16": _abi.FM_BF16, "fp8": _abi.FM_FP8_E4M3}


def make_config(cfg, exec_mode: int = FM_EXEC_AUTO) -> fm_config:
    """fm_config from any object with the workload fields (e.g. fm_synth.FMConfig)."""
    c = fm_config()
    c.abi_version = FM_ABI_VERSION
    for f in ("d_model", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "d_mlp", "action_dim", "chunk",
              "state_dim", "batch", "n_steps", "prefix_static", "frame_tokens", "n_frames", "time_dim"):
        setattr(c, f, int(getattr(cfg, f)))
    c.norm = _abi.FM_ADARMSNORM if cfg.norm == "ada" else _abi.FM_RMSNORM
    c.weight_dtype = _DT[cfg.weight_dtype]
    c.act_dtype = _DT[cfg.act_dtype]
    c.rms_eps = float(cfg.rms_eps)
    c.exec_mode = int(exec_mode)
    c.sampler = {"euler": _abi.FM_SAMPLER_EULER, "heun": _abi.FM_SAMPLER_HEUN,
                 "ab2": _abi.FM_SAMPLER_AB2}[getattr(cfg, "sampler", "euler")]
    c.state_causal = 1 if getattr(cfg, "state_causal", False) else 0
    c.kv_fp8 = 1 if getattr(cfg, "kv_fp8", False) else 0
    c.rope_theta = float(getattr(cfg, "rope_theta", 0.0))
    c.w8a8 = 1 if getattr(cfg, "w8a8", False) else 0
    c.attn_kernel = {"auto": _abi.FM_ATTN_AUTO, "register": _abi.FM_ATTN_REGISTER,
                     "streamed": _abi.FM_ATTN_STREAMED}[getattr(cfg, "attn_kernel", "auto")]
    sched = getattr(cfg, "t_schedule", None)
    if sched is not None:
        arr = (ctypes.c_float * len(sched))(*[float(t) for t in sched])
        c.t_schedule = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
        c._t_schedule_keep = arr  # alive as long as the config
    return c


def _check(status: int, ctx=None):
    if status != FM_OK:
        raise FMError(status, fm_last_error(ctx))


def fm_last_error(ctx=None) -> str:
    return lib().fm_last_error(ctx).decode(errors="replace")


def _dev_tensor(a, dtype, device):
    import numpy as np
    import torch
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


def fm_create(cfg, weights: dict, stream=None, exec_mode: int = FM_EXEC_AUTO, device="cuda"):
    """Create a context.  `weights` follows fm_synth.make_weights' layout:
    host or device arrays in W[out][in] convention; they are converted to
    the model's weight dtype on `device` (bf16 for bf16 and fp8 models)."""
    import torch
    c = make_config(cfg, exec_mode)
    wdt = torch.float32 if cfg.weight_dtype == "f32" else torch.bfloat16
    keep = []

    def put(a):
        t = _dev_tensor(a, wdt, device)
        keep.append(t)
        return _ptr(t)

    w = fm_weights()
    w.w_in, w.b_in = put(weights["w_in"]), put(weights["b_in"])
    if cfg.state_dim:
        w.w_state, w.b_state = put(weights["w_state"]), put(weights["b_state"])
    w.w_out, w.b_out = put(weights["w_out"]), put(weights["b_out"])
    if cfg.norm == "ada":
        w.w_time, w.b_time = put(weights["w_time"]), put(weights["b_time"])
        w.norm_f, w.norm_f_b = put(weights["norm_f_w"]), put(weights["norm_f_b"])
    else:
        w.norm_f = put(weights["norm_f"])
    w.layers = _layer_table(weights["layers"], cfg.norm == "rms", put)
    ctx = ctypes.c_void_p()
    st = lib().fm_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(_stream(stream)), ctypes.byref(ctx))
    _check(st)
    del keep
    return ctx


def _layer_table(layers, rms: bool, put):
    names = ["wq", "wk", "wv", "wo", "wg", "wu", "wd"]
    norms = ["norm1", None, "norm2", None] if rms else ["norm1_w", "norm1_b", "norm2_w", "norm2_b"]
    arr = (ctypes.c_void_p * (len(layers) * _abi.FM_LW_COUNT))()
    for li, L in enumerate(layers):
        for si, n in enumerate(names + norms):
            arr[li * _abi.FM_LW_COUNT + si] = put(L[n]) if n else None
    ptr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    ptr._keep = arr
    return ptr


def fm_encoder_create(cfg, weights: dict, n_tokens: int, n_seqs: int = 1, stream=None,
                      exec_mode: int = FM_EXEC_AUTO, device="cuda"):
    """Create a prefix-encoder context for `n_seqs` sequences of `n_tokens`
    tokens each.  `cfg` supplies the layer shape and dtypes (its other fields
    are ignored); `weights` is fm_synth.make_prefix_stack's {"layers": [...]}."""
    import torch
    c = make_config(cfg, exec_mode)
    c.chunk, c.batch = int(n_tokens), int(n_seqs)
    wdt = torch.float32 if cfg.weight_dtype == "f32" else torch.bfloat16
    keep = []

    def put(a):
        t = _dev_tensor(a, wdt, device)
        keep.append(t)
        return _ptr(t)

    w = fm_weights()
    w.layers = _layer_table(weights["layers"], True, put)
    ctx = ctypes.c_void_p()
    st = lib().fm_encoder_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(_stream(stream)),
                                 ctypes.byref(ctx))
    _check(st)
    del keep
    return ctx


def fm_encode_prefix(ctx, tokens, k_out=None, v_out=None):
    """tokens: fp32 device [seqs][tokens][d_model]; k_out, v_out: device
    [seqs][layers][tokens][kv_heads][head_dim] in the activation dtype, or
    both None (the output stays in the encoder for fm_append_encoded)."""
    _check(lib().fm_encode_prefix(ctx, _ptr(tokens), _ptr(k_out), _ptr(v_out)), ctx)


def fm_append_encoded(ctx, robot: int, enc_ctx, seq: int = 0):
    """Append sequence `seq` of the encoder's latest output to `robot`'s ring,
    on ctx's stream behind the encode."""
    _check(lib().fm_append_encoded(ctx, int(robot), enc_ctx, int(seq)), ctx)


def fm_set_prefix_kv(ctx, robot: int, k, v, n_tokens: int):
    """k, v: device tensors [layers][n_tokens][kv_heads][head_dim] in the activation dtype."""
    _check(lib().fm_set_prefix_kv(ctx, int(robot), _ptr(k), _ptr(v), int(n_tokens)), ctx)


def fm_append_prefix_kv(ctx, robot: int, k_frame, v_frame):
    _check(lib().fm_append_prefix_kv(ctx, int(robot), _ptr(k_frame), _ptr(v_frame)), ctx)


def fm_denoise(ctx, noise, state, actions):
    """noise, actions: fp32 device tensors [batch][chunk][action_dim]; state or None."""
    _check(lib().fm_denoise(ctx, _ptr(noise), _ptr(state), _ptr(actions)), ctx)


def fm_denoise_noalloc(ctx, noise, state, actions):
    """fm_denoise with the loop's scratch in the library's static per-GPU
    array (allocates nothing; concurrent calls on one GPU race)."""
    _check(lib().fm_denoise_noalloc(ctx, _ptr(noise), _ptr(state), _ptr(actions)), ctx)


def fm_get_info(ctx) -> fm_info:
    info = fm_info()
    _check(lib().fm_get_info(ctx, ctypes.byref(info)), ctx)
    return info


def fm_launch_phase(ctx, step: int, layer: int, phase: int):
    _check(lib().fm_launch_phase(ctx, int(step), int(layer), int(phase)), ctx)


def fm_destroy(ctx):
    lib().fm_destroy(ctx)


def fm_quantize_e4m3(w, codes, scales, stream=None):
    """w: bf16 device [rows][cols]; codes: uint8 device; scales: fp32 device [rows]."""
    rows, cols = w.shape
    _check(lib().fm_quantize_e4m3(_ptr(w), rows, cols, _ptr(codes), _ptr(scales),
                                  ctypes.c_void_p(_stream(stream))))


class _Context:
    """Owns one library context (released by close() or on collection)."""
    ctx = None

    def _setup(self, cfg, device, stream):
        import torch
        self.cfg = cfg
        self.device = device
        self.act_dtype = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
        self.stream = _stream_obj(stream, device)  # the stream the context enqueues on

    def _call(self, fn, temps):
        """Run one library call with the inputs `temps` (made on the caller's
        current stream) safely on the context's stream."""
        import torch
        cur = torch.cuda.current_stream(self.device)
        stream_enter(self.stream, cur)
        fn()
        stream_leave(self.stream, cur, temps)

    def _act(self, a):
        return _dev_tensor(a, self.act_dtype, self.device)

    def info(self) -> fm_info:
        return fm_get_info(self.ctx)

    def close(self):
        if self.ctx is not None:
            fm_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Denoiser(_Context):
    """Owns one context: load the prefix, then call `denoise` per chunk."""

    def __init__(self, cfg, weights: dict, stream=None, exec_mode: int = FM_EXEC_AUTO, device="cuda"):
        self._setup(cfg, device, stream)
        self.ctx = fm_create(cfg, weights, self.stream, exec_mode, device)

    def set_prefix_kv(self, robot: int, k, v):
        """k, v [layers][tokens][kv_heads][head_dim] (host or device)."""
        k, v = self._act(k), self._act(v)
        self._call(lambda: fm_set_prefix_kv(self.ctx, robot, k, v, k.shape[1]), (k, v))
        return k, v

    def append_prefix_kv(self, robot: int, k_frame, v_frame):
        k, v = self._act(k_frame), self._act(v_frame)
        self._call(lambda: fm_append_prefix_kv(self.ctx, robot, k, v), (k, v))
        return k, v

    def append_encoded(self, robot: int, encoder, seq: int = 0):
        """Append sequence `seq` of `encoder`'s latest output (see fm_append_encoded)."""
        self._call(lambda: fm_append_encoded(self.ctx, robot, encoder.ctx, seq), ())

    def denoise(self, noise, state=None, out=None):
        import torch
        n = _dev_tensor(noise, torch.float32, self.device)
        s = self._act(state) if state is not None else None
        if out is None:
            out = torch.empty_like(n)
        self._call(lambda: fm_denoise(self.ctx, n, s, out), (n, s, out))
        return out


class Encoder(_Context):
    """Owns one prefix-encoder context: `encode` turns token embeddings into
    the per-layer K/V that Denoiser.set_prefix_kv / append_prefix_kv take."""

    def __init__(self, cfg, weights: dict, n_tokens: int, n_seqs: int = 1, stream=None,
                 exec_mode: int = FM_EXEC_AUTO, device="cuda"):
        self._setup(cfg, device, stream)
        self.n_tokens, self.n_seqs = int(n_tokens), int(n_seqs)
        self.ctx = fm_encoder_create(cfg, weights, n_tokens, n_seqs, self.stream, exec_mode, device)

    def encode(self, tokens, k_out=None, v_out=None):
        """tokens [seqs][tokens][d_model] (host or device) -> (k, v) device
        tensors [seqs][layers][tokens][kv_heads][head_dim]."""
        import torch
        t = _dev_tensor(tokens, torch.float32, self.device)
        shape = (self.n_seqs, self.cfg.n_layers, self.n_tokens, self.cfg.n_kv_heads, self.cfg.head_dim)
        if k_out is None:
            k_out = torch.empty(shape, dtype=self.act_dtype, device=self.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=self.act_dtype, device=self.device)
        self._call(lambda: fm_encode_prefix(self.ctx, t, k_out, v_out), (t, k_out, v_out))
        return k_out, v_out

    def encode_in_place(self, tokens):
        """Encode without copying the K/V out: the output stays in the encoder
        for Denoiser.append_encoded (the async-pipeline hand-off)."""
        import torch
        t = _dev_tensor(tokens, torch.float32, self.device)
        self._call(lambda: fm_encode_prefix(self.ctx, t), (t,))
