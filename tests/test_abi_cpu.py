"""The C ABI library loads, exports every symbol include/fm.h declares, and
rejects bad arguments before touching a device (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import fm_synth as S
import flow_matching_denoising_euler_amd as fm
from flow_matching_denoising_euler_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "fm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fm_create", "fm_set_prefix_kv", "fm_append_prefix_kv", "fm_denoise", "fm_destroy"):
        assert n in names
    assert set(names) == set(_abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    for n in _declared():
        assert hasattr(L, n), n


def test_struct_layouts_match_header():
    # 26 scalars, the t_schedule pointer, attn_kernel (and 4 bytes of padding to the pointer's alignment)
    assert ctypes.sizeof(_abi.fm_config) == 26 * 4 + 8 + 8
    assert _abi.fm_config.attn_kernel.offset == 26 * 4 + 8
    assert ctypes.sizeof(_abi.fm_weights) == 11 * 8
    assert ctypes.sizeof(_abi.fm_info) == 3 * 8 + 4 * 4


def _cfg(**kw):
    return fm.make_config(S.workload("tiny_fp32").replace(**kw))


def _set_schedule(c, times):
    arr = (ctypes.c_float * len(times))(*times)
    c.t_schedule = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    c._keep = arr


def _create(c):
    w = _abi.fm_weights()
    ctx = ctypes.c_void_p()
    return fm.lib().fm_create(ctypes.byref(c) if c is not None else None, ctypes.byref(w), None, ctypes.byref(ctx)), ctx


@pytest.mark.parametrize("mutate,status", [
    (lambda c: setattr(c, "abi_version", 99), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "d_model", 0), _abi.FM_ERR_SHAPE),
    (lambda c: setattr(c, "batch", -1), _abi.FM_ERR_SHAPE),
    (lambda c: setattr(c, "n_kv_heads", 3), _abi.FM_ERR_SHAPE),
    (lambda c: setattr(c, "norm", 7), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "act_dtype", _abi.FM_FP8_E4M3), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "act_dtype", _abi.FM_BF16), _abi.FM_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "d_model", 96), _abi.FM_ERR_SHAPE),   # time_dim no longer equals d_model
    (lambda c: (setattr(c, "d_model", 96), setattr(c, "time_dim", 96)), _abi.FM_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "action_dim", 7), _abi.FM_ERR_UNSUPPORTED),
    (lambda c: setattr(c, "n_frames", 2), _abi.FM_ERR_SHAPE),   # frames without frame_tokens
    (lambda c: (setattr(c, "n_frames", 2), setattr(c, "frame_tokens", 16)), _abi.FM_ERR_UNSUPPORTED),  # frames % 32
    (lambda c: setattr(c, "rms_eps", float("nan")), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "exec_mode", 9), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "sampler", 3), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "state_causal", 2), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "kv_fp8", 2), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "w8a8", 2), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "w8a8", 1), _abi.FM_ERR_UNSUPPORTED),     # fp32 weights
    (lambda c: (setattr(c, "w8a8", 1), setattr(c, "act_dtype", _abi.FM_BF16), setattr(c, "weight_dtype", _abi.FM_FP8_E4M3)),
     _abi.FM_ERR_UNSUPPORTED),                                        # d_model 64 is not a multiple of 128
    (lambda c: setattr(c, "attn_kernel", 3), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "attn_kernel", _abi.FM_ATTN_STREAMED), _abi.FM_ERR_UNSUPPORTED),  # fp32 activations
    (lambda c: (setattr(c, "attn_kernel", _abi.FM_ATTN_STREAMED), setattr(c, "act_dtype", _abi.FM_BF16),
                setattr(c, "weight_dtype", _abi.FM_BF16), setattr(c, "head_dim", 32), setattr(c, "n_q_heads", 2),
                setattr(c, "n_kv_heads", 1), setattr(c, "kv_fp8", 1)), _abi.FM_ERR_UNSUPPORTED),  # fp8 prefix cache
    (lambda c: setattr(c, "rope_theta", -1.0), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "rope_theta", float("nan")), _abi.FM_ERR_ARG),
    (lambda c: (setattr(c, "rope_theta", 1e4), setattr(c, "n_frames", 2), setattr(c, "frame_tokens", 32)),
     _abi.FM_ERR_UNSUPPORTED),                                        # rotary positions with a ring
    (lambda c: setattr(c, "kv_fp8", 1), _abi.FM_ERR_UNSUPPORTED),   # fp32 activations
    (lambda c: (setattr(c, "kv_fp8", 1), setattr(c, "act_dtype", _abi.FM_BF16), setattr(c, "weight_dtype", _abi.FM_BF16),
                setattr(c, "prefix_static", 1100)), _abi.FM_ERR_UNSUPPORTED),  # > 1024 padded keys
    (lambda c: _set_schedule(c, [1.0, 0.5, 0.25, 0.5] + [0.1] * 6 + [0.0]), _abi.FM_ERR_ARG),  # not decreasing
    (lambda c: _set_schedule(c, [0.9] + [0.8 - 0.08 * k for k in range(9)] + [0.0]), _abi.FM_ERR_ARG),  # t_0 != 1
    (lambda c: _set_schedule(c, [1.0 - 0.095 * k for k in range(11)]), _abi.FM_ERR_ARG),  # t_N != 0
])
def test_create_rejects_bad_config_before_device_work(mutate, status):
    c = _cfg()
    mutate(c)
    st, ctx = _create(c)
    assert st == status, (st, fm.fm_last_error())
    assert ctx.value is None
    assert len(fm.fm_last_error()) > 0


def test_create_rejects_missing_weights():
    st, ctx = _create(_cfg())  # all weight pointers NULL
    assert st == _abi.FM_ERR_ARG and "missing" in fm.fm_last_error()
    L = fm.lib()
    assert L.fm_create(None, None, None, None) == _abi.FM_ERR_ARG


def test_null_context_calls_fail_cleanly():
    L = fm.lib()
    assert L.fm_set_prefix_kv(None, 0, None, None, 0) == _abi.FM_ERR_ARG
    assert L.fm_append_prefix_kv(None, 0, None, None) == _abi.FM_ERR_ARG
    assert L.fm_denoise(None, None, None, None) == _abi.FM_ERR_ARG
    assert L.fm_get_info(None, None) == _abi.FM_ERR_ARG
    L.fm_destroy(None)
    assert L.fm_quantize_e4m3(None, 4, 4, None, None, None) == _abi.FM_ERR_ARG
    assert isinstance(fm.fm_last_error(), str)


def _encoder_create(c, layers=True):
    w = _abi.fm_weights()
    keep = None
    if layers:  # non-NULL dummy host pointers: validation only looks at presence
        keep = (ctypes.c_float * 4)()
        arr = (ctypes.c_void_p * (c.n_layers * _abi.FM_LW_COUNT))()
        for i in range(len(arr)):
            arr[i] = ctypes.addressof(keep)
        w.layers = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    ctx = ctypes.c_void_p()
    st = fm.lib().fm_encoder_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(ctx))
    return st, ctx


@pytest.mark.parametrize("mutate,status", [
    (lambda c: setattr(c, "abi_version", 99), _abi.FM_ERR_ARG),
    (lambda c: setattr(c, "chunk", 0), _abi.FM_ERR_SHAPE),            # tokens per sequence
    (lambda c: setattr(c, "n_kv_heads", 3), _abi.FM_ERR_SHAPE),
    (lambda c: setattr(c, "chunk", 300), _abi.FM_ERR_UNSUPPORTED),    # fp32 path: <= 256 tokens
    (lambda c: (setattr(c, "act_dtype", _abi.FM_BF16), setattr(c, "weight_dtype", _abi.FM_BF16),
                setattr(c, "head_dim", 64), setattr(c, "chunk", 1025)), _abi.FM_ERR_UNSUPPORTED),  # bf16: <= 1024
    (lambda c: setattr(c, "exec_mode", _abi.FM_EXEC_PERSISTENT), _abi.FM_ERR_UNSUPPORTED),
])
def test_encoder_create_rejects_bad_config_before_device_work(mutate, status):
    c = _cfg()
    mutate(c)
    st, ctx = _encoder_create(c)
    assert st == status, (st, fm.fm_last_error())
    assert ctx.value is None


def test_encoder_create_ignores_the_expert_only_fields():
    # fields the encoder does not read may hold values fm_create would refuse;
    # validation then passes and stops at the (absent) layers or the device
    c = _cfg(action_dim=7, n_frames=2, norm="ada", time_dim=3)
    c.sampler = 9
    st, ctx = _encoder_create(c, layers=False)
    assert st == _abi.FM_ERR_ARG and "layers" in fm.fm_last_error(), fm.fm_last_error()
    assert ctx.value is None


def test_encoder_null_calls_fail_cleanly():
    L = fm.lib()
    assert L.fm_encoder_create(None, None, None, None) == _abi.FM_ERR_ARG
    assert L.fm_encode_prefix(None, None, None, None) == _abi.FM_ERR_ARG
    assert L.fm_append_encoded(None, 0, None, 0) == _abi.FM_ERR_ARG


class _FakeStream:
    """Stand-in for a torch stream: records the waits it is asked for."""

    def __init__(self, name):
        self.name, self.waited_on = name, []

    def wait_stream(self, other):
        self.waited_on.append(other.name)


class _FakeTensor:
    def __init__(self):
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s.name)


def test_binding_stream_guard_orders_a_foreign_current_stream():
    # the context enqueues on its own stream; inputs made on another current
    # stream must be complete before the call (ctx waits on it), must stay
    # allocated until the context's stream is done (record_stream), and the
    # caller's stream must see the outputs (it waits on the context's stream)
    ctx, cur = _FakeStream("ctx"), _FakeStream("cur")
    temps = [_FakeTensor(), None, _FakeTensor()]
    fm.stream_enter(ctx, cur)
    assert ctx.waited_on == ["cur"]
    fm.stream_leave(ctx, cur, temps)
    assert temps[0].recorded == ["ctx"] and temps[2].recorded == ["ctx"]
    assert cur.waited_on == ["ctx"]


def test_binding_stream_guard_is_a_no_op_on_the_context_stream():
    # same stream: the stream order alone serialises the copies, the call and
    # the allocator's reuse of the temporaries
    ctx = _FakeStream("ctx")
    t = _FakeTensor()
    fm.stream_enter(ctx, ctx)
    fm.stream_leave(ctx, ctx, [t])
    assert ctx.waited_on == [] and t.recorded == []


def _w8a8_cfg(**kw):
    # fp8 weights with 128-multiple sizes: only the named field breaks the W8A8 rules
    base = dict(d_model=128, time_dim=128, d_mlp=256, n_q_heads=2, n_kv_heads=1, head_dim=64,
                weight_dtype="fp8", act_dtype="bf16", batch=32, chunk=8, w8a8=True)
    base.update(kw)
    return fm.make_config(S.workload("tiny_fp32").replace(**base))


@pytest.mark.parametrize("kw,what", [
    (dict(batch=28), "rows"),                       # 28 x 9 = 252 rows < 256
    (dict(exec_mode=2), "persistent"),
    (dict(weight_dtype="bf16"), "fp8 weights"),
    (dict(d_mlp=192), "multiples of 128"),
    (dict(n_q_heads=2, head_dim=32), "multiples of 128"),  # Hq Dh = 64
])
def test_w8a8_limits_are_rejected_before_device_work(kw, what):
    exec_mode = kw.pop("exec_mode", None)
    c = _w8a8_cfg(**kw)
    if exec_mode is not None:
        c.exec_mode = exec_mode
    st, ctx = _create(c)
    assert st == _abi.FM_ERR_UNSUPPORTED, (st, fm.fm_last_error())
    assert ctx.value is None and what in fm.fm_last_error()


def test_w8a8_config_passes_validation_and_encoder_rejects_it():
    st, ctx = _create(_w8a8_cfg())   # valid: fails later, on the missing weights
    assert st == _abi.FM_ERR_ARG and "missing" in fm.fm_last_error()
    st, ctx = _encoder_create(_w8a8_cfg())
    assert st == _abi.FM_ERR_UNSUPPORTED and "w8a8" in fm.fm_last_error() and ctx.value is None
