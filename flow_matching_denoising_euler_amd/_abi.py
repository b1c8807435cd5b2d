"""ctypes mirror of include/fm.h and the loader of libfmdenoise.so.

The library is the product path: if it is not built, importing the binding
raises instead of falling back to anything else.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfmdenoise.so")

FM_ABI_VERSION = 7

FM_OK, FM_ERR_ARG, FM_ERR_SHAPE, FM_ERR_STATE, FM_ERR_OOM, FM_ERR_DEVICE, FM_ERR_UNSUPPORTED = range(7)
STATUS_NAMES = {0: "FM_OK", 1: "FM_ERR_ARG", 2: "FM_ERR_SHAPE", 3: "FM_ERR_STATE", 4: "FM_ERR_OOM",
                5: "FM_ERR_DEVICE", 6: "FM_ERR_UNSUPPORTED"}
FM_F32, FM_BF16, FM_FP8_E4M3 = 0, 1, 2
FM_RMSNORM, FM_ADARMSNORM = 0, 1
FM_EXEC_AUTO, FM_EXEC_GRAPH, FM_EXEC_PERSISTENT = 0, 1, 2
FM_SAMPLER_EULER, FM_SAMPLER_HEUN, FM_SAMPLER_AB2 = 0, 1, 2
FM_ATTN_AUTO, FM_ATTN_REGISTER, FM_ATTN_STREAMED = 0, 1, 2
(FM_LW_WQ, FM_LW_WK, FM_LW_WV, FM_LW_WO, FM_LW_WG, FM_LW_WU, FM_LW_WD,
 FM_LW_NORM1, FM_LW_NORM1_B, FM_LW_NORM2, FM_LW_NORM2_B, FM_LW_COUNT) = range(12)

EXPORTS = ("fm_create", "fm_set_prefix_kv", "fm_append_prefix_kv", "fm_denoise", "fm_get_info",
           "fm_destroy", "fm_last_error", "fm_quantize_e4m3", "fm_launch_phase", "fm_encoder_create",
           "fm_encode_prefix", "fm_append_encoded", "fm_denoise_noalloc")
FM_PHASE_QKV, FM_PHASE_ATTN, FM_PHASE_OPROJ, FM_PHASE_GATEUP, FM_PHASE_DOWN, FM_PHASE_TAIL, FM_PHASE_LOOP = range(7)


class fm_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "d_model", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "d_mlp",
        "action_dim", "chunk", "state_dim", "batch", "n_steps", "prefix_static", "frame_tokens",
        "n_frames", "norm", "time_dim", "weight_dtype", "act_dtype")] + [
        ("rms_eps", ctypes.c_float), ("exec_mode", ctypes.c_int32), ("sampler", ctypes.c_int32), ("state_causal", ctypes.c_int32), ("kv_fp8", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("w8a8", ctypes.c_int32),
        ("t_schedule", ctypes.POINTER(ctypes.c_float)), ("attn_kernel", ctypes.c_int32)]


class fm_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_in", "b_in", "w_state", "b_state", "w_out", "b_out", "w_time", "b_time",
        "norm_f", "norm_f_b")] + [("layers", ctypes.POINTER(ctypes.c_void_p))]


class fm_info(ctypes.Structure):
    _fields_ = [("arena_bytes", ctypes.c_size_t), ("weight_bytes_per_step", ctypes.c_size_t),
                ("kv_bytes_per_step", ctypes.c_size_t), ("exec_mode", ctypes.c_int32),
                ("n_phases", ctypes.c_int32), ("grid", ctypes.c_int32), ("n_cu", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libfmdenoise.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m flow_matching_denoising_euler_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.fm_create.argtypes = [ctypes.POINTER(fm_config), ctypes.POINTER(fm_weights), vp, ctypes.POINTER(vp)]
        L.fm_create.restype = ctypes.c_int
        L.fm_set_prefix_kv.argtypes = [vp, i32, vp, vp, i32]
        L.fm_set_prefix_kv.restype = ctypes.c_int
        L.fm_append_prefix_kv.argtypes = [vp, i32, vp, vp]
        L.fm_append_prefix_kv.restype = ctypes.c_int
        L.fm_denoise.argtypes = [vp, vp, vp, vp]
        L.fm_denoise.restype = ctypes.c_int
        L.fm_denoise_noalloc.argtypes = [vp, vp, vp, vp]
        L.fm_denoise_noalloc.restype = ctypes.c_int
        L.fm_get_info.argtypes = [vp, ctypes.POINTER(fm_info)]
        L.fm_get_info.restype = ctypes.c_int
        L.fm_destroy.argtypes = [vp]
        L.fm_destroy.restype = None
        L.fm_last_error.argtypes = [vp]
        L.fm_last_error.restype = ctypes.c_char_p
        L.fm_quantize_e4m3.argtypes = [vp, i32, i32, vp, vp, vp]
        L.fm_quantize_e4m3.restype = ctypes.c_int
        L.fm_launch_phase.argtypes = [vp, i32, i32, i32]
        L.fm_launch_phase.restype = ctypes.c_int
        L.fm_encoder_create.argtypes = [ctypes.POINTER(fm_config), ctypes.POINTER(fm_weights), vp, ctypes.POINTER(vp)]
        L.fm_encoder_create.restype = ctypes.c_int
        L.fm_encode_prefix.argtypes = [vp, vp, vp, vp]
        L.fm_encode_prefix.restype = ctypes.c_int
        L.fm_append_encoded.argtypes = [vp, i32, vp, i32]
        L.fm_append_encoded.restype = ctypes.c_int
        _LIB = L
    return _LIB
