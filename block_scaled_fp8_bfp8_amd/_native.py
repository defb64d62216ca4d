"""ctypes declarations of libbfp8.so's C ABI (include/bfp8.h). Loading only; no computation."""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libbfp8.so")

BFP8_OK = 0
BFP8_ERR_INVALID_ARGUMENT = 1
BFP8_ERR_UNSUPPORTED = 2
BFP8_ERR_MISALIGNED = 3
BFP8_ERR_WORKSPACE = 4
BFP8_ERR_DEVICE = 5
BFP8_ERR_LAUNCH = 6

BFP8_IN_F32 = 0
BFP8_IN_BF16 = 1
BFP8_IN_F16 = 2

SCHEDULES = {"auto": 0, "small_m": 1, "tiled": 2, "persistent": 3}

# Every symbol include/bfp8.h declares: (name, restype, argtypes)
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = [
    ("bfp8_abi_version", ctypes.c_int, []),
    ("bfp8_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("bfp8_last_error_message", ctypes.c_char_p, []),
    ("bfp8_quant_act", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    ("bfp8_gemm_workspace_bytes", _sz, [_i64, _i64, _i64]),
    ("bfp8_gemm", ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_grouped_gemm_contiguous", ctypes.c_int,
     [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_grouped_gemm_gathered", ctypes.c_int,
     [_vp, _i64, _vp, _i64, _i64, _vp, _i32, _vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _i64, _i64, _i64, _vp]),
    ("bfp8_gemm_f16", ctypes.c_int,
     [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_quant_act_1x64", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    ("bfp8_gemm_1x64", ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]),
    ("bfp8_quant_act_ue8m0", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    ("bfp8_gemm_ue8m0", ctypes.c_int,
     [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_grouped_gemm_contiguous_ue8m0", ctypes.c_int,
     [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _i64, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_moe_padded_rows", _i64, [_i64, _i32, _i32]),
    ("bfp8_moe_dispatch_workspace_bytes", _sz, [_i64, _i32]),
    ("bfp8_moe_dispatch", ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    ("bfp8_quant_act_gather", ctypes.c_int,
     [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _i64, _vp, _i64, _vp, _i64, _vp]),
    ("bfp8_quant_act_scatter", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i32, _vp]),
    ("bfp8_swiglu_quant", ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp]),
    ("bfp8_swiglu", ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
    ("bfp8_moe_combine", ctypes.c_int, [_vp, _i64, _vp, _vp, _i64, _i32, _i64, _vp, _i64, _vp]),
    ("bfp8_moe_forward_workspace_bytes", _sz, [_i64, _i32, _i32, _i64, _i64]),
    ("bfp8_moe_forward", ctypes.c_int,
     [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    ("bfp8_transpose_weights", ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp]),
    ("bfp8_transpose_scales", ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    ("bfp8_expand_act_scales", ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    ("bfp8_expand_weight_scale", ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp]),
    ("bfp8_linear_workspace_bytes", _sz, [_i64, _i64, _i64]),
    ("bfp8_linear", ctypes.c_int,
     [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    ("bfp8_linear_fuses", ctypes.c_int, [_i64, _i64, _i64, _i64]),
    ("bfp8_linear_noalloc", ctypes.c_int,
     [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _vp]),
    ("bfp8_set_schedule", ctypes.c_int, [ctypes.c_int]),
    ("bfp8_get_schedule", ctypes.c_int, []),
    ("bfp8_gemm_schedule_for", ctypes.c_int, [_i64, _i64, _i64]),
]

_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded libbfp8.so (raises LibraryMissing if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -m block_scaled_fp8_bfp8_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, restype, argtypes in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = restype
            fn.argtypes = argtypes
        _lib = handle
    return _lib


# The benchmark's measurement probes (libbfp8_probes.so, include/bfp8_probes.h).
PROBES_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbfp8_probes.so")
PROBE_SIGNATURES = [
    ("bfp8_probe_mfma_loop", ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    ("bfp8_probe_mfma_loop_flops", ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
    ("bfp8_probe_mfma32_loop", ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    ("bfp8_probe_mfma32_loop_flops", ctypes.c_double, [ctypes.c_int, ctypes.c_int]),
    ("bfp8_probe_stream_read", ctypes.c_int, [_vp, _sz, _vp, ctypes.c_int, _vp]),
    ("bfp8_probe_copy_lds", ctypes.c_int,
     [_vp, ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, ctypes.c_int, _vp]),
]
_probes = None


def probes() -> ctypes.CDLL:
    """The loaded libbfp8_probes.so (raises LibraryMissing if it has not been built)."""
    global _probes
    if _probes is None:
        if not os.path.exists(PROBES_LIB_PATH):
            raise LibraryMissing(f"{PROBES_LIB_PATH} is missing: build it with `python -m block_scaled_fp8_bfp8_amd.build`")
        handle = ctypes.CDLL(PROBES_LIB_PATH)
        for name, restype, argtypes in PROBE_SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = restype
            fn.argtypes = argtypes
        _probes = handle
    return _probes
