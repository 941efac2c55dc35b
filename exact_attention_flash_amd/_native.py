"""ctypes view of the C ABI declared in include/flash_attn.h."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

FA_BF16 = 0
FA_FP16 = 1

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEADDIM = -3
FA_ERR_DTYPE = -4
FA_ERR_SCALE = -5
FA_ERR_ALIGN = -6
FA_ERR_ALIAS = -7
FA_ERR_HIP = -8
FA_ERR_ARG = -9
FA_ERR_WORKSPACE = -10
FA_ERR_STRIDE = -11
FA_ERR_SCRATCH = -12

# bytes of the library's fixed partial-result array (FA_SPLITKV_SCRATCH_BYTES)
FA_SPLITKV_SCRATCH_BYTES = 65 * 1024 * 1024

FA_FP8_ROWS = 0
FA_FP8_KEYS_T = 1
FA_FP8_E4M3 = 0
FA_FP8_E5M2 = 1
FA_FWD_KERNEL_PIPELINED = 1
FA_FWD_KERNEL_PINGPONG = 2

_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"HIP library {LIB_PATH} is missing: build it with exact_attention_flash_amd.build.build() "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        L.flash_attn_fwd.restype = ctypes.c_int
        L.flash_attn_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
        ]
        L.flash_attn_fwd_validate.restype = ctypes.c_int
        L.flash_attn_fwd_validate.argtypes = L.flash_attn_fwd.argtypes
        P64 = ctypes.POINTER(ctypes.c_int64)
        L.flash_attn_fwd_strided.restype = ctypes.c_int
        L.flash_attn_fwd_strided.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            P64, P64, P64, P64, P64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
        ]
        L.flash_attn_fwd_strided_validate.restype = ctypes.c_int
        L.flash_attn_fwd_strided_validate.argtypes = L.flash_attn_fwd_strided.argtypes
        vp = ctypes.c_void_p
        L.flash_attn_quantize_fp8.restype = ctypes.c_int
        L.flash_attn_quantize_fp8.argtypes = [vp, vp, vp] + [ctypes.c_int64] * 4 + [ctypes.c_int, vp, ctypes.c_int,
                                                                              ctypes.c_int]
        L.flash_attn_quantize_fp8_validate.restype = ctypes.c_int
        L.flash_attn_quantize_fp8_validate.argtypes = L.flash_attn_quantize_fp8.argtypes
        L.flash_attn_fwd_fp8.restype = ctypes.c_int
        L.flash_attn_fwd_fp8.argtypes = [vp] * 8 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_float, vp,
                                                                          ctypes.c_int, ctypes.c_int]
        L.flash_attn_fwd_fp8_validate.restype = ctypes.c_int
        L.flash_attn_fwd_fp8_validate.argtypes = L.flash_attn_fwd_fp8.argtypes
        L.flash_attn_fwd_splitkv.restype = ctypes.c_int
        L.flash_attn_fwd_splitkv.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64,
            ctypes.c_void_p, ctypes.c_int,
        ]
        L.flash_attn_fwd_splitkv_validate.restype = ctypes.c_int
        L.flash_attn_fwd_splitkv_validate.argtypes = L.flash_attn_fwd_splitkv.argtypes
        L.flash_attn_fwd_splitkv_plan.restype = ctypes.c_int
        L.flash_attn_fwd_splitkv_plan.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int]
        L.flash_attn_fwd_splitkv_workspace_size.restype = ctypes.c_int64
        L.flash_attn_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int]
        L.flash_attn_fwd_splitkv_noalloc.restype = ctypes.c_int
        L.flash_attn_fwd_splitkv_noalloc.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ]
        L.flash_attn_bwd.restype = ctypes.c_int
        L.flash_attn_bwd.argtypes = [ctypes.c_void_p] * 10 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
        ]
        L.flash_attn_bwd_validate.restype = ctypes.c_int
        L.flash_attn_bwd_validate.argtypes = L.flash_attn_bwd.argtypes
        L.flash_attn_strerror.restype = ctypes.c_char_p
        L.flash_attn_strerror.argtypes = [ctypes.c_int]
        L.flash_attn_abi_version.restype = ctypes.c_int
        L.flash_attn_abi_version.argtypes = []
        L.flash_attn_fwd_kernel.restype = ctypes.c_int
        L.flash_attn_fwd_kernel.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        _lib = L
    return _lib


def fwd_raw(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype) -> int:
    """Call flash_attn_fwd with integer addresses; returns the status code."""
    return lib().flash_attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), stream, dtype)


def validate_raw(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype) -> int:
    """Call flash_attn_fwd_validate (host checks only, never launches)."""
    return lib().flash_attn_fwd_validate(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), stream, dtype)


def _strides(xs, n):
    if xs is None:
        return None
    if len(xs) != n:
        raise ValueError(f"expected {n} strides, got {len(xs)}")
    return (ctypes.c_int64 * n)(*[int(x) for x in xs])


def strided_raw(q, k, v, o, lse, B, H, N, d, qs, ks, vs, os_, ls, causal, scale, stream, dtype) -> int:
    """Call flash_attn_fwd_strided (strides as sequences: 3 for q/k/v/o, 2 for lse; None -> NULL)."""
    return lib().flash_attn_fwd_strided(q, k, v, o, lse, B, H, N, d, _strides(qs, 3), _strides(ks, 3),
                                        _strides(vs, 3), _strides(os_, 3), _strides(ls, 2), int(causal),
                                        float(scale), stream, dtype)


def validate_strided_raw(q, k, v, o, lse, B, H, N, d, qs, ks, vs, os_, ls, causal, scale, stream, dtype) -> int:
    """Call flash_attn_fwd_strided_validate (host checks only, never launches)."""
    return lib().flash_attn_fwd_strided_validate(q, k, v, o, lse, B, H, N, d, _strides(qs, 3), _strides(ks, 3),
                                                 _strides(vs, 3), _strides(os_, 3), _strides(ls, 2), int(causal),
                                                 float(scale), stream, dtype)


def quantize_raw(x, x8, se, B, H, N, d, layout, stream, dtype, fmt=FA_FP8_E4M3) -> int:
    return lib().flash_attn_quantize_fp8(x, x8, se, B, H, N, d, int(layout), stream, dtype, int(fmt))


def validate_quantize_raw(x, x8, se, B, H, N, d, layout, stream, dtype, fmt=FA_FP8_E4M3) -> int:
    return lib().flash_attn_quantize_fp8_validate(x, x8, se, B, H, N, d, int(layout), stream, dtype, int(fmt))


def fp8_raw(q8, k8, v8t, qs, ks, vs, o, lse, B, H, N, d, causal, scale, stream, out_dtype, fmt=FA_FP8_E4M3) -> int:
    return lib().flash_attn_fwd_fp8(q8, k8, v8t, qs, ks, vs, o, lse, B, H, N, d, int(causal), float(scale), stream,
                                    out_dtype, int(fmt))


def validate_fp8_raw(q8, k8, v8t, qs, ks, vs, o, lse, B, H, N, d, causal, scale, stream, out_dtype,
                     fmt=FA_FP8_E4M3) -> int:
    return lib().flash_attn_fwd_fp8_validate(q8, k8, v8t, qs, ks, vs, o, lse, B, H, N, d, int(causal),
                                             float(scale), stream, out_dtype, int(fmt))


def splitkv_raw(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, ws, ws_bytes, stream, dtype) -> int:
    """Call flash_attn_fwd_splitkv with integer addresses; returns the status code."""
    return lib().flash_attn_fwd_splitkv(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), int(num_splits),
                                        ws, int(ws_bytes), stream, dtype)


def validate_splitkv_raw(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, ws, ws_bytes, stream,
                         dtype) -> int:
    """Call flash_attn_fwd_splitkv_validate (host checks only, never launches)."""
    return lib().flash_attn_fwd_splitkv_validate(q, k, v, o, lse, B, H, N, d, int(causal), float(scale),
                                                 int(num_splits), ws, int(ws_bytes), stream, dtype)


def splitkv_noalloc_raw(q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, stream, dtype) -> int:
    """Call flash_attn_fwd_splitkv_noalloc with integer addresses; returns the status code."""
    return lib().flash_attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, int(causal), float(scale),
                                                int(num_splits), stream, dtype)


def splitkv_plan(B, H, N, d, causal, cus) -> int:
    return lib().flash_attn_fwd_splitkv_plan(B, H, N, d, int(causal), int(cus))


def splitkv_workspace_size(B, H, N, d, causal, num_splits) -> int:
    return lib().flash_attn_fwd_splitkv_workspace_size(B, H, N, d, int(causal), int(num_splits))


def bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, stream, dtype) -> int:
    """Call flash_attn_bwd with integer addresses; returns the status code."""
    return lib().flash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, int(causal), float(scale),
                                stream, dtype)


def validate_bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, stream, dtype) -> int:
    """Call flash_attn_bwd_validate (host checks only, never launches)."""
    return lib().flash_attn_bwd_validate(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, int(causal),
                                         float(scale), stream, dtype)


def strerror(status: int) -> str:
    return lib().flash_attn_strerror(int(status)).decode()


def abi_version() -> int:
    return lib().flash_attn_abi_version()


def fwd_kernel(N, d, causal) -> int:
    """flash_attn_fwd_kernel: FA_FWD_KERNEL_PIPELINED or FA_FWD_KERNEL_PINGPONG, or a negative status."""
    return lib().flash_attn_fwd_kernel(int(N), int(d), int(causal))
