"""MI355X-native exact attention forward and backward (FlashAttention-style), bf16/fp16.

The computation runs entirely in the gfx950 HIP kernels behind the C ABI of
include/flash_attn.h; this module only checks and marshals torch tensors
(device memory and streams) into that call. If the library is missing the call
raises: there is no fallback implementation.
"""
from __future__ import annotations

import math

from . import _native
from ._native import (FA_BF16, FA_FP16, FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM,  # noqa: F401
                      FA_ERR_DTYPE, FA_ERR_SCALE, FA_ERR_ALIGN, FA_ERR_ALIAS, FA_ERR_HIP, FA_ERR_ARG,
                      FA_ERR_WORKSPACE, FA_ERR_STRIDE, FA_ERR_SCRATCH, FA_SPLITKV_SCRATCH_BYTES,
                      FA_FP8_ROWS, FA_FP8_KEYS_T, FA_FP8_E4M3, FA_FP8_E5M2, FA_FWD_KERNEL_PIPELINED,
                      FA_FWD_KERNEL_PINGPONG)

__all__ = ["forward", "backward", "forward_splitkv", "flash_attn_fwd", "flash_attn_fwd_strided",
           "flash_attn_fwd_splitkv", "flash_attn_fwd_splitkv_noalloc", "flash_attn_bwd",
           "splitkv_plan", "splitkv_workspace_size", "quantize_fp8", "flash_attn_fwd_fp8", "forward_fp8",
           "flash_attn_strerror", "flash_attn_abi_version", "flash_attn_fwd_kernel"]


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, call: str = "flash_attn_fwd"):
        self.status = status
        super().__init__(f"{call} failed ({status}): {_native.strerror(status)}")


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_FP16
    raise TypeError(f"q/k/v must be bfloat16 or float16, got {t.dtype}")


def flash_attn_fwd(q, k, v, o, lse, causal: bool = False, scale: float | None = None, stream=None) -> None:
    """Run the kernel on caller-owned tensors (the C entry point with torch arguments).

    q, k, v, o: contiguous [B, H, N, d] bf16/fp16 CUDA tensors of one dtype;
    lse: contiguous [B, H, N] float32. ``stream`` is a torch.cuda.Stream (default:
    the current stream). Asynchronous, like the C call.
    """
    import torch

    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 with shape [B, H, N]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = _native.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, causal, scale, stream.cuda_stream, dtype)
    if st != FA_OK:
        raise FlashAttnError(st)


def flash_attn_fwd_strided(q, k, v, o, lse, causal: bool = False, scale: float | None = None,
                           stream=None) -> None:
    """The strided entry point on caller-owned [B, H, N, d] views (any strides with the
    head dimension contiguous; d a multiple of 8 up to 256); lse [B, H, N] float32 with
    contiguous rows."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 with shape [B, H, N]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on q's device")
        if d > 1 and t.stride(3) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
    if not lse.is_cuda or lse.device != q.device or (N > 1 and lse.stride(2) != 1):
        raise ValueError("lse must be a GPU tensor on q's device with contiguous rows")
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = _native.strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                             q.stride()[:3], k.stride()[:3], v.stride()[:3], o.stride()[:3], lse.stride()[:2],
                             causal, scale, stream.cuda_stream, dtype)
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_strided")


def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate O (q's dtype, contiguous) and LSE (float32) and run the forward pass.
    Returns (o, lse). Contiguous inputs with d of 64, 128 or 256 take flash_attn_fwd; other
    layouts and head dimensions take flash_attn_fwd_strided."""
    import torch

    B, H, N, d = q.shape
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if d in (64, 128, 256) and all(t.is_contiguous() for t in (q, k, v)):
        flash_attn_fwd(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)
    else:
        flash_attn_fwd_strided(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)
    return o, lse


def _check_fwd_tensors(q, k, v, o, lse):
    import torch

    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, H, N, _ = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 with shape [B, H, N]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")


def splitkv_plan(B: int, H: int, N: int, d: int, causal: bool, cus: int) -> int:
    """Split count the library chooses for a device with ``cus`` compute units."""
    st = _native.splitkv_plan(B, H, N, d, causal, cus)
    if st < 1:
        raise FlashAttnError(st, "flash_attn_fwd_splitkv_plan")
    return st


def splitkv_workspace_size(B: int, H: int, N: int, d: int, causal: bool, num_splits: int) -> int:
    """Workspace bytes flash_attn_fwd_splitkv needs for ``num_splits`` (>= 1)."""
    st = _native.splitkv_workspace_size(B, H, N, d, causal, num_splits)
    if st < 0:
        raise FlashAttnError(int(st), "flash_attn_fwd_splitkv_workspace_size")
    return int(st)


def flash_attn_fwd_splitkv(q, k, v, o, lse, workspace, causal: bool = False, scale: float | None = None,
                           num_splits: int = 0, stream=None) -> None:
    """The key-split forward on caller-owned tensors (the C entry point with torch arguments).

    workspace: a CUDA tensor (any dtype, contiguous) of at least
    splitkv_workspace_size(...) bytes for the resolved split count, or None when
    that count is 1.
    """
    import torch

    _check_fwd_tensors(q, k, v, o, lse)
    B, H, N, d = q.shape
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if workspace is None:
        ws, ws_bytes = 0, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous GPU tensor on q's device")
        ws, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = _native.splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             B, H, N, d, causal, scale, num_splits, ws, ws_bytes, stream.cuda_stream, dtype)
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_splitkv")


def flash_attn_fwd_splitkv_noalloc(q, k, v, o, lse, causal: bool = False, scale: float | None = None,
                                   num_splits: int = 0, stream=None) -> None:
    """The key-split forward with its partial results in the library's fixed device
    array (FA_SPLITKV_SCRATCH_BYTES per GPU) instead of a workspace: no device memory
    is allocated by the call. Calls that overlap in time on one GPU race."""
    import torch

    _check_fwd_tensors(q, k, v, o, lse)
    B, H, N, d = q.shape
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = _native.splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         B, H, N, d, causal, scale, num_splits, stream.cuda_stream, dtype)
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_splitkv_noalloc")


def forward_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0,
                    stream=None):
    """Allocate O, LSE and the split workspace and run the key-split forward. Returns
    (o, lse, splits) with the split count used. num_splits = 0 lets the library
    choose from the device's compute-unit count."""
    import torch

    B, H, N, d = q.shape
    if num_splits == 0:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = splitkv_plan(B, H, N, d, causal, cus)
    nbytes = splitkv_workspace_size(B, H, N, d, causal, num_splits)
    ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=q.device) if nbytes else None
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    flash_attn_fwd_splitkv(q, k, v, o, lse, ws, causal=causal, scale=scale, num_splits=num_splits, stream=stream)
    splits = nbytes // max(1, B * H * N * (d + 1) * 4) if nbytes else 1
    return o, lse, splits


def flash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, causal: bool = False, scale: float | None = None,
                   stream=None) -> None:
    """Run the backward kernels on caller-owned tensors (the C entry point with torch arguments).

    q, k, v, o, dout, dq, dk, dv: contiguous [B, H, N, d] CUDA tensors of q's dtype;
    lse (the forward's) and delta (workspace): contiguous [B, H, N] float32.
    Asynchronous on ``stream`` (default: the current stream).
    """
    import torch

    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    B, H, N, d = q.shape
    for name, t in (("lse", lse), ("delta", delta)):
        if t.shape != (B, H, N) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 with shape [B, H, N]")
    tensors = (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse), ("dq", dq), ("dk", dk),
               ("dv", dv), ("delta", delta))
    for name, t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = _native.bwd_raw(*(t.data_ptr() for _, t in tensors), B, H, N, d, causal, scale, stream.cuda_stream, dtype)
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd")


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate dq, dk, dv (q's dtype) and the delta workspace and run the backward pass.

    o and lse are the forward's outputs for the same q, k, v, causal and scale.
    Returns (dq, dk, dv).
    """
    import torch

    B, H, N, _ = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    flash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, causal=causal, scale=scale, stream=stream)
    return dq, dk, dv


_FP8_FORMATS = {"e4m3": FA_FP8_E4M3, "e5m2": FA_FP8_E5M2}


def _fp8_format(fmt: str) -> int:
    if fmt not in _FP8_FORMATS:
        raise ValueError(f"fp8 format must be one of {sorted(_FP8_FORMATS)}, not {fmt!r}")
    return _FP8_FORMATS[fmt]


def quantize_fp8(x, keys_transposed: bool = False, stream=None, fmt: str = "e4m3"):
    """Block-quantize a contiguous [B, H, N, d] bf16/fp16 CUDA tensor to FP8 (fmt "e4m3"
    or "e5m2").

    Returns (x8, scale_codes): x8 is uint8 [B, H, N, d] (rows layout) or
    [B, H, ceil(N/64), d, 64] (keys-transposed layout, for values); scale_codes is
    int32 [B, H, ceil(N/64)] holding e + 127 of each 64-row block's scale 2^e.
    """
    import torch

    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] GPU tensor")
    B, H, N, d = x.shape
    t = -(-N // 64)
    shape8 = (B, H, t, d, 64) if keys_transposed else (B, H, N, d)
    x8 = torch.empty(shape8, dtype=torch.uint8, device=x.device)
    se = torch.empty((B, H, t), dtype=torch.int32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = _native.quantize_raw(x.data_ptr(), x8.data_ptr(), se.data_ptr(), B, H, N, d,
                              FA_FP8_KEYS_T if keys_transposed else FA_FP8_ROWS, stream.cuda_stream, _dtype_code(x),
                              _fp8_format(fmt))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_quantize_fp8")
    return x8, se


def flash_attn_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, o, lse, causal: bool = False,
                       scale: float | None = None, stream=None, fmt: str = "e4m3") -> None:
    """The FP8 forward on caller-owned tensors (outputs of quantize_fp8 in format fmt;
    o [B, H, N, d] bf16/fp16 with d 64 or 128, and lse [B, H, N] float32)."""
    import torch

    B, H, N, d = o.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8t", v8t), ("q_scale", q_scale), ("k_scale", k_scale),
                    ("v_scale", v_scale), ("o", o), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous() or t.device != o.device:
            raise ValueError(f"{name} must be a contiguous GPU tensor on o's device")
    if q8.shape != (B, H, N, d) or k8.shape != (B, H, N, d) or lse.shape != (B, H, N):
        raise ValueError("shape mismatch among q8, k8, o, lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(o.device)
    st = _native.fp8_raw(q8.data_ptr(), k8.data_ptr(), v8t.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
                         v_scale.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, causal, scale,
                         stream.cuda_stream, _dtype_code(o), _fp8_format(fmt))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_fp8")


def forward_fp8(q, k, v, causal: bool = False, scale: float | None = None, stream=None, fmt: str = "e4m3"):
    """Quantize q, k, v to FP8 (fmt "e4m3" or "e5m2", 64-row blocks) and run the FP8
    forward; o has q's dtype. Returns (o, lse)."""
    import torch

    q8, qs = quantize_fp8(q, stream=stream, fmt=fmt)
    k8, ks = quantize_fp8(k, stream=stream, fmt=fmt)
    v8, vs = quantize_fp8(v, keys_transposed=True, stream=stream, fmt=fmt)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    flash_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, causal=causal, scale=scale, stream=stream, fmt=fmt)
    return o, lse


def flash_attn_strerror(status: int) -> str:
    return _native.strerror(status)


def flash_attn_abi_version() -> int:
    return _native.abi_version()


def flash_attn_fwd_kernel(N: int, d: int, causal: bool = False) -> str:
    """Name of the forward kernel an unsplit call of this shape runs: "pipelined" or
    "pingpong" (flash_attn_fwd_kernel; FLASH_ATTN_FWD_KERNEL forces one)."""
    st = _native.fwd_kernel(N, d, causal)
    if st < 0:
        raise FlashAttnError(st, "flash_attn_fwd_kernel")
    return "pipelined" if st == FA_FWD_KERNEL_PIPELINED else "pingpong"
