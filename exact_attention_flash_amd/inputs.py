"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and converts them to the 16-bit storage
formats; it holds none of the attention arithmetic. Both the GPU path's tests
and benchmark and the CPU oracle receive their inputs from here, so that the two
sides see the very same bytes.

Recipe (every workload): numpy ``default_rng(seed)`` (PCG64) draws float32
standard normals of shape ``[B, H, N, d]`` in the order Q, then K, then V. Each
array is multiplied by ``sigma`` in float32 and rounded to the storage dtype with
round-to-nearest-even. Arrays are kept as raw uint16 bit patterns so that the
oracle can widen them to float64 exactly and the GPU gets identical bytes.

The five workloads below are the problem sizes the forward pass is measured and
checked on: a single small head, a multi-head d=64 case, a LLaMA-7B-shaped causal
case (the headline), a long-context causal case and an edge-case stress with
ragged tiles and extreme logits.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
DTYPES = (BF16, FP16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    sigma: float
    causal: tuple  # which masks to run on the same inputs
    seed: int

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def flops(self, causal: bool) -> float:
        """Metric FLOP count: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f

    def compulsory_bytes(self) -> int:
        """Q, K, V read once and O written once (16-bit) plus fp32 LSE."""
        return 8 * self.B * self.H * self.N * self.d + 4 * self.B * self.H * self.N


WORKLOADS = {
    "single_head_n256_d64": Workload("single_head_n256_d64", 1, 1, 256, 64, FP16, 1.0, (False,), 1),
    "mha_b4_h16_n1024_d64": Workload("mha_b4_h16_n1024_d64", 4, 16, 1024, 64, BF16, 1.0, (False,), 2),
    "llama7b_b2_h32_n4096_d128_causal": Workload(
        "llama7b_b2_h32_n4096_d128_causal", 2, 32, 4096, 128, BF16, 1.0, (True,), 3),
    "longctx_b1_h32_n16384_d128_causal": Workload(
        "longctx_b1_h32_n16384_d128_causal", 1, 32, 16384, 128, BF16, 1.0, (True,), 4),
    "stress_b3_h8_n4099_d128_sigma8": Workload(
        "stress_b3_h8_n4099_d128_sigma8", 3, 8, 4099, 128, FP16, 8.0, (False, True), 5),
}
HEADLINE = "llama7b_b2_h32_n4096_d128_causal"

# Shapes with fewer (batch, head, 256-row query tile) work items than the GPU has
# compute units, where the key-split forward applies: a few heads of a long causal
# sequence (e.g. one tensor-parallel shard's heads) and one long non-causal head.
SPLIT_WORKLOADS = {
    "few_heads_b1_h4_n4096_d128_causal": Workload(
        "few_heads_b1_h4_n4096_d128_causal", 1, 4, 4096, 128, BF16, 1.0, (True,), 6),
    "one_head_b1_h1_n8192_d128": Workload("one_head_b1_h1_n8192_d128", 1, 1, 8192, 128, BF16, 1.0, (False,), 7),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits.

    Only finite inputs are supported (the generators never produce others).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    b = x.view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy rounds to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="raise"):
        h = x.astype(np.float16)
    return h.view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP16:
        return f32_to_fp16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 16-bit storage patterns to float64 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    return bits_to_f64(bits, dtype).astype(np.float32)


def draw_qkv(shape, dtype: str, sigma: float, seed: int):
    """Q, K, V as uint16 bit arrays of ``shape`` following the recipe above."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out.append(to_bits(x, dtype))
    return tuple(out)


def workload_qkv(w: Workload, seed_offset: int = 0):
    return draw_qkv(w.shape, w.dtype, w.sigma, w.seed + seed_offset)


def default_scale(d: int) -> float:
    """1/sqrt(d) as the float32 value the GPU receives, returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(d)))


def to_torch(bits: np.ndarray, dtype: str, device="cpu"):
    """Reinterpret uint16 bits as a torch bf16/fp16 tensor (no rounding)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.to(device)


def from_torch_bits(t) -> np.ndarray:
    """uint16 bit patterns of a bf16/fp16 torch tensor (any device)."""
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
