"""FP8 (E4M3) block quantization and attention on the quantized inputs, in float64 --
TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

Source: [IO] "FlashAttention: IO-Aware Tiling, Online Softmax Mathematics, Memory
Hierarchy Dynamics, and Kernel Evolution", section on FlashAttention-3: attention
in 8-bit floating point (E4M3 / E5M2) with block-level quantization and dynamic
scaling factors. The page fixes no more than that; the readings taken here:

* Formats: E4M3 and E5M2 as in the OCP 8-bit floating-point specification (the
  formats the gfx950 matrix cores take). E4M3: 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits; subnormals below 2^-6 with spacing 2^-9; largest finite 448;
  no infinities (exponent and mantissa all ones is NaN). E5M2: 1 sign bit, 5
  exponent bits with bias 15, 2 mantissa bits; subnormals below 2^-14 with spacing
  2^-16; largest finite 57344; exponent all ones is infinity (mantissa 0) or NaN.
  Rounding to nearest, ties to even, in both.
* Blocks: 64 consecutive rows of one (batch, head) slice of Q, K or V (the key
  tile of the kernels), each with its own scale.
* Dynamic scale: a power of two 2^e with e the smallest integer such that the
  block's largest magnitude a satisfies a <= F * 2^e, F the format's largest finite
  value (e = 0 for an all-zero block), limited to [-127, 127] (the exponent range of
  an E8M0 scale). Stored values are FP8(x / 2^e); x / 2^e is exact, so the only
  rounding is the FP8 one.
* The attention the FP8 path computes is exact attention on the dequantized
  inputs code * 2^e; ``attention_dequantized`` evaluates it with the dense
  definition (oracle.dense is not imported; the same three-pass softmax is
  written out here).
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
BLOCK = 64


def e4m3_decode(codes):
    """Float64 values of E4M3 codes (uint8 array); NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7)))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


# all finite non-negative codes in increasing order of value
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x):
    """Round finite values with |x| <= 448 to the nearest E4M3 code, ties to the code
    with an even mantissa (the even code). Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: values must be finite with |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _POS_VALS[hi], _POS_VALS[lo]
    dhi, dlo = vhi - a, a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    pick_hi |= vhi == a
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    # the sign is kept, also when the magnitude rounds to zero (-0 is code 0x80)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def e5m2_decode(codes):
    """Float64 values of E5M2 codes (uint8 array); infinity and NaN codes decode to them."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    val = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.ldexp(1.0, (e - 15)))
    val = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


_POS_CODES_E5 = np.arange(0x7C, dtype=np.uint8)   # finite non-negative codes, increasing
_POS_VALS_E5 = e5m2_decode(_POS_CODES_E5)


def _encode_nearest_even(x, codes, vals, fmax, name):
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > fmax):
        raise ValueError(f"{name}: values must be finite with |x| <= {fmax:g}")
    a = np.abs(x)
    hi = np.searchsorted(vals, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = vals[hi], vals[lo]
    dhi, dlo = vhi - a, a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    pick_hi |= vhi == a
    code = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    # the sign is kept, also when the magnitude rounds to zero (-0 is code 0x80)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def e5m2_encode(x):
    """Round finite values with |x| <= 57344 to the nearest E5M2 code, ties to the
    code with an even mantissa. Returns uint8 codes."""
    return _encode_nearest_even(x, _POS_CODES_E5, _POS_VALS_E5, E5M2_MAX, "e5m2_encode")


# format name -> (largest finite value, encode, decode)
FORMATS = {"e4m3": (E4M3_MAX, None, None), "e5m2": (E5M2_MAX, None, None)}


def block_scale_exp(amax, fmax=E4M3_MAX):
    """Smallest integer e with amax <= fmax * 2^e (0 for amax = 0), limited to [-127, 127]."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / fmax))
    # make the comparison exact whatever log2 rounds to
    while amax > fmax * 2.0 ** e:
        e += 1
    while amax <= fmax * 2.0 ** (e - 1):
        e -= 1
    return max(-127, min(127, e))


def quantize_blocks(x, block=BLOCK, fmt="e4m3"):
    """Quantize [..., N, d] float64 values per block of `block` rows of each slice to
    `fmt` ("e4m3" or "e5m2").

    Returns (codes uint8 [..., N, d], exps int64 [..., ceil(N / block)]).
    """
    fmax, encode, _ = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    lead, (n, d) = x.shape[:-2], x.shape[-2:]
    g = int(np.prod(lead)) if lead else 1
    xf = x.reshape(g, n, d)
    t = -(-n // block)
    codes = np.zeros((g, n, d), dtype=np.uint8)
    exps = np.zeros((g, t), dtype=np.int64)
    for gi in range(g):
        for ti in range(t):
            blk = xf[gi, ti * block:(ti + 1) * block]
            e = block_scale_exp(np.abs(blk).max() if blk.size else 0.0, fmax)
            exps[gi, ti] = e
            codes[gi, ti * block:(ti + 1) * block] = encode(np.ldexp(blk, -e))
    return codes.reshape(x.shape), exps.reshape(lead + (t,))


def dequantize_blocks(codes, exps, block=BLOCK, fmt="e4m3"):
    """Values code * 2^e of quantize_blocks' output, float64 [..., N, d]."""
    _, _, decode = FORMATS[fmt]
    codes = np.asarray(codes, dtype=np.uint8)
    lead, (n, d) = codes.shape[:-2], codes.shape[-2:]
    g = int(np.prod(lead)) if lead else 1
    cf = codes.reshape(g, n, d)
    ef = np.asarray(exps, dtype=np.int64).reshape(g, -1)
    row_e = np.repeat(ef, block, axis=1)[:, :n]                  # exponent of every row
    return np.ldexp(decode(cf), row_e[..., None]).reshape(codes.shape)


# ---- accumulation model of the scaled FP8 matrix instruction ----
# The pages give no accumulation precision for FP8 matrix products, and the
# instruction's internal one is not stated here either. The tolerance of the FP8 path
# takes this model: one instruction forms the exact products of its K = 64 FP8 pairs
# (an E4M3 or E5M2 product has at most 8 significant bits), aligns them to the
# leading bit of the largest, truncates each toward zero below
# 2^(emax - ACC_FRAC_BITS), and adds the sum to its fp32 accumulator. Its error per
# instruction is at most 64 * 2^(emax - ACC_FRAC_BITS) <= ACC_REL * sum |products|.
ACC_TERMS = 64
ACC_FRAC_BITS = 18
ACC_REL = ACC_TERMS * 2.0 ** -ACC_FRAC_BITS   # 2^-12


def aligned_dot(a, b, frac_bits=ACC_FRAC_BITS):
    """One instruction's dot product under the accumulation model: exact products of
    a and b (1-D, FP8 values as float64), aligned to the leading bit of the largest,
    truncated toward zero below 2^(emax - frac_bits), summed exactly."""
    p = np.asarray(a, dtype=np.float64) * np.asarray(b, dtype=np.float64)
    amax = float(np.max(np.abs(p))) if p.size else 0.0
    if amax == 0.0:
        return 0.0
    emax = math.floor(math.log2(amax))
    quantum = math.ldexp(1.0, emax - frac_bits)
    return math.fsum(np.trunc(p / quantum) * quantum)


def attention_dequantized(q, k, v, scale, causal=False, row_block=512):
    """Exact attention (float64) of already-dequantized q, k, v [..., N, d]: scores
    scale * q k^T, causal pairs dropped, three-pass softmax over each full row,
    O = P V, LSE = m + ln l. Returns (O, LSE)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    lead, (n, d) = q.shape[:-2], q.shape[-2:]
    g = int(np.prod(lead)) if lead else 1
    qf, kf, vf = (t.reshape(g, n, d) for t in (q, k, v))
    out = np.zeros((g, n, d))
    lse = np.zeros((g, n))
    keys = np.arange(n)
    for gi in range(g):
        for r0 in range(0, n, row_block):
            rows = np.arange(r0, min(n, r0 + row_block))
            s = float(scale) * (qf[gi, rows] @ kf[gi].T)
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            out[gi, rows] = (e / l) @ vf[gi]
            lse[gi, rows] = (m + np.log(l))[:, 0]
    return out.reshape(lead + (n, d)), lse.reshape(lead + (n,))


FORMATS["e4m3"] = (E4M3_MAX, e4m3_encode, e4m3_decode)
FORMATS["e5m2"] = (E5M2_MAX, e5m2_encode, e5m2_decode)
