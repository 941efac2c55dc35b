"""Pins for the FP8 (E4M3 and E5M2) quantization oracle (CPU only).

oracle.fp8 is checked against torch's own float8_e4m3fn and float8_e5m2 conversions
(independent implementations of the same OCP formats and rounding), the formats'
defining values,
a brute-force search for the block exponent, the round-to-nearest error bound, and
torch's CPU float64 attention on the dequantized inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.dense import attention

RNG = np.random.default_rng(88)


def _torch_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_defining_values():
    d = fp8.e4m3_decode
    assert d(0x38) == 1.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x07) == 7 * 2.0 ** -9 and d(0x01) == 2.0 ** -9
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and math.copysign(1, d(0x80)) < 0
    assert d(0xC0) == -2.0 and d(0x3F) == 1.875
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    vals = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)          # codes 0..126 increase strictly


def test_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_matches_torch():
    vals = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties
    rnd = np.ldexp(RNG.uniform(-1, 1, 20000), RNG.integers(-12, 9, 20000))
    rnd = rnd[np.abs(rnd) <= 448]
    x = np.concatenate([vals, -vals, mids, -mids, rnd, [0.0, -0.0, 2.0 ** -11, -2.0 ** -11]])
    x = x.astype(np.float32).astype(np.float64)             # values torch sees exactly
    assert np.array_equal(fp8.e4m3_encode(x), _torch_codes(x))


def test_encode_rejects_out_of_range():
    for bad in (449.0, -1e4, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            fp8.e4m3_encode(np.array([bad]))


@pytest.mark.parametrize("amax", list(np.ldexp(RNG.uniform(0.01, 1.0, 40), RNG.integers(-30, 30, 40))))
def test_block_exponent_is_the_smallest(amax):
    e = fp8.block_scale_exp(amax)
    assert amax <= 448 * 2.0 ** e
    assert amax > 448 * 2.0 ** (e - 1)


def test_block_exponent_edges():
    for k in (-20, -3, 0, 1, 7, 40):
        assert fp8.block_scale_exp(448 * 2.0 ** k) == k
        assert fp8.block_scale_exp(448 * 2.0 ** k * (1 + 2 ** -40)) == k + 1
    assert fp8.block_scale_exp(0.0) == 0
    assert fp8.block_scale_exp(2.0 ** -140) == -127          # limited to the E8M0 range
    assert fp8.block_scale_exp(2.0 ** 200) == 127


def test_quantize_error_bound_and_layout():
    """Every value within half a unit of E4M3 at its magnitude, times the block scale:
    |deq - x| <= 2^-4 |x| + 2^(e - 10); blocks of 64 rows have their own exponent."""
    x = RNG.standard_normal((2, 3, 200, 16)) * np.array([1.0, 1e-3, 50.0])[None, :, None, None]
    x[0, 0, 64:128] *= 1e4                                   # one block much larger than its neighbours
    codes, exps = fp8.quantize_blocks(x)
    assert exps.shape == (2, 3, 4)
    deq = fp8.dequantize_blocks(codes, exps)
    row_e = np.repeat(exps, 64, axis=-1)[..., :200, None]
    assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + np.ldexp(1.0, row_e - 10))
    assert exps[0, 0, 1] > exps[0, 0, 0] + 10
    for t in range(4):                                       # the block maximum is not clipped
        blk = np.abs(x[..., 64 * t:64 * (t + 1), :]).max(axis=(-1, -2))
        assert np.all(blk <= 448 * np.ldexp(1.0, exps[..., t]))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_on_dequantized_inputs(causal):
    """attention_dequantized equals torch CPU float64 SDPA and the dense oracle."""
    x = [fp8.dequantize_blocks(*fp8.quantize_blocks(RNG.standard_normal((2, 2, 150, 32)))) for _ in range(3)]
    o, lse = fp8.attention_dequantized(*x, 0.2, causal=causal)
    t = torch.nn.functional.scaled_dot_product_attention(*(torch.tensor(a) for a in x), is_causal=causal,
                                                         scale=0.2)
    np.testing.assert_allclose(o, t.numpy(), rtol=1e-11, atol=1e-12)
    ro, rl = attention(*x, 0.2, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


# ---- E5M2 ----

def _torch_codes_e5(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_defining_values():
    d = fp8.e5m2_decode
    assert d(0x3C) == 1.0 and d(0x7B) == 57344.0 and d(0xFB) == -57344.0
    assert d(0x04) == 2.0 ** -14 and d(0x03) == 3 * 2.0 ** -16 and d(0x01) == 2.0 ** -16
    assert d(0x00) == 0.0 and math.copysign(1, d(0x80)) < 0
    assert d(0x3D) == 1.25 and d(0x3F) == 1.75 and d(0xC0) == -2.0
    assert d(0x7C) == np.inf and d(0xFC) == -np.inf
    assert np.isnan(d(0x7D)) and np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    vals = d(np.arange(0x7C, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)          # codes 0..123 increase strictly


def test_e5m2_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.tensor(codes).view(torch.float8_e5m2).double().numpy()
    mine = fp8.e5m2_decode(codes)
    both_nan = np.isnan(t) & np.isnan(mine)
    assert np.array_equal(np.where(both_nan, 0, t), np.where(both_nan, 0, mine))


def test_e5m2_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)
    assert np.array_equal(fp8.e5m2_encode(fp8.e5m2_decode(codes)), codes)


def test_e5m2_encode_matches_torch():
    vals = fp8.e5m2_decode(np.arange(0x7C, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties
    rnd = np.ldexp(RNG.uniform(-1, 1, 20000), RNG.integers(-20, 17, 20000))
    rnd = rnd[np.abs(rnd) <= 57344]
    x = np.concatenate([vals, -vals, mids, -mids, rnd, [0.0, -0.0, 2.0 ** -17, -3 * 2.0 ** -17]])
    x = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(fp8.e5m2_encode(x), _torch_codes_e5(x))


def test_e5m2_encode_rejects_out_of_range():
    for bad in (57345.0, -1e6, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            fp8.e5m2_encode(np.array([bad]))


def test_e5m2_block_exponent():
    for k in (-20, -3, 0, 1, 40):
        assert fp8.block_scale_exp(57344 * 2.0 ** k, fp8.E5M2_MAX) == k
        assert fp8.block_scale_exp(57344 * 2.0 ** k * (1 + 2 ** -40), fp8.E5M2_MAX) == k + 1
    for amax in np.ldexp(RNG.uniform(0.01, 1.0, 40), RNG.integers(-30, 30, 40)):
        e = fp8.block_scale_exp(amax, fp8.E5M2_MAX)
        assert amax <= 57344 * 2.0 ** e < 2 * amax


def test_e5m2_quantize_error_bound():
    """Every value within half a unit of E5M2 at its magnitude, times the block scale:
    |deq - x| <= 2^-3 |x| + 2^(e - 17)."""
    x = RNG.standard_normal((2, 3, 200, 16)) * np.array([1.0, 1e-3, 50.0])[None, :, None, None]
    codes, exps = fp8.quantize_blocks(x, fmt="e5m2")
    deq = fp8.dequantize_blocks(codes, exps, fmt="e5m2")
    row_e = np.repeat(exps, 64, axis=-1)[..., :200, None]
    assert np.all(np.abs(deq - x) <= 2.0 ** -3 * np.abs(x) + np.ldexp(1.0, row_e - 17))
    # the same values through E4M3 are closer (one more mantissa bit)
    deq4 = fp8.dequantize_blocks(*fp8.quantize_blocks(x))
    assert np.abs(deq4 - x).mean() < np.abs(deq - x).mean()


# ---- accumulation model (the A8 term of the FP8 tolerance) ----

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_accumulation_model_bound(fmt):
    """The aligned-accumulator model of one K = 64 instruction stays within
    ACC_REL * sum |a_i b_i| of the exact dot product (ACC_REL = 64 * 2^-18 = 2^-12),
    on random FP8 operands of mixed magnitudes; the bound is reached to within a small
    factor (cancellation with many small terms), so the model is not vacuous."""
    fmax, encode, decode = fp8.FORMATS[fmt]
    assert fp8.ACC_REL == 2.0 ** -12
    worst = 0.0
    for _ in range(400):
        a = decode(encode(np.clip(RNG.standard_normal(64) * np.ldexp(1.0, RNG.integers(-6, 6, 64)), -fmax, fmax)))
        b = decode(encode(np.clip(RNG.standard_normal(64) * 4.0, -fmax, fmax)))
        exact = math.fsum(a * b)
        got = fp8.aligned_dot(a, b)
        bound = fp8.ACC_REL * float(np.sum(np.abs(a * b)))
        assert abs(got - exact) <= bound
        worst = max(worst, abs(got - exact) / bound)
    assert worst > 1e-3


def test_accumulation_model_exact_cases():
    """Products that all sit on the quantum are summed exactly; one product far below
    the largest is truncated toward zero; fp32 sequential accumulation of the same
    products is well inside the model's bound."""
    a = np.array([1.0, 2.0 ** -3, -0.5] + [0.0] * 61)
    b = np.ones(64)
    assert fp8.aligned_dot(a, b) == 0.625
    c = np.array([1.0, 2.0 ** -20] + [0.0] * 62)
    assert fp8.aligned_dot(c, b) == 1.0                        # below 2^(0 - 18): dropped
    assert fp8.aligned_dot(-c, b) == -1.0                      # toward zero on both signs
    x = fp8.e4m3_decode(fp8.e4m3_encode(np.clip(RNG.standard_normal(64) * 8, -448, 448)))
    y = fp8.e4m3_decode(fp8.e4m3_encode(np.clip(RNG.standard_normal(64) * 8, -448, 448)))
    acc = np.float32(0.0)
    for t in (x * y).astype(np.float32):
        acc = np.float32(acc + t)
    assert abs(float(acc) - math.fsum(x * y)) <= fp8.ACC_REL * np.sum(np.abs(x * y))

