"""The seeded input generator: rounding, reproducibility and workload metadata."""
import numpy as np
import pytest
import torch

from exact_attention_flash_amd import inputs
from tests import _golden


def test_bf16_round_to_nearest_even_known_values():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 2.0**-130, 3.0e38], np.float32)
    got = inputs.bits_to_f64(inputs.f32_to_bf16_bits(x), inputs.BF16)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: the even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2**-6 and got[3] == -1.0
    assert got[4] == np.float64(np.float32(2.0**-130))     # subnormal kept exactly (7 bits)
    assert np.isfinite(got[5])


@pytest.mark.parametrize("dtype,tdtype", [(inputs.BF16, torch.bfloat16), (inputs.FP16, torch.float16)])
def test_rounding_matches_torch(dtype, tdtype):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-12, 12, 100000))).astype(np.float32)
    if dtype == inputs.FP16:
        x = np.clip(x, -60000, 60000)
    bits = inputs.to_bits(x, dtype)
    ref = torch.from_numpy(x).to(tdtype).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    t = inputs.to_torch(bits, dtype)
    assert t.dtype == tdtype
    assert np.array_equal(inputs.from_torch_bits(t), bits)
    assert np.array_equal(inputs.bits_to_f64(bits, dtype), t.double().numpy())


def test_draw_is_seeded_and_ordered():
    a = inputs.draw_qkv((2, 3, 17, 8), inputs.BF16, 1.0, 42)
    b = inputs.draw_qkv((2, 3, 17, 8), inputs.BF16, 1.0, 42)
    c = inputs.draw_qkv((2, 3, 17, 8), inputs.BF16, 1.0, 43)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    # Q, then K, then V from one stream
    rng = np.random.default_rng(42)
    qf = rng.standard_normal((2, 3, 17, 8), dtype=np.float32)
    kf = rng.standard_normal((2, 3, 17, 8), dtype=np.float32)
    assert np.array_equal(a[0], inputs.f32_to_bf16_bits(qf))
    assert np.array_equal(a[1], inputs.f32_to_bf16_bits(kf))


def test_sigma_scaling_statistics():
    q, k, v = inputs.draw_qkv((1, 1, 4096, 64), inputs.FP16, 8.0, 5)
    x = inputs.bits_to_f64(v, inputs.FP16)
    assert abs(x.std() - 8.0) < 0.1 and abs(x.mean()) < 0.1


def test_workload_table():
    w = inputs.WORKLOADS[inputs.HEADLINE]
    assert w.shape == (2, 32, 4096, 128) and w.dtype == inputs.BF16 and w.causal == (True,)
    assert abs(w.flops(True) - 2.749e11) / 2.749e11 < 1e-3
    assert w.compulsory_bytes() == 8 * 2 * 32 * 4096 * 128 + 4 * 2 * 32 * 4096
    s = inputs.WORKLOADS["stress_b3_h8_n4099_d128_sigma8"]
    assert s.causal == (False, True) and s.sigma == 8.0 and s.N % 64 != 0
    assert inputs.default_scale(128) == float(np.float32(1 / np.sqrt(128)))


def test_materialised_score_sizes_printed_by_the_pages():
    """Sizes the pages print for a 16-bit N x N score matrix (2 bytes per element)."""
    for n, heads, bpe, value, unit in _golden.materialised_scores():
        size = n * n * bpe * heads
        div = {"MiB": 2**20, "MB": 1e6, "GB": 1e9}[unit]
        assert round(size / div, 2) == value


def test_half_ulp_of_output_dtypes():
    from tests._parity import half_ulp

    assert half_ulp(1.0, inputs.BF16) == 2.0**-8 and half_ulp(1.99, inputs.BF16) == 2.0**-8
    assert half_ulp(2.0, inputs.BF16) == 2.0**-7 and half_ulp(-3.5, inputs.BF16) == 2.0**-7
    assert half_ulp(47.0, inputs.FP16) == 2.0**-6 and half_ulp(1.0, inputs.FP16) == 2.0**-11
    assert half_ulp(0.0, inputs.FP16) == 2.0**-25 and half_ulp(1e-6, inputs.FP16) == 2.0**-25
    # every representable neighbour pair is exactly two half-ulps apart
    for dt in inputs.DTYPES:
        x = np.float32([0.3, 1.7, 9.1, 47.2])
        b = inputs.to_bits(x, dt)
        lo = inputs.bits_to_f64(b, dt)
        hi = inputs.bits_to_f64(b + 1, dt)
        assert np.allclose(hi - lo, 2 * half_ulp(lo, dt), rtol=0, atol=0)
