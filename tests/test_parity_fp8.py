"""GPU parity of the FP8 path: flash_attn_quantize_fp8 and flash_attn_fwd_fp8 against
oracle.fp8.

* Quantization is byte and index work: the E4M3 / E5M2 codes and the scale codes
  must equal the oracle's bit for bit (rows layout, and the keys-transposed layout
  after undoing its documented key order), for bf16 and fp16 inputs, d = 64 and 128,
  ragged N, an all-zero block and blocks of very different magnitudes.
* The attention is compared with exact attention on the dequantized inputs
  (oracle.fp8.attention_dequantized) with a bound derived from the kernel's
  arithmetic (the pages fix none for FP8), with a factor 4 of slack:

      |O - O*| <= 4 (u8 sum_j p_j |v_j| + eta8 sum_j |v_j| / 256 + a8 sum_j p_j |v_j|
                     + 4 dS max_j |v_j|) + 1/2 ulp(O*)

  u8 = 2^-4 is E4M3's unit roundoff for P (rounded as p' = 256 p), eta8 = 2^-10 half
  its subnormal spacing, a8 = oracle.fp8.ACC_REL = 2^-12 the accumulation error of
  one FP8 matrix instruction relative to the sum of the magnitudes of its terms
  under the CPU model oracle.fp8.aligned_dot (exact products aligned to the largest,
  truncated 18 bits below its leading bit; pinned in tests/test_oracle_fp8.py), and
  dS = a8 scale sum_d |q_d k_d| the resulting error of a score (over the row's keys,
  its maximum). The test thereby checks that the instruction is no less accurate
  than that model. The mean error
  must stay within twice the root mean square of the P rounding model,
  2^-4 / sqrt(3) sqrt(sum_j p_j^2 v_j^2), plus half an ulp. The log-sum-exp carries
  the score error of its row's maximum: |LSE - LSE*| <= max(1e-3, 4 dS) (for unit
  variance inputs 4 dS is below 1e-2; with sigma 8 inputs the scores reach the
  hundreds and dS follows).
* The error against the unquantized inputs (the quantization itself) is reported.
"""
import math
import sys

import numpy as np
import pytest

from exact_attention_flash_amd import inputs
from oracle import fp8 as ofp8
from oracle.dense import attention as oracle_attention
from tests._parity import half_ulp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U8, ETA8, A8 = 2.0 ** -4, 2.0 ** -10, ofp8.ACC_REL


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_flash_amd as fa_mod

    fa_mod._native.lib()
    return fa_mod


def _keys_t_to_rows(x8t, n):
    """Undo the keys-transposed layout: [G, T, d, 64] -> [G, T*64, d] (key order of the block)."""
    g, t, d, _ = x8t.shape
    p = np.arange(64)
    key = 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
    rows = np.zeros((g, t, 64, d), dtype=np.uint8)
    rows[:, :, key, :] = np.swapaxes(x8t, -1, -2)
    return rows.reshape(g, t * 64, d)[:, :n]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("keys_t", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("shape", [(1, 2, 1, 64), (2, 1, 130, 128), (1, 3, 257, 64), (1, 1, 700, 128)])
def test_quantize_bit_exact(fa, shape, dtype, keys_t, fmt):
    B, H, N, d = shape
    rng = np.random.default_rng(1000 + N + d)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.float32(4.0)
    if N > 64:
        x[0, 0, 0:64] = 0.0                                     # an all-zero block
        x[0, -1, 64:min(N, 128)] *= np.float32(3000.0 if dtype == inputs.BF16 else 500.0)
    bits = inputs.to_bits(x, dtype)
    xt = inputs.to_torch(bits, dtype, torch.device("cuda:0"))
    x8, se = fa.quantize_fp8(xt, keys_transposed=keys_t, fmt=fmt)
    torch.cuda.synchronize()
    codes, exps = ofp8.quantize_blocks(inputs.bits_to_f64(bits, dtype), fmt=fmt)
    g = B * H
    got_se = se.cpu().numpy().reshape(g, -1)
    assert np.array_equal(got_se, exps.reshape(g, -1) + 127)
    got = x8.cpu().numpy()
    if keys_t:
        t = -(-N // 64)
        full = got.reshape(g, t, d, 64)
        rows = _keys_t_to_rows(full, N)
        assert np.array_equal(rows, codes.reshape(g, N, d))
        pad = _keys_t_to_rows(full, t * 64)[:, N:]              # keys past N are zero codes
        assert np.all(pad == 0)
    else:
        assert np.array_equal(got.reshape(g, N, d), codes.reshape(g, N, d))


def _fp8_case(fa, shape, dtype, causal, sigma, seed, heads=None, scale=None, fmt="e4m3"):
    B, H, N, d = shape
    scale = float(np.float32(1.0 / math.sqrt(d))) if scale is None else scale
    qb, kb, vb = inputs.draw_qkv(shape, dtype, sigma, seed)
    dev = torch.device("cuda:0")
    q, k, v = (inputs.to_torch(x, dtype, dev) for x in (qb, kb, vb))
    o, lse = fa.forward_fp8(q, k, v, causal=causal, scale=scale, fmt=fmt)
    torch.cuda.synchronize()
    g = B * H
    og = inputs.bits_to_f64(inputs.from_torch_bits(o), dtype).reshape(g, N, d)
    lg = lse.double().cpu().numpy().reshape(g, N)
    heads = range(g) if heads is None else heads
    worst, means, vs_orig, lse_max = 0.0, [], [], []
    for hh in heads:
        xs = [inputs.bits_to_f64(x.reshape(g, N, d)[hh], dtype) for x in (qb, kb, vb)]
        qd, kd, vd = (ofp8.dequantize_blocks(*ofp8.quantize_blocks(x, fmt=fmt), fmt=fmt) for x in xs)
        ro, rl = ofp8.attention_dequantized(qd, kd, vd, scale, causal=causal)
        s = scale * (qd @ kd.T)
        if causal:
            s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
        p = np.exp(s - rl[:, None])                             # exact probabilities
        av = np.abs(vd)
        ds = (A8 * scale * (np.abs(qd) @ np.abs(kd).T) * (p > 0)).max(axis=1)
        bound = 4 * (U8 * (p @ av) + ETA8 / 256 * av.sum(axis=0)[None, :] + A8 * (p @ av)
                     + 4 * ds[:, None] * av.max(axis=0)[None, :]) + half_ulp(ro, dtype)
        err = np.abs(og[hh] - ro)
        assert np.all(np.isfinite(og[hh])) and np.all(np.isfinite(lg[hh]))
        ratio = float((err / bound).max())
        worst = max(worst, ratio)
        assert ratio <= 1.0, f"head {hh}: O error reaches {ratio:.3f} of its bound"
        rms = U8 / math.sqrt(3) * np.sqrt((p ** 2) @ (vd ** 2))
        assert err.mean() <= 2 * rms.mean() + half_ulp(ro, dtype).mean(), f"head {hh}: mean O error {err.mean()}"
        lse_err = np.abs(lg[hh] - rl)
        assert np.all(lse_err <= np.maximum(1e-3, 4 * ds)), f"head {hh}: LSE error {lse_err.max()}"
        means.append(float(err.mean()))
        lse_max.append(float(lse_err.max()))
        oo, _ = oracle_attention(*xs, scale, causal=causal)
        vs_orig.append(float(np.abs(og[hh] - oo).max()))
    return worst, float(np.mean(means)), max(vs_orig), max(lse_max)


SMALL = [(1, 1, 1, 128), (1, 2, 63, 128), (2, 1, 130, 128), (1, 2, 257, 128), (1, 1, 700, 128),
         (1, 1, 1, 64), (1, 2, 63, 64), (2, 1, 130, 64), (1, 2, 257, 64), (1, 1, 700, 64)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("shape", SMALL)
def test_fp8_small(fa, shape, dtype, causal, fmt):
    w, mean, orig, le = _fp8_case(fa, shape, dtype, causal, 1.0, 1100 + SMALL.index(shape), fmt=fmt)
    _log(f"fp8 {fmt} {shape} {dtype} causal={causal}: error/bound {w:.3f}, mean |err| {mean:.2e}, "
         f"LSE err {le:.2e}, max |O - O(unquantized)| {orig:.2e}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_multi_item_workgroups(fa, d, causal, fmt):
    """Several work items per workgroup (16 x 32 slices of two 256-row query tiles,
    the last ragged: 1024 items on at most 256 workgroups), sampled heads."""
    shape, dtype = (16, 32, 450, d), inputs.BF16
    w, mean, orig, le = _fp8_case(fa, shape, dtype, causal, 1.0, 1300 + d + int(causal), heads=[0, 257, 511],
                                  fmt=fmt)
    _log(f"fp8 {fmt} multi-item {shape} causal={causal}: error/bound {w:.3f}, mean |err| {mean:.2e}, "
         f"LSE err {le:.2e}, max |O - O(unquantized)| {orig:.2e}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("name,heads", [("llama7b_b2_h32_n4096_d128_causal", [0, 40, 63]),
                                        ("stress_b3_h8_n4099_d128_sigma8", [0, 23]),
                                        ("mha_b4_h16_n1024_d64", [0, 37, 63])])
def test_fp8_workloads(fa, name, heads, fmt):
    w = inputs.WORKLOADS[name]
    for causal in w.causal:
        ws, mean, orig, le = _fp8_case(fa, w.shape, w.dtype, causal, w.sigma, w.seed, heads=heads, fmt=fmt)
        _log(f"fp8 {fmt} {name} causal={causal} heads {heads}: error/bound {ws:.3f}, mean |err| {mean:.2e}, "
             f"LSE err {le:.2e}, max |O - O(unquantized)| {orig:.2e}")


def test_fp8_deterministic(fa):
    shape, dtype = (1, 2, 500, 128), inputs.BF16
    qb, kb, vb = inputs.draw_qkv(shape, dtype, 1.0, 1200)
    q, k, v = (inputs.to_torch(x, dtype, torch.device("cuda:0")) for x in (qb, kb, vb))
    a = fa.forward_fp8(q, k, v, causal=True)
    b = fa.forward_fp8(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
