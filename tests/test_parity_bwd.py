"""GPU parity of the backward pass: the HIP kernels behind flash_attn_bwd against
the float64 backward oracle.

Every case draws seeded q, k, v and dO (exact_attention_flash_amd.inputs), runs
the GPU forward to get O and LSE (as training would), then the GPU backward, and
compares dQ, dK and dV element by element with oracle.backward on the same bytes.

Bound per element (the pages fix no tolerance for the backward; this follows the
arithmetic of the kernels, with a factor 4 of slack): the kernels use fp32 for
everything except the 16-bit MFMA operands P and dS (unit roundoff u: 2^-8 bf16,
2^-11 fp16), D is formed from the stored 16-bit O, and P carries the fp32 error
of the recomputed score and of the forward's LSE (ds). With |.| elementwise,

    |dV - dV*| <= 4 (u P + eta)^T |dO| + 1/2 ulp
    |dQ - dQ*| <= 4 scale (u |dS| + eta + P |dD| + P ds |dP - D|) |K| + 1/2 ulp
    |dK - dK*| <= 4 scale (u |dS| + eta + P |dD| + P ds |dP - D|)^T |Q| + 1/2 ulp

where |dD_i| = u_o sum_d |dO_id O_id| (O rounded once to the dtype), ds_ij = 2^-24 d
scale sum_d |q_id k_jd| + 4e-6, and 1/2 ulp is the output rounding at the oracle's
value. eta is the absolute error of rounding a value below the smallest normal
number (the standard model fl(x) = x (1 + delta) + eta with gradual underflow):
half the subnormal spacing, 2^-25 for fp16 and 2^-134 for bf16. It matters for fp16
when P or dS is tiny (large logits), where the 16-bit operand is a subnormal.
The float64 quantities come from the same widened inputs.
"""
import math
import sys

import numpy as np
import pytest

from exact_attention_flash_amd import inputs
from oracle.backward import attention_backward
from tests._parity import half_ulp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_flash_amd as fa_mod

    fa_mod._native.lib()
    return fa_mod


UNIT = {inputs.BF16: 2.0 ** -8, inputs.FP16: 2.0 ** -11}
UNDERFLOW = {inputs.BF16: 2.0 ** -134, inputs.FP16: 2.0 ** -25}


def _draw(shape, dtype, sigma, seed):
    qb, kb, vb = inputs.draw_qkv(shape, dtype, sigma, seed)
    dob, _, _ = inputs.draw_qkv(shape, dtype, 1.0, seed + 7)
    return qb, kb, vb, dob


def _run_gpu(fa, bits, dtype, causal, scale):
    dev = torch.device("cuda:0")
    q, k, v, do = (inputs.to_torch(x, dtype, dev) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    conv = lambda t: inputs.bits_to_f64(inputs.from_torch_bits(t), dtype)
    return conv(dq), conv(dk), conv(dv), conv(o)


def _bounds(q, k, v, do, o16, scale, causal, dtype, row_block=2048):
    """Per-element error bounds (see the module docstring) for one slice [N, d], over
    blocks of complete query rows (dQ's bound per block, dK's and dV's summed over
    the blocks) so that long slices need no N x N arrays."""
    u = UNIT[dtype]
    n, d = q.shape
    eta = UNDERFLOW[dtype]
    dd = u * np.sum(np.abs(do * o16), axis=1)                       # D from the rounded O
    b_dq = np.zeros((n, d))
    b_dk = np.zeros((n, d))
    b_dv = np.zeros((n, d))
    keys = np.arange(n)
    for r0 in range(0, n, row_block):
        rows = np.arange(r0, min(n, r0 + row_block))
        s = scale * (q[rows] @ k.T)
        if causal:
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = do[rows] @ v.T
        dlt = (dp * p).sum(axis=1)
        ds = p * (dp - dlt[:, None])
        dsc = 2.0 ** -24 * d * scale * (np.abs(q[rows]) @ np.abs(k).T) + 4e-6  # score and LSE error
        err_ds = u * np.abs(ds) + eta + p * dd[rows, None] + p * dsc * np.abs(dp - dlt[:, None])
        b_dv += 4 * ((u * p + eta).T @ np.abs(do[rows]))
        b_dq[rows] = 4 * scale * (err_ds @ np.abs(k))
        b_dk += 4 * scale * (err_ds.T @ np.abs(q[rows]))
    return b_dq, b_dk, b_dv


def _check(name, got, ref, bound, dtype):
    tol = bound + half_ulp(ref, dtype) + 1e-30
    ratio = np.abs(got - ref) / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert worst <= 1.0, f"{name}: error reaches {worst:.3f} of its bound"
    return worst


def _compare(fa, shape, dtype, causal, sigma, seed, scale=None, heads=None):
    d = shape[-1]
    scale = float(np.float32(1.0 / math.sqrt(d))) if scale is None else scale
    bits = _draw(shape, dtype, sigma, seed)
    gq, gk, gv, go = _run_gpu(fa, bits, dtype, causal, scale)
    bh = shape[0] * shape[1]
    n = shape[2]
    flat = lambda x: x.reshape(bh, n, d)
    q, k, v, do = (flat(inputs.bits_to_f64(x, dtype)) for x in bits)
    gq, gk, gv, go = (flat(x) for x in (gq, gk, gv, go))
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for hh in (range(bh) if heads is None else heads):
        rq, rk, rv, _ = attention_backward(q[hh], k[hh], v[hh], do[hh], scale, causal=causal)
        b_dq, b_dk, b_dv = _bounds(q[hh], k[hh], v[hh], do[hh], go[hh], scale, causal, dtype)
        worst["dq"] = max(worst["dq"], _check(f"dq head {hh}", gq[hh], rq, b_dq, dtype))
        worst["dk"] = max(worst["dk"], _check(f"dk head {hh}", gk[hh], rk, b_dk, dtype))
        worst["dv"] = max(worst["dv"], _check(f"dv head {hh}", gv[hh], rv, b_dv, dtype))
    return worst


SMALL_SHAPES = [(1, 1, 1, 64), (1, 1, 3, 128), (1, 2, 63, 64), (1, 1, 64, 128), (2, 3, 130, 64),
                (1, 2, 200, 128), (1, 1, 257, 128), (2, 2, 384, 64), (1, 1, 511, 128), (1, 2, 700, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_shapes(fa, shape, dtype, causal):
    w = _compare(fa, shape, dtype, causal, 1.0, 31)
    _log(f"bwd {shape} {dtype} causal={causal}: error / bound {w}")


@pytest.mark.parametrize("name,causal,heads", [
    ("llama7b_b2_h32_n4096_d128_causal", True, [0, 37, 63]),
    ("mha_b4_h16_n1024_d64", False, [0, 21, 63]),
    ("mha_b4_h16_n1024_d64", True, [5, 63]),
    ("stress_b3_h8_n4099_d128_sigma8", False, [0, 23]),
    ("stress_b3_h8_n4099_d128_sigma8", True, [0, 23]),
])
def test_workload_heads(fa, name, causal, heads):
    """The workloads at full size and launch shape; complete gradients of sampled heads."""
    w = inputs.WORKLOADS[name]
    res = _compare(fa, w.shape, w.dtype, causal, w.sigma, w.seed, heads=heads)
    _log(f"bwd {name} causal={causal} heads {heads}: error / bound {res}")


def test_long_context_invariants(fa):
    """B1 H32 N16384 d128 causal bf16: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    (exact identities of the backward) on every head, within the summed bounds'
    order of magnitude (4 u per term); and one complete head against the oracle
    element by element, with the bounds of the module docstring."""
    w = inputs.WORKLOADS["longctx_b1_h32_n16384_d128_causal"]
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    bits = _draw(w.shape, w.dtype, w.sigma, w.seed)
    gq, gk, gv, go = _run_gpu(fa, bits, w.dtype, True, scale)
    hh = 17
    sl = [inputs.bits_to_f64(x, w.dtype).reshape(w.H, w.N, w.d)[hh] for x in bits]
    rq, rk, rv, _ = attention_backward(*sl, scale, causal=True)
    flat = lambda x: x.reshape(w.H, w.N, w.d)[hh]
    b_dq, b_dk, b_dv = _bounds(*sl, flat(go), scale, True, w.dtype)
    res = {n: _check(f"{n} head {hh}", flat(g), r, b, w.dtype)
           for n, g, r, b in (("dq", gq, rq, b_dq), ("dk", gk, rk, b_dk), ("dv", gv, rv, b_dv))}
    _log(f"bwd longctx head {hh} vs oracle: error / bound {res}")
    do = inputs.bits_to_f64(bits[3], w.dtype)
    u = UNIT[w.dtype]
    col_dk = gk.sum(axis=-2)
    col_dv = gv.sum(axis=-2)
    ref_dv = do.sum(axis=-2)
    scale_dk = np.abs(gk).sum(axis=-2)
    scale_dv = np.abs(do).sum(axis=-2)
    assert np.all(np.isfinite(gq)) and np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
    assert np.all(np.abs(col_dk) <= 4 * u * scale_dk + 1e-6)
    assert np.all(np.abs(col_dv - ref_dv) <= 4 * u * scale_dv + 1e-6)


def test_single_key_closed_form(fa):
    """N = 1: P = 1, so dV = dO exactly (P rounds to 1), and dQ, dK vanish up to the
    rounding of dP - D (within the bounds)."""
    shape, dtype = (2, 3, 1, 64), inputs.BF16
    bits = _draw(shape, dtype, 1.0, 5)
    _, _, gv, _ = _run_gpu(fa, bits, dtype, False, 0.125)
    np.testing.assert_array_equal(gv, inputs.bits_to_f64(bits[3], dtype))
    _compare(fa, shape, dtype, False, 1.0, 5, scale=0.125)


@pytest.mark.parametrize("causal", [False, True])
def test_large_logits(fa, causal):
    """Scores in the thousands (fp16, sigma 8, scale 2): finite gradients within the bounds."""
    _compare(fa, (1, 2, 190, 64), inputs.FP16, causal, 8.0, 91, scale=2.0)


def test_deterministic(fa):
    """No atomics: two runs give bitwise identical gradients."""
    shape, dtype = (1, 4, 333, 128), inputs.BF16
    bits = _draw(shape, dtype, 1.0, 8)
    a = _run_gpu(fa, bits, dtype, True, 0.088)
    b = _run_gpu(fa, bits, dtype, True, 0.088)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
