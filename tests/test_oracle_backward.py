"""Pins for the float64 backward oracle (CPU only).

Each test checks oracle.backward against something other than its own formulas:
central finite differences of the forward oracle (a separate module), torch's CPU
float64 autograd, the tokenlab worked example with the textbook softmax
derivative, and invariants every exact attention gradient satisfies. A dropped
D term, a missing or doubled scale, a transposed dS, an unmasked causal pair or a
swapped dK/dQ each fail at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle.backward import attention_backward
from oracle.dense import attention
from tests import _golden

RNG = np.random.default_rng(2024)


def _rand(*shape, sigma=1.0):
    return RNG.standard_normal(shape) * sigma


def _loss(q, k, v, do, scale, causal):
    o, _ = attention(q, k, v, scale, causal=causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    """Central differences of sum(dO * O) through the forward oracle."""
    n, d, scale = 5, 3, 0.7
    q, k, v, do = (_rand(n, d) for _ in range(4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, causal=causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(q, k, v, do, scale, causal)
            x[idx] = keep - h
            dn = _loss(q, k, v, do, scale, causal)
            x[idx] = keep
            num[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 17, 8), (1, 1, 64, 16), (1, 2, 130, 32)])
def test_matches_torch_autograd(shape, causal):
    """torch CPU float64 autograd of softmax(scale QK^T) V (a library routine)."""
    scale = 1.0 / math.sqrt(shape[-1])
    q, k, v, do = (_rand(*shape) for _ in range(4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale, causal=causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_worked_example_gradients():
    """Tokenlab worked example (scores [2, 1, 0], values [1, 3, 5], d = 1, scale 1) with dO = 1.

    The textbook derivative of O = sum_j p_j v_j with p = softmax(s) is
    dO/dv_j = p_j and dO/ds_j = p_j (v_j - O); with q = 1 and k_j = s_j this gives
    dV, and dQ = sum_j (dO/ds_j) k_j, dK_j = (dO/ds_j) q.
    """
    g = _golden.worked_example()
    s = np.array(g["scores"], dtype=np.float64)
    vals = np.array(g["values"], dtype=np.float64)
    n = s.size
    p = np.array([math.exp(x) for x in s]) / math.fsum(math.exp(x) for x in s)
    o = math.fsum(p * vals)
    assert round(o, int(g["printed_decimals"])) == pytest.approx(float(g["u_over_l"]))
    q = np.ones((n, 1))
    k = s.reshape(n, 1)
    v = vals.reshape(n, 1)
    do = np.ones((n, 1))
    dq, dk, dv, delta = attention_backward(q, k, v, do, 1.0)
    dsj = p * (vals - o)
    np.testing.assert_allclose(dv[:, 0], n * p, rtol=1e-14)        # every row has the same p
    np.testing.assert_allclose(dq[:, 0], math.fsum(dsj * s), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dk[:, 0], n * dsj, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(delta, o, rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Exact identities: D = rowsum(dO ∘ O); sum_j dK_j = 0; sum_j dV_j = sum_i dO_i
    (rows of P sum to 1); dQ does not change when every key moves by one vector
    (rows of dS sum to 0); dO = 0 gives zero gradients."""
    n, d, scale = 37, 6, 0.5
    q, k, v, do = (_rand(2, n, d) for _ in range(4))
    dq, dk, dv, delta = attention_backward(q, k, v, do, scale, causal=causal)
    o, _ = attention(q, k, v, scale, causal=causal)
    np.testing.assert_allclose(delta, np.sum(do * o, axis=-1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=-2), do.sum(axis=-2), rtol=1e-12, atol=1e-12)
    shift = _rand(1, 1, d)
    dq2, _, _, _ = attention_backward(q, k + shift, v, do, scale, causal=causal)
    np.testing.assert_allclose(dq2, dq, rtol=1e-10, atol=1e-12)
    z = attention_backward(q, k, v, np.zeros_like(do), scale, causal=causal)
    for t in z[:3]:
        assert np.all(t == 0.0)


def test_single_key_and_causal_first_row():
    """One key: P = 1, so dV = dO and dQ = dK = 0. Causal row 0 sees only key 0 and
    contributes nothing to dQ_0 (dS_00 = 0)."""
    q, k, v, do = (_rand(1, 4) for _ in range(4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, 0.9)
    np.testing.assert_allclose(dv, do, rtol=1e-15)
    assert np.all(np.abs(dq) < 1e-15) and np.all(np.abs(dk) < 1e-15)
    q, k, v, do = (_rand(9, 4) for _ in range(4))
    dq, _, _, _ = attention_backward(q, k, v, do, 0.9, causal=True)
    assert np.all(np.abs(dq[0]) < 1e-15)


def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        attention_backward(np.zeros((3, 4)), np.zeros((3, 4)), np.zeros((3, 4)), np.zeros((2, 4)), 1.0)
