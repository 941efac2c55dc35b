"""Pins for the tiled online-softmax checker (CPU only).

The checker follows the (m, l, u) recurrence of the tokenlab note, section 02.
It is pinned by that note's worked example (the printed value and the facts the
page states in words about each step), by its exact agreement with the dense
definition for every tile size and visiting order ("6.1 FlashAttention V1 in
detail", §3.3: the rescaling identity makes the tiled form exact up to rounding),
and by the page's warning that padded key columns must be masked.
"""
import math

import numpy as np
import pytest

from oracle.dense import attention
from oracle.tiled import attention_tiled
from tests import _golden

RNG = np.random.default_rng(777)


def _example():
    g = _golden.worked_example()
    n = len(g["scores"])
    q = np.ones((n, 1))
    k = np.array(g["scores"]).reshape(n, 1)
    v = np.array(g["values"]).reshape(n, 1)
    return g, q, k, v


@pytest.mark.parametrize("order", ["forward", "reverse"])
def test_worked_example_both_orders(order):
    g, q, k, v = _example()
    bc = int(g["tile_sizes"][0])          # tiles [2, 1] | [0]
    o, lse = attention_tiled(q, k, v, 1.0, br=1, bc=bc, order=order)
    dec = int(g["printed_decimals"])
    assert np.all(np.round(o[:, 0], dec) == g["u_over_l"])
    assert np.allclose(lse, math.log(math.exp(2) + math.exp(1) + 1), atol=1e-14)


def test_worked_example_forward_steps():
    """Forward order: the second tile has a smaller max, m stays 2, l += e^-2, u += 5e^-2."""
    g, q, k, v = _example()
    trace = []
    attention_tiled(q, k, v, 1.0, br=3, bc=2, order="forward", trace=trace)
    # one query tile holding the (identical) rows, two key tiles
    first, second = trace[0], trace[1]
    assert first["m"][0] == 2.0
    assert second["m"][0] == 2.0
    assert abs(second["l"][0] - first["l"][0] - math.exp(-2)) < 1e-15
    assert abs(second["u"][0, 0] - first["u"][0, 0] - 5 * math.exp(-2)) < 1e-15


def test_worked_example_reverse_steps():
    """Reversed order: m rises from 0 to 2, so old l and u are scaled by e^-2 first."""
    g, q, k, v = _example()
    trace = []
    attention_tiled(q, k, v, 1.0, br=3, bc=2, order="reverse", trace=trace)
    first, second = trace[0], trace[1]
    assert first["m"][0] == 0.0 and first["l"][0] == 1.0 and first["u"][0, 0] == 5.0
    assert second["m"][0] == 2.0
    new_l = math.exp(0.0) + math.exp(-1.0)          # tile [2, 1] relative to m = 2
    new_u = 1.0 * math.exp(0.0) + 3.0 * math.exp(-1.0)
    assert abs(second["l"][0] - (math.exp(-2) * 1.0 + new_l)) < 1e-15
    assert abs(second["u"][0, 0] - (math.exp(-2) * 5.0 + new_u)) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,br,bc", [(1, 1, 1), (3, 2, 2), (37, 8, 5), (64, 16, 64), (65, 64, 16), (100, 7, 33)])
@pytest.mark.parametrize("order", ["forward", "reverse", "shuffle"])
def test_tiled_equals_dense(n, br, bc, causal, order):
    d = 6
    q, k, v = (RNG.standard_normal((2, n, d)) for _ in range(3))
    tc = -(-n // bc)
    ordr = RNG.permutation(tc).tolist() if order == "shuffle" else order
    o_t, l_t = attention_tiled(q, k, v, 0.4, causal=causal, br=br, bc=bc, order=ordr)
    o_d, l_d = attention(q, k, v, 0.4, causal=causal)
    assert np.allclose(o_t, o_d, atol=1e-12, rtol=0)
    assert np.allclose(l_t, l_d, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_extreme_logits(causal):
    n, d = 45, 8
    q, k, v = (RNG.standard_normal((n, d)) * 8.0 for _ in range(3))
    scale = 50.0        # logits of order 1e4
    o_t, l_t = attention_tiled(q, k, v, scale, causal=causal, br=16, bc=8, order="reverse")
    o_d, l_d = attention(q, k, v, scale, causal=causal)
    assert np.all(np.isfinite(o_t)) and np.all(np.isfinite(l_t))
    assert np.allclose(o_t, o_d, atol=1e-12)
    assert np.allclose(l_t, l_d, rtol=1e-14, atol=1e-9)


def test_unmasked_padding_pollutes_the_denominator():
    """Padded key columns left at score 0 change the result (V1 guide §8.3, takeaway 3)."""
    n, d = 10, 4
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    good, lse_good = attention_tiled(q, k, v, 0.5, br=4, bc=4)
    bad, lse_bad = attention_tiled(q, k, v, 0.5, br=4, bc=4, mask_padding=False)
    o_d, l_d = attention(q, k, v, 0.5)
    assert np.allclose(good, o_d, atol=1e-12) and np.allclose(lse_good, l_d, atol=1e-12)
    # 10 keys in tiles of 4 leave 2 fake zero-score keys with zero values
    assert np.all(lse_bad > lse_good + 1e-6)
    assert np.max(np.abs(bad - good)) > 1e-3
    # an exact multiple of the tile has no padding, so the flag changes nothing
    q8, k8, v8 = q[:8], k[:8], v[:8]
    a, _ = attention_tiled(q8, k8, v8, 0.5, br=4, bc=4, mask_padding=False)
    b, _ = attention_tiled(q8, k8, v8, 0.5, br=4, bc=4)
    assert np.array_equal(a, b)


def test_bad_order_rejected():
    q = np.zeros((5, 2))
    with pytest.raises(ValueError):
        attention_tiled(q, q, q, 1.0, bc=2, order=[0, 0, 1])
