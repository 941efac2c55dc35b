"""Pins for the key-split partials and their merge (CPU only).

oracle.splitkv is checked against things that do not re-type its rule: the
tokenlab worked example (printed u/l for the split [2, 1] | [0], in both orders),
the dense definition (merging the blocks of any key partition is exact up to
rounding, because the two-block rule is an identity), a brute-force fsum
evaluation, torch's CPU float64 attention, scipy's logsumexp of the blocks'
log-sum-exps, and the stated handling of a block with no visible key. A dropped
l1 weight, a wrong sign in exp(m_k - m), a swapped pair of blocks or a mask that
ignores the range offset each fail one of them.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.dense import attention
from oracle.splitkv import merge, partial
from tests import _golden

RNG = np.random.default_rng(4242)


def _blocks(n, cuts):
    edges = [0, *cuts, n]
    return list(zip(edges[:-1], edges[1:]))


def _split(q, k, v, scale, cuts, causal=False):
    n = q.shape[-2]
    return [partial(q, k, v, scale, b, e, causal=causal) for b, e in _blocks(n, cuts)]


@pytest.mark.parametrize("reverse", [False, True])
def test_worked_example(reverse):
    """Scores [2, 1, 0], values [1, 3, 5], blocks [2, 1] | [0]: u/l = 1.849579 (printed)."""
    g = _golden.worked_example()
    n = len(g["scores"])
    q = np.ones((n, 1))
    k = np.array(g["scores"]).reshape(n, 1)
    v = np.array(g["values"]).reshape(n, 1)
    parts = _split(q, k, v, 1.0, [int(g["tile_sizes"][0])])
    if reverse:
        parts = parts[::-1]
    o, lse = merge(parts)
    assert np.all(np.round(o[:, 0], int(g["printed_decimals"])) == g["u_over_l"])
    assert np.allclose(lse, math.log(math.exp(2) + math.exp(1) + 1), atol=1e-14)


def test_worked_example_block_statistics():
    """The page's per-block statistics: block [2, 1] has m1 = 2, l1 = 1 + e^-1;
    block [0] has m2 = 0, l2 = 1 and output 5."""
    g = _golden.worked_example()
    n = len(g["scores"])
    q = np.ones((n, 1))
    k = np.array(g["scores"]).reshape(n, 1)
    v = np.array(g["values"]).reshape(n, 1)
    (o1, m1, l1), (o2, m2, l2) = _split(q, k, v, 1.0, [2])
    assert np.all(m1 == 2.0) and np.allclose(l1, 1 + math.exp(-1), rtol=1e-15)
    assert np.allclose(o1[:, 0], (1 + 3 * math.exp(-1)) / (1 + math.exp(-1)), rtol=1e-15)
    assert np.all(m2 == 0.0) and np.all(l2 == 1.0) and np.all(o2[:, 0] == 5.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[], [1], [37], [64, 65], [10, 20, 90, 91], list(range(8, 100, 8))])
def test_any_partition_matches_dense(causal, cuts):
    n, d, scale = 100, 16, 0.3
    q, k, v = (RNG.standard_normal((2, n, d)) for _ in range(3))
    o, lse = merge(_split(q, k, v, scale, cuts, causal=causal))
    ro, rl = attention(q, k, v, scale, causal=causal)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_merge_order_does_not_matter():
    n, d, scale = 60, 8, 0.5
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    parts = _split(q, k, v, scale, [7, 30, 31, 50], causal=True)
    o1, l1 = merge(parts)
    for perm in ([4, 3, 2, 1, 0], [2, 0, 4, 1, 3]):
        o2, l2 = merge([parts[i] for i in perm])
        np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l2, l1, rtol=1e-14, atol=1e-14)


def test_lse_is_logsumexp_of_block_lses():
    """scipy's logsumexp over the blocks' m_k + ln l_k equals the merged LSE."""
    n, d, scale = 80, 12, 0.7
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    parts = _split(q, k, v, scale, [16, 40, 41], causal=True)
    with np.errstate(divide="ignore"):
        blk = np.stack([m + np.log(l) for _, m, l in parts])
    _, lse = merge(parts)
    np.testing.assert_allclose(lse, logsumexp(blk, axis=0), rtol=1e-14, atol=1e-14)


def test_empty_blocks():
    """Causal rows that end before a block starts see nothing in it: m = -inf,
    l = 0, o = 0, and merging such a block changes nothing."""
    n, d, scale = 20, 4, 1.0
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    o, m, l = partial(q, k, v, scale, 12, 20, causal=True)
    assert np.all(np.isneginf(m[:12])) and np.all(l[:12] == 0) and np.all(o[:12] == 0)
    assert np.all(np.isfinite(m[12:])) and np.all(l[12:] >= 1.0)
    head = partial(q, k, v, scale, 0, 12, causal=True)
    mo, ml = merge([head, (o, m, l)])
    ro, rl = attention(q, k, v, scale, causal=True)
    np.testing.assert_allclose(mo, ro, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ml, rl, rtol=1e-14, atol=1e-14)
    # an empty key range is empty for every row
    o0, m0, l0 = partial(q, k, v, scale, 5, 5)
    assert np.all(np.isneginf(m0)) and np.all(l0 == 0) and np.all(o0 == 0)
    po, pl = merge([(o0, m0, l0), head])
    ho, hl = merge([head])
    np.testing.assert_allclose(po, ho, rtol=4e-16, atol=4e-16)  # (1 / l) (l o) rounds once more
    np.testing.assert_array_equal(pl, hl)


@pytest.mark.parametrize("causal", [False, True])
def test_small_cases_against_fsum(causal):
    """Brute force: every output element as an fsum over exactly computed weights."""
    n, d, scale = 6, 3, 0.9
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    o, lse = merge(_split(q, k, v, scale, [2, 3], causal=causal))
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = [scale * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        den = math.fsum(w)
        assert abs(lse[i] - (mx + math.log(den))) < 1e-13
        for c in range(d):
            ref = math.fsum(wj * v[j, c] for wj, j in zip(w, keys)) / den
            assert abs(o[i, c] - ref) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_cpu_float64(causal):
    shape = (2, 3, 70, 16)
    q, k, v = (RNG.standard_normal(shape) for _ in range(3))
    o, _ = merge(_split(q, k, v, 0.25, [20, 21, 64], causal=causal))
    t = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)), is_causal=causal, scale=0.25)
    np.testing.assert_allclose(o, t.numpy(), rtol=1e-11, atol=1e-12)


def test_rejects_bad_ranges():
    x = np.zeros((4, 2))
    for b, e in ((-1, 2), (3, 2), (0, 5)):
        with pytest.raises(ValueError):
            partial(x, x, x, 1.0, b, e)
    with pytest.raises(ValueError):
        merge([])
