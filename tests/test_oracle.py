"""Pins for the dense float64 oracle (CPU only).

Each test checks the oracle against something other than its own formula: the
worked example printed by the tokenlab note, closed forms, invariants of softmax
attention, an fsum evaluation of softmax written in a different algebraic form,
and torch's CPU float64 attention. Together they catch the plausible mistakes:
a dropped max-subtraction (extreme logits), a sign flip (two-key closed form), a
transposed operand or wrong axis (non-square shapes, torch comparison), an off-by-
one causal mask (causal row 0, torch causal), a missing or doubled scale (torch,
two-key form) and a wrong log base (Q = 0 closed form).
"""
import math

import numpy as np
import pytest
import torch

from oracle.dense import attention
from tests import _golden

RNG = np.random.default_rng(12345)


def _rand(*shape, sigma=1.0, rng=RNG):
    return rng.standard_normal(shape) * sigma


# --------------------------------------------------------------------------- worked example
def test_worked_example_value():
    """Tokenlab note, "Mechanism map & worked derivation": row [2,1,0], values [1,3,5]."""
    g = _golden.worked_example()
    scores = np.array(g["scores"])
    vals = np.array(g["values"])
    n = scores.size
    # d = 1, scale = 1: q = 1 and k_j = score_j give exactly the printed scores.
    q = np.ones((n, 1))
    k = scores.reshape(n, 1)
    v = vals.reshape(n, 1)
    o, lse = attention(q, k, v, 1.0, causal=False)
    dec = int(g["printed_decimals"])
    assert np.all(np.round(o[:, 0], dec) == g["u_over_l"])
    # the row's log-sum-exp is ln(e^2 + e + 1) by definition of the normaliser
    assert np.allclose(lse, math.log(math.exp(2) + math.exp(1) + 1.0), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_visible_values(causal):
    """Q = 0 makes every logit 0: O_i is the mean of visible V rows, LSE_i = ln(#visible)."""
    n, d = 37, 5
    q = np.zeros((n, d))
    k = _rand(n, d)
    v = _rand(n, d)
    o, lse = attention(q, k, v, 0.7, causal=causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.allclose(o[i], v[:cnt].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - math.log(cnt)) < 1e-13


def test_equal_keys_give_uniform_weights():
    n, d = 19, 7
    q = _rand(n, d)
    k = np.tile(_rand(1, d), (n, 1))
    v = _rand(n, d)
    scale = 0.3
    o, lse = attention(q, k, v, scale)
    for i in range(n):
        assert np.allclose(o[i], v.mean(axis=0), atol=1e-13)
        s = scale * float(q[i] @ k[0])
        assert abs(lse[i] - (s + math.log(n))) < 1e-12


def test_causal_first_row_sees_only_first_key():
    n, d = 11, 6
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = attention(q, k, v, 0.45, causal=True)
    assert np.array_equal(o[0], v[0])
    assert abs(lse[0] - 0.45 * float(q[0] @ k[0])) < 1e-14


def test_two_keys_logistic_form():
    """With two keys, softmax is the logistic function of the logit difference."""
    d = 3
    q = _rand(4, d)
    k = _rand(2, d)
    v = _rand(2, d)
    scale = 0.9
    # two keys, four queries: pad keys to N = 4 is not allowed (shared N), so use N = 2
    for i in range(4):
        qi = np.stack([q[i], q[i]])
        o, lse = attention(qi, k, v, scale)
        s0 = scale * float(q[i] @ k[0])
        s1 = scale * float(q[i] @ k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(o[0], w0 * v[0] + (1.0 - w0) * v[1], atol=1e-14)
        assert abs(lse[0] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-14


def test_constant_values_give_ones():
    """V = 1 everywhere: rows of P sum to 1, so O = 1."""
    for causal in (False, True):
        n, d = 29, 4
        o, _ = attention(_rand(n, d), _rand(n, d), np.ones((n, d)), 0.5, causal=causal)
        assert np.allclose(o, 1.0, atol=1e-14)


def test_probabilities_from_lse_sum_to_one():
    n, d = 33, 8
    q, k, v = _rand(n, d, sigma=2.0), _rand(n, d), _rand(n, d)
    scale = 0.35
    for causal in (False, True):
        _, lse = attention(q, k, v, scale, causal=causal)
        s = scale * np.einsum("id,jd->ij", q, k)
        for i in range(n):
            cnt = i + 1 if causal else n
            assert abs(math.fsum(np.exp(s[i, :cnt] - lse[i])) - 1.0) < 1e-13


def test_extreme_logits_pick_argmax_value():
    """Logits of size ~1e4: no overflow, O equals the V row of the largest logit."""
    n, d = 16, 8
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = attention(q, k, v, 1e4)
    s = 1e4 * (q @ k.T)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for i in range(n):
        j = int(np.argmax(s[i]))
        gap = np.sort(s[i])[-1] - np.sort(s[i])[-2]
        if gap > 50:
            assert np.allclose(o[i], v[j], atol=1e-12)
            assert abs(lse[i] - s[i, j]) < 1e-9 * abs(s[i, j]) + 1e-12


# --------------------------------------------------------------------------- invariants
def test_shift_invariance_through_extra_dimension():
    """An extra feature with q=1, k=c/scale adds c to every logit: O unchanged, LSE + c."""
    n, d = 21, 6
    scale = 0.25
    c = 3.0
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    q2 = np.concatenate([q, np.ones((n, 1))], axis=1)
    k2 = np.concatenate([k, np.full((n, 1), c / scale)], axis=1)
    v2 = np.concatenate([v, _rand(n, 1)], axis=1)
    for causal in (False, True):
        o, lse = attention(q, k, v, scale, causal=causal)
        o2, lse2 = attention(q2, k2, v2, scale, causal=causal)
        assert np.allclose(o2[:, :d], o, atol=1e-13)
        assert np.allclose(lse2, lse + c, atol=1e-12)


def test_permutation_equivariance_noncausal():
    n, d = 24, 5
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = attention(q, k, v, 0.6)
    pk = RNG.permutation(n)
    o2, lse2 = attention(q, k[pk], v[pk], 0.6)
    assert np.allclose(o2, o, atol=1e-13) and np.allclose(lse2, lse, atol=1e-13)
    pq = RNG.permutation(n)
    o3, lse3 = attention(q[pq], k, v, 0.6)
    assert np.allclose(o3, o[pq], atol=1e-13) and np.allclose(lse3, lse[pq], atol=1e-13)


def test_linear_in_values():
    n, d = 18, 4
    q, k, v1, v2 = _rand(n, d), _rand(n, d), _rand(n, d), _rand(n, d)
    for causal in (False, True):
        o1, _ = attention(q, k, v1, 0.5, causal=causal)
        o2, _ = attention(q, k, v2, 0.5, causal=causal)
        o12, _ = attention(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal=causal)
        assert np.allclose(o12, 2.0 * o1 - 3.0 * o2, atol=1e-12)


def test_causal_prefix_property():
    """Rows < M of a causal problem only see keys < M: they equal the size-M problem."""
    n, m, d = 50, 31, 6
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = attention(q, k, v, 0.4, causal=True)
    om, lsem = attention(q[:m], k[:m], v[:m], 0.4, causal=True)
    assert np.allclose(o[:m], om, atol=1e-14) and np.allclose(lse[:m], lsem, atol=1e-14)


def test_row_subset_matches_full():
    q, k, v = _rand(2, 3, 40, 8), _rand(2, 3, 40, 8), _rand(2, 3, 40, 8)
    rows = np.array([0, 7, 39, 13])
    for causal in (False, True):
        o, lse = attention(q, k, v, 0.3, causal=causal)
        os_, ls_ = attention(q, k, v, 0.3, causal=causal, rows=rows, row_block=3)
        assert np.allclose(os_, o[..., rows, :], atol=1e-14)
        assert np.allclose(ls_, lse[..., rows], atol=1e-14)


# --------------------------------------------------------------------------- independent evaluations
def _fsum_reference(q, k, v, scale, causal):
    """softmax_j = 1 / sum_k exp(s_k - s_j): a different algebraic form, exact sums."""
    n, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        vis = i + 1 if causal else n
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in range(vis)]
        w = [1.0 / math.fsum(math.exp(s[t] - s[j]) for t in range(vis)) for j in range(vis)]
        for c in range(d):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in range(vis))
        lse[i] = math.log(math.fsum(math.exp(x) for x in s))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("n,d,causal", [(1, 3, False), (5, 2, False), (8, 3, True), (7, 9, True), (3, 11, False)])
def test_small_cases_against_fsum(n, d, causal):
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    scale = 0.6
    o, lse = attention(q, k, v, scale, causal=causal)
    ro, rl = _fsum_reference(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    assert np.allclose(o, ro, atol=1e-13) and np.allclose(lse, rl, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 70, 16), (1, 2, 129, 64), (1, 1, 5, 128)])
def test_against_torch_cpu_float64(shape, causal):
    q, k, v = _rand(*shape), _rand(*shape), _rand(*shape, sigma=2.0)
    scale = 1.0 / math.sqrt(shape[-1])
    o, lse = attention(q, k, v, scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        n = shape[-2]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    tl = torch.logsumexp(s, dim=-1)
    assert np.allclose(o, to.numpy(), atol=1e-12)
    assert np.allclose(lse, tl.numpy(), atol=1e-12)


def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        attention(np.zeros((4, 3)), np.zeros((5, 3)), np.zeros((5, 3)), 1.0)
