"""Tiled online-softmax attention in float64: a checker for the dense oracle.

TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.
This module does not import ``oracle.dense``; the two are compared in tests.

It follows the running-state recurrence of "FlashAttention: optimize data
movement before counting FLOPs", section 02 (The mechanism): for each new key
tile with scores s and values V,

    m' = max(m, max s)
    l' = exp(m - m') l + sum_j exp(s_j - m')
    u' = exp(m - m') u + sum_j exp(s_j - m') V_j
    output = u' / l'

with m = -inf, l = 0, u = 0 at the start ("6.1 FlashAttention V1 in detail",
§5.2 and code takeaway 4 of §8.3: the first correction factor is exp(-inf) = 0).
Queries are cut into tiles of ``br`` rows and keys into tiles of ``bc`` rows
(V1 guide §4.1: Tr = ceil(N/Br), Tc = ceil(N/Bc)); the last tiles are zero-padded
and the padded key columns are set to -inf before the softmax (V1 guide §8.3,
code takeaway 3: otherwise fake zeros pollute the denominator). Padded query
rows are computed and never stored. The log-sum-exp is m + ln l (IO-aware survey,
"Backward Pass Recomputation").

Key tiles may be visited in any order (forward, reversed, or a given
permutation): the worked example of the tokenlab note walks both orders.

While iterating it asserts the stability facts of V1 guide §5.3: every exponent
argument is <= 0 and every correction factor is <= 1.
"""
from __future__ import annotations

import numpy as np


def _tile_order(tc, order):
    if order == "forward":
        return list(range(tc))
    if order == "reverse":
        return list(range(tc - 1, -1, -1))
    perm = [int(x) for x in order]
    if sorted(perm) != list(range(tc)):
        raise ValueError("order must be 'forward', 'reverse' or a permutation of the key tiles")
    return perm


def attention_tiled(q, k, v, scale, causal=False, br=64, bc=64, order="forward",
                    mask_padding=True, trace=None):
    """Online-softmax attention over (br x bc) tiles, float64.

    q, k, v: [..., N, d]. Returns (O, LSE) with shapes [..., N, d] and [..., N].
    mask_padding=False leaves padded key columns at score 0 instead of -inf;
    it exists only so a test can show that the mask is required.
    trace: optional list; for every (query tile, key tile) step a dict with the
    running m, l, u of that query tile is appended (used by worked-example tests).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    if br < 1 or bc < 1:
        raise ValueError("tile sizes must be positive")
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    g = int(np.prod(lead)) if lead else 1
    qf, kf, vf = (x.reshape(g, n, d) for x in (q, k, v))
    tr = -(-n // br)
    tc = -(-n // bc)
    visit = _tile_order(tc, order)
    sigma = float(scale)
    out = np.zeros((g, n, d))
    lse = np.zeros((g, n))

    for gi in range(g):
        for i in range(tr):
            r0 = i * br
            q_tile = np.zeros((br, d))
            q_tile[: min(br, n - r0)] = qf[gi, r0:r0 + br]
            q_idx = r0 + np.arange(br)
            m = np.full(br, -np.inf)
            l = np.zeros(br)
            u = np.zeros((br, d))
            for j in visit:
                c0 = j * bc
                k_tile = np.zeros((bc, d))
                v_tile = np.zeros((bc, d))
                k_tile[: min(bc, n - c0)] = kf[gi, c0:c0 + bc]
                v_tile[: min(bc, n - c0)] = vf[gi, c0:c0 + bc]
                k_idx = c0 + np.arange(bc)

                s = sigma * (q_tile @ k_tile.T)                   # [br, bc]
                if mask_padding:
                    s = np.where(k_idx[None, :] >= n, -np.inf, s)
                if causal:
                    s = np.where(k_idx[None, :] > q_idx[:, None], -np.inf, s)

                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)          # rows that have seen a key
                # correction exp(m - m'); a row with m = -inf gets 0, one whose
                # m' is still -inf keeps its (empty) state unchanged.
                ref = np.where(live, m_new, 0.0)
                alpha = np.where(live, np.exp(m - ref), 1.0)
                arg = np.where(np.isfinite(s), s - ref[:, None], -np.inf)
                assert np.all(alpha <= 1.0), "correction factor above 1"
                assert np.all(arg <= 0.0), "positive exponent argument"
                p = np.exp(arg)                                   # exp(-inf) = 0
                l = alpha * l + p.sum(axis=1)
                u = alpha[:, None] * u + p @ v_tile
                m = m_new
                if trace is not None:
                    trace.append({"q_tile": i, "k_tile": j, "m": m.copy(),
                                  "l": l.copy(), "u": u.copy()})
            rows = min(br, n - r0)
            out[gi, r0:r0 + rows] = (u / l[:, None])[:rows]
            lse[gi, r0:r0 + rows] = (m + np.log(l))[:rows]
    return out.reshape(lead + (n, d)), lse.reshape(lead + (n,))
