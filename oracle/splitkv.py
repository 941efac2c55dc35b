"""Attention over a key range, and the merge of such partials, in float64 --
TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

This module imports neither ``dense`` nor ``tiled``; tests compare them.

Source: [IO] "FlashAttention: IO-Aware Tiling, Online Softmax Mathematics,
Memory Hierarchy Dynamics, and Kernel Evolution", section "Online Softmax
Mathematics". A score row cut into two contiguous blocks has per-block maxima
m1, m2 and denominators l1 = sum exp(x1 - m1), l2 = sum exp(x2 - m2); the whole
row has

    m = max(m1, m2),    l = exp(m1 - m) l1 + exp(m2 - m) l2,

and, under "Dynamic Accumulation of Attention Output", the output of the whole
row follows from block 1's output O1 (normalised with its own l1) and block 2's
unnormalised product P2 V2 (P2 = exp(x2 - m2)):

    O = (l1 exp(m1 - m) / l) O1 + (exp(m2 - m) / l) P2 V2.

``partial`` computes one block's (O_k, m_k, l_k) for the keys of a range;
``merge`` folds a list of blocks into the row result two at a time with the
rule above (block 2's product P2 V2 is l2 O2). A block can hold no visible key
for a row (a causal row that ends before the range starts): then m_k = -inf,
l_k = 0 and O_k = 0, and the rule gives it weight exp(-inf) = 0. The log-sum-exp
of the row is m + ln l (same page, "Backward Pass Recomputation").
"""
from __future__ import annotations

import numpy as np


def partial(q, k, v, scale, k_begin, k_end, causal=False):
    """Attention of every query over keys [k_begin, k_end) only, float64.

    q, k, v: [..., N, d] (one shape). Causal: query i also drops keys j > i.
    Returns (o, m, l): o [..., N, d] normalised by the block's own l; m, l [..., N]
    the block's row maximum of the scaled scores and sum of exp(s - m). Rows with
    no visible key get o = 0, m = -inf, l = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    n = q.shape[-2]
    if not (0 <= k_begin <= k_end <= n):
        raise ValueError("key range must satisfy 0 <= k_begin <= k_end <= N")
    kb, vb = k[..., k_begin:k_end, :], v[..., k_begin:k_end, :]
    s = float(scale) * (q @ np.swapaxes(kb, -1, -2))             # [..., N, R]
    keys = np.arange(k_begin, k_end)
    if causal:
        s = np.where(keys[None, :] > np.arange(n)[:, None], -np.inf, s)
    m = s.max(axis=-1, initial=-np.inf)
    live = np.isfinite(m)
    shift = np.where(live, m, 0.0)
    e = np.exp(s - shift[..., None])                              # exp(-inf) = 0 for dropped keys
    l = e.sum(axis=-1)
    pv = e @ vb
    o = np.where(live[..., None], pv / np.where(live, l, 1.0)[..., None], 0.0)
    return o, m, l


def merge(parts):
    """Fold block results [(o, m, l), ...] into (O, LSE) with the two-block rule."""
    if not parts:
        raise ValueError("need at least one block")
    o, m, l = (np.array(x, dtype=np.float64) for x in parts[0])
    for o2, m2, l2 in parts[1:]:
        o2, m2, l2 = (np.asarray(x, dtype=np.float64) for x in (o2, m2, l2))
        mm = np.maximum(m, m2)
        fin = np.isfinite(mm)
        ref = np.where(fin, mm, 0.0)
        a1 = np.where(np.isfinite(m), np.exp(m - ref), 0.0)       # exp(m1 - m), 0 for an empty block
        a2 = np.where(np.isfinite(m2), np.exp(m2 - ref), 0.0)
        ll = a1 * l + a2 * l2
        safe = np.where(ll > 0, ll, 1.0)
        o = np.where((ll > 0)[..., None],
                     (l * a1 / safe)[..., None] * o + (a2 / safe)[..., None] * (l2[..., None] * o2), 0.0)
        m, l = mm, ll
    with np.errstate(divide="ignore"):
        lse = m + np.log(l)
    return o, lse
