"""Dense exact attention in float64: the definition the GPU path must reproduce.

TEST INFRASTRUCTURE ONLY (see the package header): never called by the product.

Definition followed, for every (batch, head) slice and query row i:

1. scores  s_ij = scale * sum_k q_ik k_jk  -- "6.1 FlashAttention V1 in detail",
   §1.1 (S = QK^T / sqrt(d)); the FlashAttention IO-aware survey, section
   "Standard Multi-Head Attention Execution Flow". ``scale`` is an argument; the
   caller passes the float32 value that the GPU receives, widened to float64.
   With ``causal`` the pairs j > i are dropped (query i attends keys j <= i,
   top-left aligned, one shared length N for queries and keys).
2. three-pass safe softmax over the full row -- V1 guide §3.1:
   pass 1 m_i = max_j s_ij; pass 2 l_i = sum_j exp(s_ij - m_i);
   pass 3 p_ij = exp(s_ij - m_i) / l_i.
3. output O_i = sum_j p_ij v_j -- V1 guide §1.1 (O = PV).
4. log-sum-exp L_i = m_i + ln l_i -- IO-aware survey, section "Backward Pass
   Recomputation" (the forward stores O and L = m + log(l)); natural log.

Rows are processed in blocks only to bound memory; each row's softmax is taken
over its complete row, so blocking does not change the arithmetic. The two
contractions use numpy's float64 matmul.
"""
from __future__ import annotations

import numpy as np


def attention(q, k, v, scale, causal=False, rows=None, row_block=512):
    """Exact softmax attention and its row log-sum-exp, in float64.

    q, k, v: arrays of shape [..., N, d] (leading dims are batch/head slices,
    the same for all three); converted to float64.
    scale: the logit multiplier (a float; use the float32 value the GPU gets).
    causal: if true, query i sees keys 0..i only.
    rows: optional 1-D array of query indices to evaluate (all if None);
    every row is computed independently, so a subset is exact.

    Returns (O, LSE) with shapes [..., R, d] and [..., R], R = len(rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [..., N, d]")
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise ValueError("row index out of range")
    g = int(np.prod(lead)) if lead else 1
    qf = q.reshape(g, n, d)
    kf = k.reshape(g, n, d)
    vf = v.reshape(g, n, d)
    out = np.empty((g, rows.size, d), dtype=np.float64)
    lse = np.empty((g, rows.size), dtype=np.float64)
    sigma = float(scale)
    keys = np.arange(n)
    for gi in range(g):
        kt = kf[gi].T
        for r0 in range(0, rows.size, row_block):
            rb = rows[r0:r0 + row_block]
            s = sigma * (qf[gi, rb] @ kt)  # [R, N]
            if causal:
                s = np.where(keys[None, :] > rb[:, None], -np.inf, s)
            m = s.max(axis=1)                       # pass 1
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)                       # pass 2
            p = e / l[:, None]                      # pass 3
            out[gi, r0:r0 + rb.size] = p @ vf[gi]
            lse[gi, r0:r0 + rb.size] = m + np.log(l)
    return out.reshape(lead + (rows.size, d)), lse.reshape(lead + (rows.size,))
