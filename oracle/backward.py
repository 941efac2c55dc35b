"""Dense backward pass of exact attention in float64 -- TEST INFRASTRUCTURE ONLY.

Nothing on the product path may import or call this module (see the package
header). It does not import ``dense`` or ``tiled``: the forward quantities it
needs (P, and O for the row statistic D) are formed here from the definition.

Definitions followed, per (batch, head) slice, with S = scale * Q K^T (causal:
pairs j > i dropped) and P = softmax(S) row-wise:

* [V1] §6.1 ("Backward challenge") and [IO] "Backward Pass Recomputation":
      dV = P^T dO,   dP = dO V^T,   dS = P ∘ (dP - rowsum(dP ∘ P) 1^T).
  [V1] §6.1 names D_i = rowsum(dP ∘ P)_i and states the identity
  D_i = rowsum(dO ∘ O)_i; the oracle uses the first form (the definition) and
  returns D so that tests can check the identity.
* [IO] "Backward Pass Recomputation": dQ = dS K / sqrt(d) and dK = dS^T Q / sqrt(d).
  That page writes the 1/sqrt(d) of S = QK^T/sqrt(d); with a general logit
  multiplier ``scale`` the chain rule through S = scale * Q K^T gives
  dQ = scale * dS K and dK = scale * dS^T Q.

Rows are processed in blocks only to bound memory; each block's softmax is taken
over complete rows and dK, dV accumulate the blocks' contributions, so blocking
does not change the arithmetic (float64 sums in a different order).
"""
from __future__ import annotations

import numpy as np


def attention_backward(q, k, v, dout, scale, causal=False, row_block=512):
    """Gradients of L = sum(dout * O) with O = softmax(scale Q K^T) V, in float64.

    q, k, v, dout: arrays of shape [..., N, d] (same shape); converted to float64.
    scale: the logit multiplier (use the float32 value the GPU receives).
    causal: if true, query i sees keys 0..i only (top-left aligned).

    Returns (dq, dk, dv, delta) with shapes [..., N, d] x3 and [..., N], where
    delta_i = rowsum(dP ∘ P)_i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must share one shape [..., N, d]")
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    g = int(np.prod(lead)) if lead else 1
    qf, kf, vf, of = (x.reshape(g, n, d) for x in (q, k, v, dout))
    dq = np.zeros((g, n, d))
    dk = np.zeros((g, n, d))
    dv = np.zeros((g, n, d))
    delta = np.zeros((g, n))
    sigma = float(scale)
    keys = np.arange(n)
    for gi in range(g):
        for r0 in range(0, n, row_block):
            rows = np.arange(r0, min(n, r0 + row_block))
            s = sigma * (qf[gi, rows] @ kf[gi].T)            # [R, N]
            if causal:
                s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)              # P = softmax(S)
            dov = of[gi, rows]                                # dO rows [R, d]
            dv[gi] += p.T @ dov                               # dV = P^T dO
            dp = dov @ vf[gi].T                               # dP = dO V^T
            dlt = (dp * p).sum(axis=1)                        # D = rowsum(dP ∘ P)
            ds = p * (dp - dlt[:, None])                      # dS
            dq[gi, rows] = sigma * (ds @ kf[gi])              # dQ = scale dS K
            dk[gi] += sigma * (ds.T @ qf[gi, rows])           # dK = scale dS^T Q
            delta[gi, rows] = dlt
    shp = lead + (n, d)
    return dq.reshape(shp), dk.reshape(shp), dv.reshape(shp), delta.reshape(lead + (n,))
