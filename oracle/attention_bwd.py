"""Float64 oracle of the attention backward pass (test infrastructure only;
see the package docstring).

What is computed: the gradients of a scalar loss L with dL/dO = dO through
O = softmax(S) V, S = scale * Q K^T (masked as in attention_f64), for each
batch b and head h:

  P     = softmax(S)                   rows that see no key: P = 0
  dV    = P^T dO
  dP    = dO V^T
  D_i   = sum_j P_ij dP_ij  (= sum_c dO_ic O_ic)
  dS    = P * (dP - D)                 the softmax Jacobian applied row by row
  dQ    = scale * dS K
  dK    = scale * dS^T Q

This is the closed form of the derivative (the five products the MXFP8 page
counts: S, dP, dV, dK, dQ), written out directly; nothing is blocked or
fused. Sources:
  * "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and backward
    for Blackwell", section "TMEM allocation and scale factor placement"
    (the backward pass has five GEMMs; dK and dV accumulate over the whole
    kernel) and section "Quantization along both axes and jagged tensors"
    (dP, dV, dK and dQ, and dS as the operand shared by dK and dQ).
  * "Lecture 2 -- Online Softmax and Numerical Correctness", section "Use
    it in the real stack" (the forward kernel also returns the per-row
    log-sum-exp, which is what makes the backward pass cheap): P is rebuilt
    here the same way, P = exp(S - LSE).
The masks and the empty-row convention are those of attention_f64.
"""
from __future__ import annotations

import numpy as np

from .attention import _default_scale, attention_f64, causal_offset


def _one_head_bwd(q, k, v, do, causal, scale):
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    off = causal_offset(causal, nq, nk)
    if off is not None:
        s = np.where(np.arange(nk)[None, :] > np.arange(nq)[:, None] + off, -np.inf, s)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    with np.errstate(divide="ignore", invalid="ignore"):     # rows without keys: log(0), then masked
        lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        p = np.where(empty[:, None], 0.0, np.exp(s - lse[:, None]))
    dv = p.T @ do
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, dd


def attention_bwd_f64(q, k, v, do, causal=False, scale=None):
    """dQ [B,H,Nq,d], dK [B,H,Nk,d], dV [B,H,Nk,dv] float64, and D [B,H,Nq].

    q: [B, H, Nq, d], k: [B, H, Nk, d], v: [B, H, Nk, dv], do: [B, H, Nq, dv];
    causal as for attention_f64."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, Nq, d = q.shape
    scale = _default_scale(d, scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dd = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], dd[b, h] = _one_head_bwd(q[b, h], k[b, h], v[b, h], do[b, h],
                                                                   causal, scale)
    return dq, dk, dv, dd


def attention_loss_f64(q, k, v, do, causal=False, scale=None):
    """L = sum(O * dO) through attention_f64: the scalar whose gradients
    attention_bwd_f64 returns (used by the finite-difference pins)."""
    o, _ = attention_f64(q, k, v, causal=causal, scale=scale)
    return float((o * np.asarray(do, dtype=np.float64)).sum())
