"""Float64 attention oracle (test infrastructure only; see the package docstring).

What is computed, for each batch b and head h, on the exact values the
kernel receives (float32 as is, bf16 widened, MXFP8 dequantised):

  S = scale * Q K^T                      attention scores
  S[i, j] = -inf for j > i  (causal)     the diagonal mask, top-left aligned
  m_i   = max_j S[i, j]                  safe-softmax shift
  l_i   = sum_j exp(S[i, j] - m_i)       denominator
  O_i   = sum_j exp(S[i, j] - m_i) V_j / l_i
  LSE_i = m_i + ln(l_i)                  natural log of the scaled scores

Sources:
  * "Flash Attention 4 -- the algorithm and the two-MMA problem", section
    "The memory-bound trap, restated from the roofline" (O = softmax(QK^T
    scaled) V).
  * "Lecture 2 -- Online Softmax and Numerical Correctness", section "The
    classical safe softmax" (the shifted softmax and the LSE), and section
    "Causal masking just changes which blocks contribute" (S_ij = -inf for
    j > i).
  * For blockwise_f64: the same lecture's "Combining two blocks exactly" and
    the six-line per-block update in the lesson's section "Online softmax --
    three running states instead of one big matrix" (running max, scale,
    unnormalised P, running sum, O rescale, commit), with the exp2 fold of
    its section "The exp2 trick" and the lagging-max rule of "FlashAttention-4's
    Softmax Tricks", section "Conditional rescaling, and when it's exact"
    (keep the stale max while the max grows by at most tau in log2 units).
"""
from __future__ import annotations

import math

import numpy as np

_LOG2E = 1.0 / math.log(2.0)


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def causal_offset(causal, nq: int, nk: int):
    """None for no mask, else the offset c of the mask "key j is hidden from
    query i when j > i + c". True or "top_left": c = 0, the lecture's
    S_ij = -inf for j > i. "bottom_right": c = Nk - Nq, so the last query sees
    every key (the same mask when Nq = Nk)."""
    if causal is False or causal is None:
        return None
    if causal is True or causal == "top_left":
        return 0
    if causal == "bottom_right":
        return nk - nq
    raise ValueError(f"causal={causal!r}")


def _one_head(q, k, v, causal, scale, rows, nq):
    """Plain definition for one head. q: [R, d] at global query indices `rows`
    of nq. A row that sees no key (possible bottom-right with Nq > Nk) has no
    softmax; it gets O = 0 and LSE = -inf."""
    s = scale * (q @ k.T)                                   # [R, Nk]
    off = causal_offset(causal, nq, k.shape[0])
    if off is not None:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] > rows[:, None] + off, -np.inf, s)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.exp(s - m[:, None])
    den = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(empty[:, None], 0.0, (e @ v) / den[:, None])
        lse = np.where(empty, -np.inf, m + np.log(den))
    return o, lse


def attention_f64(q, k, v, causal=False, scale=None, chunk: int = 256):
    """O [B, H, Nq, dv] float64 and LSE [B, H, Nq] float64.

    causal: False, True / "top_left", or "bottom_right" (see causal_offset).

    q: [B, H, Nq, d], k: [B, H, Nk, d], v: [B, H, Nk, dv]; any real dtype.
    Query rows are processed in chunks only to bound memory; every row is a
    one-shot softmax over all of its keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    scale = _default_scale(d, scale)
    o = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, chunk):
                rows = np.arange(r0, min(Nq, r0 + chunk))
                o[b, h, rows], lse[b, h, rows] = _one_head(q[b, h, rows], k[b, h], v[b, h],
                                                           causal, scale, rows, Nq)
    return o, lse


def attention_rows_f64(q, k, v, b: int, h: int, rows, causal: bool = False, scale=None):
    """The plain definition for the query rows `rows` of head (b, h) only."""
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[-1]
    qq = np.asarray(q[b, h, rows], dtype=np.float64)
    kk = np.asarray(k[b, h], dtype=np.float64)
    vv = np.asarray(v[b, h], dtype=np.float64)
    return _one_head(qq, kk, vv, causal, _default_scale(d, scale), rows, q.shape[2])


def blockwise_f64(q, k, v, causal: bool = False, scale=None, block: int = 64,
                  tau: float = 0.0, group: int = 32, scores_log2=None):
    """The streaming recurrence over key blocks, in float64.

    Per key block, for each query row (notation of the lesson's update):
      S       = Q K_block^T in raw units; the exponent is taken in log2 units,
                x * scale_log2 with scale_log2 = scale * log2(e)
      m_new   = max(row_max, rowmax(S))
      acc     = (row_max - m_new) * scale_log2
      if acc >= -tau: m_new = row_max, factor = 1     (lagging max)
      else:           factor = 2^acc                   (commit, rescale)
      P       = 2^((S - m_new) * scale_log2)
      row_sum = row_sum * factor + rowsum(P)
      O       = O * factor + P V_block
      row_max = m_new
    At the end O / row_sum and LSE = ln2 * (row_max * scale_log2 + log2 row_sum).

    A row's first block always commits (its row_max starts at -inf). A block
    in which a row sees no key (every score masked) leaves that row's state
    unchanged.

    With `scores_log2` ([R, N] float array, log2 units) the function instead
    runs the rule on given scores with V = 0, which is what the rescale
    counts need.

    Returns (O, LSE, stats); stats["rows"] is the [rows, blocks] bool array
    of rescale events (commits with a finite old max), stats["groups"] the
    same OR-ed over each `group` consecutive rows.
    """
    if scores_log2 is not None:
        s2_all = np.asarray(scores_log2, dtype=np.float64)[None, None]
        B, H, Nq, Nk = s2_all.shape
        dv = 1
        vv_all = np.zeros((B, H, Nk, 1))
        scale_log2 = 1.0
    else:
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        vv_all = np.asarray(v, dtype=np.float64)
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        dv = vv_all.shape[-1]
        scale_log2 = _default_scale(d, scale) * _LOG2E
    nblk = -(-Nk // block)
    off = causal_offset(causal, Nq, Nk)
    o_out = np.empty((B, H, Nq, dv))
    lse_out = np.empty((B, H, Nq))
    events = np.zeros((B, H, Nq, nblk), dtype=bool)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            row_max = np.full(Nq, -np.inf)
            row_sum = np.zeros(Nq)
            acc_o = np.zeros((Nq, dv))
            for j in range(nblk):
                k0, k1 = j * block, min(Nk, (j + 1) * block)
                if scores_log2 is not None:
                    s = s2_all[b, h, :, k0:k1]
                else:
                    s = q[b, h] @ k[b, h, k0:k1].T              # raw units
                if off is not None:
                    cols = np.arange(k0, k1)
                    s = np.where(cols[None, :] > rows[:, None] + off, -np.inf, s)
                seen = np.isfinite(s).any(axis=1)
                m_new = np.maximum(row_max, s.max(axis=1))
                with np.errstate(invalid="ignore"):
                    acc = (row_max - m_new) * scale_log2
                keep = (acc >= -tau) | ~seen
                commit = ~keep
                events[b, h, :, j] = commit & np.isfinite(row_max)
                m_use = np.where(keep, row_max, m_new)
                factor = np.where(keep, 1.0, np.exp2(np.where(commit, acc, 0.0)))
                m_exp = np.where(np.isfinite(m_use), m_use, 0.0)
                p = np.exp2((s - m_exp[:, None]) * scale_log2)
                row_sum = row_sum * factor + p.sum(axis=1)
                acc_o = acc_o * factor[:, None] + p @ vv_all[b, h, k0:k1]
                row_max = m_use
            with np.errstate(divide="ignore", invalid="ignore"):
                empty = row_sum == 0                 # rows that saw no key
                o_out[b, h] = np.where(empty[:, None], 0.0, acc_o / row_sum[:, None])
                lse_out[b, h] = np.where(empty, -np.inf,
                                         math.log(2.0) * (row_max * scale_log2 + np.log2(row_sum)))
    ev = events.reshape(B * H * Nq, nblk)
    ng = (B * H * Nq) // group
    groups = ev[: ng * group].reshape(ng, group, nblk).any(axis=1)
    return o_out, lse_out, {"rows": ev, "groups": groups}
