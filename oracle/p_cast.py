"""P cast to a narrow float type under the lagging max (test infrastructure
only; see the package docstring).

"FlashAttention-4's Softmax Tricks", section "Where 'exact' breaks: P in FP8":
the lagging max lets P = 2^(s - m_stale) reach 2^tau; the FP8 path further
multiplies P by 2^max_offset (max_offset = 8) before casting it to the MMA
type, so E4M3 (largest finite 448, about 2^8.81) saturates once tau > 0.81,
while the float32 denominator keeps the unclamped P and the output shrinks.
The page simulates this on 256 rows x 8192 keys with 128-key blocks and
reports the relative L2 error of O; `lagging_max_p_cast_f64` is that
simulation, written from the page's description:

  per 128-key block, per row, in log2 units of the scores s:
    m_new = max(m, rowmax(s)); keep the stale m while m - m_new >= -tau
    (else commit and rescale l and O by 2^(m - m_new))
    P     = 2^(s - m)                         float64
    l     = l * factor + rowsum(P)            from the uncast P
    O     = O * factor + cast(P * 2^max_offset) V / 2^max_offset
  O / l at the end.

`round_to_format` is the cast: round to nearest, ties to even, onto the
value grid of a binary floating-point format given by its fraction bits and
smallest normal exponent (subnormals below it keep that exponent's spacing),
saturating at the largest finite value.
"""
from __future__ import annotations

import numpy as np

# fraction bits, smallest normal exponent, largest finite value
FORMATS = {
    "bf16": (7, -126, float.fromhex("0x1.fep127")),
    "e4m3": (3, -6, 448.0),       # OCP E4M3 (e4m3fn: no infinities, 0x7F is NaN)
    "e5m2": (2, -14, 57344.0),    # OCP E5M2
}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Nearest value of format `fmt` (ties to even), saturated at its largest
    finite magnitude; float64 in and out."""
    mant, emin, vmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e2 = np.frexp(a)                     # a = f * 2^e2 with f in [0.5, 1)
    e = np.maximum(e2.astype(np.float64) - 1.0, emin)
    ulp = np.exp2(e - mant)
    r = np.round(a / ulp) * ulp             # np.round rounds half to even
    r = np.minimum(r, vmax)
    return np.copysign(r, x)


def lagging_max_p_cast_f64(scores_log2, v, *, block: int = 128, tau: float = 0.0,
                           fmt: str | None = None, max_offset: int = 0) -> np.ndarray:
    """O of the page's simulation for scores [R, N] (log2 units) and V [N, d].
    fmt=None leaves P uncast (the exact recurrence)."""
    s_all = np.asarray(scores_log2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, N = s_all.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, v.shape[1]))
    up = 2.0 ** max_offset
    for k0 in range(0, N, block):
        s = s_all[:, k0:k0 + block]
        m_new = np.maximum(m, s.max(axis=1))
        with np.errstate(invalid="ignore"):
            acc = m - m_new                      # -inf on the first block
        keep = acc >= -tau
        m_use = np.where(keep, m, m_new)
        factor = np.where(keep, 1.0, np.exp2(np.where(keep, 0.0, acc)))
        p = np.exp2(s - m_use[:, None])
        l = l * factor + p.sum(axis=1)
        pc = p if fmt is None else round_to_format(p * up, fmt) / up
        o = o * factor[:, None] + pc @ v[k0:k0 + block]
        m = m_use
    return o / l[:, None]


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
