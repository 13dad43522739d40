"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, the bench and the smoke check. It holds
only input preparation: random draws, the bf16 round-to-nearest-even cast,
and the OCP e4m3 + E8M0 block quantiser that turns float samples into the
MXFP8 tensors the block-scaled path receives. It holds none of the
attention arithmetic, and it imports neither the oracle nor the HIP binding.

Layouts: Q, K, V are ``[B, H, N, d]`` C-order, d innermost. MX scales are
``[B, H, N/32, d/32]`` uint8 (one E8M0 byte per 32x32 block; V is blocked
along the sequence with the same square blocks, so one layout serves Q, K
and V). The pages that describe this format: "PyTorch FlashAttention-4 adds
MXFP8 block-scaled forward and backward for Blackwell", section
"Quantization along both axes and jagged tensors" (square 32x32 blocks,
E4M3 payload, E8M0 scales).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_inputs", "make_grad_output", "mx_quantize_packed", "mx_compact_offsets", "bf16_bits", "bf16_bits_to_f32",
    "e4m3_decode_table", "e4m3_encode", "e8m0_for_amax", "mx_quantize",
    "mx_dequantize", "make_score_inputs", "make_packed_inputs",
]


# --------------------------------------------------------------------------
# Workloads. Each is named by what it is; the seeds fix every draw.
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str            # "f32", "bf16" or "mxfp8"
    causal: tuple         # causal settings this workload is run with
    exp2_mode: str        # "hw", "emu" or "mix"
    tau: float
    seed: int
    spike_frac: float = 0.0   # fraction of K rows per (b, h) multiplied by spike_gain
    spike_gain: float = 1.0

    @property
    def flops_noncausal(self) -> float:
        return 4.0 * self.B * self.H * self.Nq * self.Nk * self.d


WORKLOADS = {
    w.name: w for w in [
        Workload("fp32_b1h1_n128_d64", 1, 1, 128, 128, 64, "f32", (False,), "emu", 8.0, 1001),
        Workload("bf16_b2h8_n1024_d128_causal", 2, 8, 1024, 1024, 128, "bf16", (True,), "hw", 8.0, 1002),
        Workload("bf16_b4h16_n4096_d128", 4, 16, 4096, 4096, 128, "bf16", (False, True), "mix", 8.0, 1003),
        Workload("bf16_b2h32_n8192_d64_causal_spiky", 2, 32, 8192, 8192, 64, "bf16", (True,), "mix", 8.0, 1004,
                 spike_frac=0.01, spike_gain=8.0),
        Workload("mxfp8_b2h16_n8192_d128", 2, 16, 8192, 8192, 128, "mxfp8", (False,), "mix", 8.0, 1005),
        # the larger head dims of the tuning-table rows ("The emulated exp2":
        # causal d = 192 is one of them), at the headline batch and length
        Workload("bf16_b4h16_n4096_d192", 4, 16, 4096, 4096, 192, "bf16", (False, True), "mix", 8.0, 1006),
        Workload("bf16_b4h16_n4096_d256", 4, 16, 4096, 4096, 256, "bf16", (False, True), "mix", 8.0, 1007),
        # one query row per head against a long key sequence (a decoding
        # step): too few query tiles to fill the GPU whole, the shape the
        # key-split launch is for
        Workload("bf16_b1h8_nq1_nk32768_d128", 1, 8, 1, 32768, 128, "bf16", (False,), "hw", 8.0, 1008),
    ]
}


# --------------------------------------------------------------------------
# bf16 (round to nearest, ties to even) on raw bits.
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even.

    NaN is not expected in synthetic inputs and is not treated specially.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# OCP e4m3 ("e4m3fn": bias 7, no infinities, 0x7F/0xFF NaN, max 448).
# --------------------------------------------------------------------------
def e4m3_decode_table() -> np.ndarray:
    """float64 value of every e4m3 byte (NaN for 0x7F and 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:0x7F]          # codes 0x00..0x7E, ascending, all finite


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to e4m3 bytes: nearest, ties to even code, saturate at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")        # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    return np.where(np.signbit(x) & (code != 0), code | np.uint8(0x80), code).astype(np.uint8)


def e8m0_for_amax(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte of the smallest power of two X with amax / X <= 448.

    Read off the float32 exponent and mantissa bits of amax: with
    amax = 1.f * 2^e, X = 2^(e-8) when 1.f <= 1.75, else 2^(e-7). An all-zero
    block gets X = 1 (byte 127); its codes are all zero whatever X is.
    """
    a = np.asarray(amax, dtype=np.float32)
    u = a.view(np.uint32)
    e = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64) - 127
    mant = u & np.uint32(0x7FFFFF)
    bump = (mant > np.uint32(0x600000)).astype(np.int64)      # 1.f > 1.75
    byte = e - 8 + bump + 127
    byte = np.where(a > 0, byte, 127)
    return np.clip(byte, 0, 254).astype(np.uint8)


def mx_quantize(x: np.ndarray):
    """[..., N, d] float -> (e4m3 bytes [..., N, d], E8M0 bytes [..., N/32, d/32])."""
    x = np.asarray(x, dtype=np.float32)
    *lead, n, d = x.shape
    assert n % 32 == 0 and d % 32 == 0, "MX blocks are 32x32"
    blk = x.reshape(*lead, n // 32, 32, d // 32, 32)
    amax = np.abs(blk).max(axis=(-3, -1))
    sbyte = e8m0_for_amax(amax)
    xs = np.ldexp(1.0, sbyte.astype(np.int64) - 127)          # float64 2^(byte-127)
    q = e4m3_encode(blk / xs[..., :, None, :, None])
    return q.reshape(x.shape), sbyte


def mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact float64 values of MX tensors (e4m3 times 2^(E8M0-127))."""
    *lead, n, d = q.shape
    v = _E4M3[q].reshape(*lead, n // 32, 32, d // 32, 32)
    xs = np.ldexp(1.0, s.astype(np.int64) - 127)
    return (v * xs[..., :, None, :, None]).reshape(q.shape)


# --------------------------------------------------------------------------
# The seeded draws.
# --------------------------------------------------------------------------
def make_inputs(w: Workload | str, *, B=None, H=None, Nq=None, Nk=None, seed=None):
    """Draw Q, K, V for a workload, optionally at reduced sizes.

    Returns a dict with the device-ready host arrays and the exact float64
    values the kernel receives:
      f32:   q, k, v float32                         ; q64, k64, v64
      bf16:  q, k, v uint16 bit patterns             ; q64, k64, v64
      mxfp8: q, k, v uint8 e4m3; qs, ks, vs uint8 E8M0 ; q64, k64, v64 (dequantised)
    Draw order: Q, K, V float32 standard normals (C order), then, if the
    workload has spikes, per (b, h) in C order round(spike_frac * Nk) key
    indices without replacement; those K rows are multiplied by spike_gain
    after the cast (a power of two, so exact in every dtype).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    Nq = w.Nq if Nq is None else Nq
    Nk = w.Nk if Nk is None else Nk
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal((B, H, Nq, w.d), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, w.d), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, w.d), dtype=np.float32)
    out = {"B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": w.d, "dtype": w.dtype}
    if w.dtype == "f32":
        tensors = {"q": q, "k": k, "v": v}
        vals = {n: t.astype(np.float64) for n, t in tensors.items()}
    elif w.dtype == "bf16":
        tensors = {n: bf16_bits(t) for n, t in (("q", q), ("k", k), ("v", v))}
        vals = {n: bf16_bits_to_f32(t).astype(np.float64) for n, t in tensors.items()}
    elif w.dtype == "mxfp8":
        tensors, vals = {}, {}
        for n, t in (("q", q), ("k", k), ("v", v)):
            qb, sb = mx_quantize(t)
            tensors[n], tensors[n + "s"] = qb, sb
            vals[n] = mx_dequantize(qb, sb)
    else:
        raise ValueError(w.dtype)
    if w.spike_frac > 0:
        nsp = int(round(w.spike_frac * Nk))
        for b in range(B):
            for h in range(H):
                idx = rng.choice(Nk, size=nsp, replace=False)
                _spike(tensors, vals, w.dtype, b, h, idx, w.spike_gain)
    out.update(tensors)
    out.update({n + "64": vals[n] for n in ("q", "k", "v")})
    return out


def _spike(tensors, vals, dtype, b, h, idx, gain):
    e = int(round(math.log2(gain)))
    assert 2.0 ** e == gain, "spike gain must be a power of two"
    vals["k"][b, h, idx] *= gain
    if dtype == "f32":
        tensors["k"][b, h, idx] *= np.float32(gain)
    elif dtype == "bf16":
        f = bf16_bits_to_f32(tensors["k"][b, h, idx]) * np.float32(gain)
        tensors["k"][b, h, idx] = bf16_bits(f)
    else:
        raise ValueError("spikes are defined for f32 and bf16 workloads")


def make_score_inputs(sigma: float, seed: int, rows: int = 256, keys: int = 8192, d: int = 128):
    """Scores and values for the P-cast study of "FlashAttention-4's Softmax
    Tricks" (section "Where 'exact' breaks: P in FP8"): 256 rows x 8192 keys of
    iid N(0, sigma^2) scores in log2 units, drawn first, then V [keys, d] iid
    N(0, 1), both float64 standard normals from default_rng(seed). The page
    gives the score distribution and the sizes; V's distribution and d are
    this recipe's choice."""
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((rows, keys)) * sigma
    v = rng.standard_normal((keys, d))
    return scores, v


def make_grad_output(shape, seed: int, dtype: str = "bf16"):
    """dO for the backward pass: float32 standard normals of `shape` from
    default_rng(seed), as bf16 bit patterns (dtype "bf16") or float32, with
    the exact float64 values the kernel receives."""
    g = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        bits = bf16_bits(g)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    return g, g.astype(np.float64)


def make_packed_inputs(w: Workload | str, q_lens, k_lens, H: int, seed: int):
    """A packed batch of sequences of different lengths in the workload's dtype:
    Q [total_q, H, d], K and V [total_k, H, d] token-major, drawn as float32
    standard normals in the order Q, K, V from default_rng(seed); cu_q / cu_k
    int32 [B+1] sequence starts. Also returns the exact float64 values
    (q64, k64, v64) the kernel receives. MXFP8 adds the compact scales qs, ks,
    vs [rows, H, d/32] (mx_quantize_packed) and their per-sequence first rows
    sq_off / sk_off (mx_compact_offsets)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((int(cu_q[-1]), H, w.d), dtype=np.float32)
    k = rng.standard_normal((int(cu_k[-1]), H, w.d), dtype=np.float32)
    v = rng.standard_normal((int(cu_k[-1]), H, w.d), dtype=np.float32)
    out = {"cu_q": cu_q, "cu_k": cu_k, "H": H, "d": w.d, "dtype": w.dtype}
    for n, t, cu in (("q", q, cu_q), ("k", k, cu_k), ("v", v, cu_k)):
        if w.dtype == "f32":
            out[n], out[n + "64"] = t, t.astype(np.float64)
        elif w.dtype == "bf16":
            bits = bf16_bits(t)
            out[n], out[n + "64"] = bits, bf16_bits_to_f32(bits).astype(np.float64)
        elif w.dtype == "mxfp8":
            out[n], out[n + "s"], out[n + "64"] = mx_quantize_packed(t, cu)
        else:
            raise ValueError(w.dtype)
    if w.dtype == "mxfp8":
        out["sq_off"] = mx_compact_offsets(cu_q)
        out["sk_off"] = mx_compact_offsets(cu_k)
    return out


def mx_compact_offsets(cu) -> np.ndarray:
    """First row of each sequence in a compact packed scale tensor: the
    exclusive prefix sum of ceil(len / 32), int32 [B+1]."""
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    return np.concatenate([[0], np.cumsum((lens + 31) // 32)]).astype(np.int32)


def mx_quantize_packed(x: np.ndarray, cu):
    """MX-quantise a packed [total, H, d] float32 tensor per sequence: 32x32
    blocks of (tokens, d) start at each sequence's first token, a partial last
    block is quantised as if padded with zeros (zeros change no amax). Returns
    (e4m3 bytes [total, H, d], compact E8M0 scales [sum ceil(len/32), H, d/32],
    exact float64 values [total, H, d])."""
    total, H, d = x.shape
    q = np.empty((total, H, d), dtype=np.uint8)
    x64 = np.empty((total, H, d), dtype=np.float64)
    scales = []
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        npad = (n + 31) // 32 * 32
        blk = np.zeros((H, npad, d), dtype=np.float32)
        blk[:, :n] = x[s0:s1].transpose(1, 0, 2)
        qb, sb = mx_quantize(blk)
        q[s0:s1] = qb[:, :n].transpose(1, 0, 2)
        x64[s0:s1] = mx_dequantize(qb, sb)[:, :n].transpose(1, 0, 2)
        scales.append(sb.transpose(1, 0, 2))
    sc = np.concatenate(scales) if scales else np.zeros((0, H, d // 32), dtype=np.uint8)
    return q, np.ascontiguousarray(sc), x64
