"""GPU parity of the MXFP8 backward pass (attn_bwd_ex, ATTN_MXFP8_E4M3) and of
the square-block quantiser (attn_mx_quantize).

The oracle (oracle.attention_bwd_f64) sees the exact values the kernels
receive: Q, K, V, dO dequantised (dO quantised on the host with the input
module's quantiser, the rule attn_mx_quantize is checked against bit for bit).

Bound per element, derived from the kernels' arithmetic: P is cast to e4m3
times 2^8 with one fixed scale (relative error <= 2^-4, plus half an e4m3
subnormal step, 2^-10 / 2^8, in P's units); dS is cast with one E8M0 scale X
per 32x32 block, amax / X in (224, 448] (relative error <= 2^-4, plus
2^-10 X <= 2^-10 amax / 224 below the normal range); D is formed from a bf16
O (dD_i = c_O sum_c |dO_ic| |O_ic|, c_O = 2^-7 for an O rounded from the
exact one, 2^-4 for the MXFP8 forward's O, whose P carries the same 2^-4);
results are rounded to bf16. Each term is doubled for slack:

  |dV_j - ref| <= sum_i (2^-3 P_ij + 2^-17) |dO_i| + 2^-8 |dV_j|
  |dK_j - ref| <= scale sum_i (2^-3 |dS_ij| + 2^-9 amax_b(ij) / 224 + P_ij dD_i) |Q_i| + 2^-8 |dK_j|
  |dQ_i - ref| <= scale sum_j (the same weights) |K_j| + 2^-8 |dQ_i|       (+ 1e-5 each)
"""
import numpy as np
import pytest

from attn_inputs import (WORKLOADS, bf16_bits, bf16_bits_to_f32, make_grad_output, make_inputs, mx_dequantize,
                         mx_quantize)
from oracle import attention_bwd_f64, attention_f64
from oracle.attention import causal_offset

from _gpu import announce, attn_module, host64

pytestmark = pytest.mark.gpu

MX = WORKLOADS["mxfp8_b2h16_n8192_d128"]


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return attn_module()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def test_mx_quantize_matches_host(attn):
    """attn_mx_quantize against the input module's quantiser (E8M0 rule and
    e4m3 rounding), bit for bit, over blocks of very different magnitudes,
    an all-zero block and values in e4m3's subnormal range."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 96, 128)).astype(np.float32)
    mag = np.exp2(rng.integers(-30, 30, size=(2, 3, 3, 1, 4, 1))).astype(np.float32)
    x = (x.reshape(2, 3, 3, 32, 4, 32) * mag).reshape(2, 3, 96, 128)
    x[0, 0, :32, :32] = 0.0
    x[1, 2, 32:64, 64:96] *= np.float32(2.0 ** -12)
    bits = bf16_bits(x)
    q_ref, s_ref = mx_quantize(bf16_bits_to_f32(bits))
    q, s = attn.mx_quantize(_dev_bf16(bits))
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    announce(f"mx_quantize: {np.sum(qh != q_ref)} e4m3 and {np.sum(sh != s_ref)} E8M0 bytes differ")
    assert np.array_equal(sh, s_ref)
    assert np.array_equal(qh, q_ref)


def _bounds(q, k, v, do, o, causal, scale, c_o):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    bq, bk, bv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    off = causal_offset(causal, Nq, Nk)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if off is not None:
                s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off, -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s - m)
            den = e.sum(axis=1, keepdims=True)
            p = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            amax = np.abs(ds).reshape(Nq // 32, 32, Nk // 32, 32).max(axis=(1, 3))
            sub = np.repeat(np.repeat(amax, 32, axis=0), 32, axis=1) * 2.0 ** -9 / 224
            dd = c_o * (np.abs(do[b, h]) * np.abs(o[b, h])).sum(axis=1, keepdims=True)
            w = 2.0 ** -3 * np.abs(ds) + sub + p * dd
            bv[b, h] = (2.0 ** -3 * p + 2.0 ** -17).T @ np.abs(do[b, h])
            bk[b, h] = scale * (w.T @ np.abs(q[b, h]))
            bq[b, h] = scale * (w @ np.abs(k[b, h]))
    return bq, bk, bv


def _check(what, got, ref, bound):
    err = np.abs(got - ref)
    tol = bound + 2.0 ** -8 * np.abs(ref) + 1e-5
    ratio = (err / tol).max() if err.size else 0.0
    announce(f"{what}: max|err|={err.max() if err.size else 0:.3e} max(err/bound)={ratio:.3f}")
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= tol), (what, ratio)


def _run(attn, B, H, Nq, Nk, causal, source, seed=11):
    import torch
    x = make_inputs(MX, B=B, H=H, Nq=Nq, Nk=Nk, seed=seed)
    g_bits, _ = make_grad_output((B, H, Nq, 128), seed + 500)
    g_q, g_s = mx_quantize(bf16_bits_to_f32(g_bits))
    g64 = mx_dequantize(g_q, g_s)
    q, k, v, qs, ks, vs = (_dev(x[n]) for n in ("q", "k", "v", "qs", "ks", "vs"))
    do, dos = _dev(g_q), _dev(g_s)
    if source == "oracle":
        o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
        o_bits = bf16_bits(o_ref.astype(np.float32))
        o, lse = _dev_bf16(o_bits), _dev(lse_ref.astype(np.float32))
        o64, c_o = bf16_bits_to_f32(o_bits).astype(np.float64), 2.0 ** -7
    else:
        o, lse = attn.fwd(q, k, v, causal=causal, exp2_mode="hw", tau=0.0, q_scale=qs, k_scale=ks, v_scale=vs)
        o64, c_o = host64(o), 2.0 ** -4
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, causal=causal, q_scale=qs, k_scale=ks, v_scale=vs, do_scale=dos)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(128)
    rq, rk, rv, _ = attention_bwd_f64(x["q64"], x["k64"], x["v64"], g64, causal=causal)
    bq, bk, bv = _bounds(x["q64"], x["k64"], x["v64"], g64, o64, causal, scale, c_o)
    tag = f"mxfp8 bwd B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} O/LSE from {source}"
    _check(tag + " dQ", host64(dq), rq, bq)
    _check(tag + " dK", host64(dk), rk, bk)
    _check(tag + " dV", host64(dv), rv, bv)
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, "top_left", "bottom_right"])
@pytest.mark.parametrize("source", ["oracle", "kernel"])
def test_mxfp8_bwd_small(attn, causal, source):
    """320 queries (five 64-row tiles), 352 keys (a half tile at the end)."""
    announce(f"mxfp8 bwd small causal={causal} {source}")
    _run(attn, 1, 2, 320, 352, causal, source)


@pytest.mark.parametrize("nq,nk,causal", [(96, 160, "bottom_right"), (160, 96, "bottom_right"), (160, 96, "top_left"),
                                          (32, 32, "top_left"), (64, 32, False), (32, 224, False)])
def test_mxfp8_bwd_edge_shapes(attn, nq, nk, causal):
    """Nq != Nk both ways (bottom-right with Nq > Nk leaves rows without keys),
    single 32-row blocks, half tiles."""
    announce(f"mxfp8 bwd edge Nq={nq} Nk={nk} causal={causal}")
    _run(attn, 1, 2, nq, nk, causal, "oracle", seed=nq + 3 * nk)


def test_mxfp8_bwd_larger(attn):
    announce("mxfp8 bwd 2x3x1024 causal")
    _run(attn, 2, 3, 1024, 1024, "top_left", "kernel", seed=21)


def test_mxfp8_bwd_deterministic(attn):
    import torch
    a = _run(attn, 1, 2, 320, 352, "top_left", "kernel", seed=5)
    b = _run(attn, 1, 2, 320, 352, "top_left", "kernel", seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
