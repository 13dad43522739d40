"""GPU parity of the backward pass (attn_bwd, bf16) against the float64
oracle (oracle.attention_bwd_f64), element by element.

Bound per element, derived from the arithmetic of the kernels (float32
accumulation of bf16 operands; P and dS rounded to bf16 before the dV, dK and
dQ products; O read as bf16 to form D; results rounded to bf16): each rounded
operand carries a relative error of at most 2^-9, taken here with a factor 4
of slack, so

  |dV_j - ref| <= 2^-7 sum_i P_ij |dO_i| + 2^-8 |dV_j| + 1e-5
  |dK_j - ref| <= scale sum_i (2^-7 |dS_ij| + P_ij dD_i) |Q_i| + 2^-8 |dK_j| + 1e-5
  |dQ_i - ref| <= scale sum_j (2^-7 |dS_ij| + P_ij dD_i) |K_j| + 2^-8 |dQ_i| + 1e-5
  dD_i = 2^-7 sum_c |dO_ic| |O_ic|      (D formed from a bf16 O)

with P, dS and O from the float64 definition. O and LSE fed to the kernel
come either from the oracle (O rounded to bf16, LSE to float32) or from the
forward kernel itself (the way the pair is used).
"""
import numpy as np
import pytest

from attn_inputs import WORKLOADS, bf16_bits, bf16_bits_to_f32, make_grad_output, make_inputs
from oracle import attention_bwd_f64, attention_f64
from oracle.attention import causal_offset

from _gpu import announce, attn_module, host64

pytestmark = pytest.mark.gpu

BF16 = {64: WORKLOADS["bf16_b2h32_n8192_d64_causal_spiky"], 128: WORKLOADS["bf16_b4h16_n4096_d128"]}


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return attn_module()


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bounds(q, k, v, do, o, causal, scale):
    """Per-element bounds of dQ, dK, dV (float64 numpy), as in the module docstring."""
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
            dd = (p * dp).sum(axis=1, keepdims=True)
            ds = np.abs(p * (dp - dd))
            ddd = 2.0 ** -7 * (np.abs(do[b, h]) * np.abs(o[b, h])).sum(axis=1, keepdims=True)
            w = 2.0 ** -7 * ds + p * ddd
            bv[b, h] = 2.0 ** -7 * (p.T @ np.abs(do[b, h]))
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


def _run_case(attn, d, B, H, Nq, Nk, causal, source, seed=7):
    import torch
    w = BF16[d]
    x = make_inputs(w, B=B, H=H, Nq=Nq, Nk=Nk, seed=seed)
    g_bits, g64 = make_grad_output((B, H, Nq, d), seed + 1000)
    scale = 1.0 / np.sqrt(d)
    q, k, v = (_dev_bf16(x[n]) for n in ("q", "k", "v"))
    do = _dev_bf16(g_bits)
    if source == "oracle":
        o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
        o_bits = bf16_bits(o_ref.astype(np.float32))
        o = _dev_bf16(o_bits)
        lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
        o64 = bf16_bits_to_f32(o_bits).astype(np.float64)
    else:
        o, lse = attn.fwd(q, k, v, causal=causal, exp2_mode="hw", tau=8.0)
        o64 = host64(o)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, _ = attention_bwd_f64(x["q64"], x["k64"], x["v64"], g64, causal=causal)
    bq, bk, bv = _bounds(x["q64"], x["k64"], x["v64"], g64, o64, causal, scale)
    tag = f"bwd d={d} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} O/LSE from {source}"
    _check(tag + " dQ", host64(dq), rq, bq)
    _check(tag + " dK", host64(dk), rk, bk)
    _check(tag + " dV", host64(dv), rv, bv)
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, "top_left", "bottom_right"])
@pytest.mark.parametrize("source", ["oracle", "kernel"])
def test_bwd_small_ragged(attn, d, causal, source):
    """Several tiles with ragged tails on both sides (query tiles of 64, 128
    and 256 rows, key blocks of 128 and tiles of 64)."""
    announce(f"bwd small d={d} causal={causal} {source}")
    _run_case(attn, d, 1, 2, 300, 333, causal, source)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,causal", [(100, 333, "bottom_right"), (333, 100, "bottom_right"),
                                          (333, 100, "top_left"), (1, 300, False), (300, 1, False),
                                          (1, 1, "top_left"), (64, 64, "top_left"), (129, 257, False),
                                          (600, 100, "bottom_right")])
def test_bwd_edge_shapes(attn, d, nq, nk, causal):
    """Nq != Nk both ways (bottom-right with Nq > Nk leaves rows without keys:
    their dQ is 0 and they add nothing; at 600 x 100 whole 256-row dQ
    workgroups see no key), single rows and keys, exact tiles."""
    announce(f"bwd edge d={d} Nq={nq} Nk={nk} causal={causal}")
    _run_case(attn, d, 1, 2, nq, nk, causal, "oracle", seed=nq + 7 * nk)


# d = 128 launches with B*H*ceil(Nq/256) >= 256 take the ping-pong dQ kernel
# (256 query rows per workgroup); smaller ones the streaming dQ kernel.
DQ_PINGPONG_MIN_TILES = 256


@pytest.mark.parametrize("nq,nk,causal", [(300, 333, False), (300, 333, "top_left"), (300, 333, "bottom_right"),
                                          (600, 100, "bottom_right"), (1100, 1030, "top_left")])
def test_bwd_pingpong_dq(attn, nq, nk, causal):
    """Enough heads for the ping-pong dQ kernel, every element: ragged query
    and key tails, 1 to 17 key tiles per workgroup (every count mod 3, the
    kernel's unroll), workgroups that see no key (bottom-right 600 x 100)."""
    n_qt = -(-nq // 256)
    H = -(-DQ_PINGPONG_MIN_TILES // n_qt)
    announce(f"bwd ping-pong dQ d=128 H={H} Nq={nq} Nk={nk} causal={causal}")
    _run_case(attn, 128, 1, H, nq, nk, causal, "oracle", seed=nq + 3 * nk)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_larger_heads(attn, d):
    """B=2, H=3 at 1024 x 1024 (a causal triangle of 16 query tiles), every element."""
    announce(f"bwd 2x3x1024 d={d}")
    _run_case(attn, d, 2, 3, 1024, 1024, "top_left", "kernel", seed=99)


def test_bwd_no_queries_or_no_keys(attn):
    """Nq = 0: dK = dV = 0. Nk = 0: every row sees no key, dQ = 0 (LSE = -inf)."""
    import torch
    B, H, d = 1, 2, 128
    q = torch.zeros((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((B, H, 50, d), device="cuda").to(torch.bfloat16)
    lse = torch.zeros((B, H, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    dq, dk, dv = attn.bwd(q, k, k, q, q, lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    q = torch.randn((B, H, 40, d), device="cuda").to(torch.bfloat16)
    k0 = torch.zeros((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, 40), float("-inf"), device="cuda")
    dq = torch.full_like(q, 7.0)
    dq, _, _ = attn.bwd(q, k0, k0, q, q, lse, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_bwd_deterministic(attn):
    """No atomics anywhere: two runs give the same bits."""
    import torch
    announce("bwd determinism")
    a = _run_case(attn, 128, 1, 2, 300, 333, "top_left", "kernel", seed=5)
    b = _run_case(attn, 128, 1, 2, 300, 333, "top_left", "kernel", seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
