"""Pins of the backward oracle (oracle.attention_bwd_f64) against things
other than its own formula: central finite differences of the forward
oracle's loss, torch autograd in float64 on a separate implementation,
and invariants the softmax fixes exactly."""
import numpy as np
import pytest

from oracle import attention_bwd_f64, attention_f64, attention_loss_f64

CAUSALS = [False, "top_left", "bottom_right"]


def _draw(seed, B=1, H=2, Nq=5, Nk=7, d=4, dv=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Nq, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, dv)), rng.standard_normal((B, H, Nq, dv)))


@pytest.mark.parametrize("causal", CAUSALS)
@pytest.mark.parametrize("nq,nk", [(5, 7), (7, 5), (6, 6), (1, 4)])
def test_every_entry_matches_central_differences(causal, nq, nk):
    """Each entry of dQ, dK, dV against (L(x + h) - L(x - h)) / 2h of the
    forward oracle's loss sum(O * dO); h = 1e-5 leaves an O(h^2) truncation
    error near 1e-10, far below the tolerance."""
    q, k, v, do = _draw(11 + nq + 3 * nk, Nq=nq, Nk=nk)
    dq, dk, dv, _ = attention_bwd_f64(q, k, v, do, causal=causal, scale=0.7)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            lp = attention_loss_f64(**{**args, name: xp}, do=do, causal=causal, scale=0.7)
            lm = attention_loss_f64(**{**args, name: xm}, do=do, causal=causal, scale=0.7)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * (1 + abs(fd)), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", CAUSALS)
def test_matches_torch_autograd_float64(causal):
    """torch autograd through an independent float64 implementation (masked
    scores, torch.softmax, matmul) at a few tiles' worth of rows."""
    import torch
    q, k, v, do = _draw(5, B=2, H=3, Nq=70, Nk=90, d=16, dv=16)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = (tq @ tk.transpose(-1, -2)) * 0.25
    if causal:
        off = 0 if causal == "top_left" else 90 - 70
        mask = torch.arange(90)[None, :] > torch.arange(70)[:, None] + off
        s = s.masked_fill(mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv, _ = attention_bwd_f64(q, k, v, do, causal=causal, scale=0.25)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", CAUSALS)
def test_invariants(causal):
    """Every row's dS sums to zero (a common shift of the scores changes no
    softmax), so the dK rows sum to zero; every row's P sums to one, so the
    dV rows sum to the dO rows of the rows that see a key; D = rowsum(dO * O)."""
    q, k, v, do = _draw(9, B=1, H=2, Nq=40, Nk=30, d=8, dv=8)
    dq, dk, dv, dd = attention_bwd_f64(q, k, v, do, causal=causal, scale=0.5)
    o, lse = attention_f64(q, k, v, causal=causal, scale=0.5)
    seen = np.isfinite(lse)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), (do * seen[..., None]).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dd, (do * o).sum(axis=-1), atol=1e-12)
    if causal == "bottom_right":
        assert not seen.all()                    # Nq > Nk: rows without keys get no gradient
        assert np.all(dq[~seen] == 0.0)


def test_constant_values_and_single_key():
    """V rows all equal: O does not depend on Q or K, so dQ = dK = 0 and dV
    splits dO by P. One key: P = 1, so dV = sum of dO rows and dQ = dK = 0."""
    q, k, v, do = _draw(3, Nq=6, Nk=9, d=5, dv=4)
    v[:] = v[:, :, :1, :]
    dq, dk, dv, _ = attention_bwd_f64(q, k, v, do)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    q, k, v, do = _draw(4, Nq=6, Nk=1, d=5, dv=4)
    dq, dk, dv, _ = attention_bwd_f64(q, k, v, do)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), atol=1e-13)
