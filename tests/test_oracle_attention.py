"""Pins for the float64 attention oracle (CPU only).

Each test pins the oracle to something other than itself: closed forms of
the softmax definition, a 50-digit brute force, scipy's own softmax and
logsumexp routines (not the numpy calls the oracle makes), the exact
two-block combine of the streaming recurrence, and the rescale-frequency
table printed on the first page. A plausible slip in the oracle (a dropped
shift, a sign, a transposed operand, the wrong side of the causal mask, the
wrong scale) fails at least one of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special

from oracle import attention_f64, attention_rows_f64, blockwise_f64


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --- closed forms -----------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_mean_of_allowed_values(causal):
    # Q = 0 makes every score equal, so the softmax is uniform over the keys a
    # row may see: O_i = mean(V_0..V_last), LSE_i = ln(#keys)   (safe softmax)
    B, H, N, d = 2, 3, 37, 8
    q = np.zeros((B, H, N, d))
    k = _rand((B, H, N, d), 1)
    v = _rand((B, H, N, 5), 2)
    o, lse = attention_f64(q, k, v, causal=causal, scale=0.7)
    for i in range(N):
        n_allowed = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n_allowed].mean(axis=2), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(n_allowed), rtol=0, atol=1e-14)


def test_dominant_key_copies_its_value_row():
    # one key whose scaled score beats all others by >= 40 natural units:
    # the softmax weight of every other key is < e^-40, so O_i = V_j*, and
    # LSE_i = S_ij* up to log(1 + N e^-40)
    N, d = 50, 16
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d)) * 0.1
    jstar = 17
    # every query shares a large component on dimension 0 and only key j*
    # has a large entry there
    q[..., 0] += 30.0
    k[0, 0, jstar] = 0.0
    k[0, 0, jstar, 0] = 10.0
    scale = 1.0 / math.sqrt(d)
    v = rng.standard_normal((1, 1, N, 4))
    s = scale * (q[0, 0] @ k[0, 0].T)
    margin = s[:, jstar] - np.delete(s, jstar, axis=1).max(axis=1)
    assert margin.min() >= 40.0
    o, lse = attention_f64(q, k, v, causal=False, scale=scale)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, jstar], (N, 4)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], s[:, jstar], rtol=0, atol=1e-14)


def test_causal_row_zero_sees_only_key_zero():
    # causal mask S_ij = -inf for j > i: row 0 keeps key 0 only, so O_0 = V_0
    # exactly and LSE_0 = S_00
    q, k, v = _rand((2, 2, 9, 8), 4), _rand((2, 2, 9, 8), 5), _rand((2, 2, 9, 8), 6)
    o, lse = attention_f64(q, k, v, causal=True, scale=0.3)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-15)


def test_constant_values_and_lse_bounds():
    # V = 1 gives O = 1; LSE_i lies in [m_i, m_i + ln(#keys)]
    q, k = _rand((1, 2, 30, 8), 7, 2.0), _rand((1, 2, 30, 8), 8, 2.0)
    v = np.ones((1, 2, 30, 3))
    for causal in (False, True):
        o, lse = attention_f64(q, k, v, causal=causal, scale=0.5)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)
        s = 0.5 * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.triu(np.ones((30, 30), bool), 1), -np.inf, s)
        m = s.max(-1)
        cnt = (np.arange(30) + 1) if causal else np.full(30, 30)
        assert np.all(lse >= m - 1e-12) and np.all(lse <= m + np.log(cnt) + 1e-12)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = _rand((1, 1, 6, 9), 9), _rand((1, 1, 6, 9), 10), _rand((1, 1, 6, 9), 11)
    o1, l1 = attention_f64(q, k, v)
    o2, l2 = attention_f64(q, k, v, scale=1.0 / 3.0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --- brute force at 50 digits ------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_mpmath(causal):
    mpmath.mp.dps = 50
    Nq, Nk, d, dv = 5, 7, 4, 3
    q, k, v = _rand((1, 1, Nq, d), 12, 1.5), _rand((1, 1, Nk, d), 13, 1.5), _rand((1, 1, Nk, dv), 14)
    scale = 0.61
    o, lse = attention_f64(q, k, v, causal=causal, scale=scale)
    for i in range(Nq):
        keys = range(min(Nk, i + 1)) if causal else range(Nk)
        sc = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, 0, i, t]) * mpmath.mpf(k[0, 0, j, t])
                                                  for t in range(d)) for j in keys}
        z = mpmath.fsum(mpmath.exp(s) for s in sc.values())
        assert abs(float(mpmath.log(z)) - lse[0, 0, i]) < 1e-14
        for c in range(dv):
            oc = mpmath.fsum(mpmath.exp(sc[j]) * mpmath.mpf(v[0, 0, j, c]) for j in keys) / z
            assert abs(float(oc) - o[0, 0, i, c]) < 1e-14


# --- scipy's softmax / logsumexp ----------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_against_scipy_routines(causal):
    B, H, Nq, Nk, d = 2, 3, 70, 90, 16
    q, k, v = _rand((B, H, Nq, d), 15), _rand((B, H, Nk, d), 16), _rand((B, H, Nk, d), 17)
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_f64(q, k, v, causal=causal, scale=scale, chunk=32)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    if causal:
        s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, np.matmul(scipy.special.softmax(s, axis=-1), v), rtol=0, atol=1e-13)


def test_rows_subset_matches_full():
    q, k, v = _rand((2, 2, 64, 8), 18), _rand((2, 2, 80, 8), 19), _rand((2, 2, 80, 8), 20)
    o, lse = attention_f64(q, k, v, causal=True, scale=0.4)
    rows = np.array([0, 5, 63, 31])
    o1, l1 = attention_rows_f64(q, k, v, 1, 0, rows, causal=True, scale=0.4)
    np.testing.assert_allclose(o1, o[1, 0, rows], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l1, lse[1, 0, rows], rtol=0, atol=1e-15)


def test_key_permutation_invariance():
    # non-causal attention does not depend on the order of the (K, V) pairs
    q, k, v = _rand((1, 2, 20, 8), 21), _rand((1, 2, 33, 8), 22), _rand((1, 2, 33, 6), 23)
    perm = np.random.default_rng(24).permutation(33)
    o1, l1 = attention_f64(q, k, v)
    o2, l2 = attention_f64(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


# --- the streaming recurrence equals the one-shot definition ------------------
@pytest.mark.parametrize("block", [16, 64, 128])
@pytest.mark.parametrize("tau", [0.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_equals_one_shot_small(block, tau, causal):
    # exact two-block combine: the blockwise result equals the one-shot
    # softmax up to float64 reduction-order noise, for either max policy
    q, k, v = _rand((1, 2, 100, 16), 25, 2.0), _rand((1, 2, 150, 16), 26, 2.0), _rand((1, 2, 150, 16), 27)
    o1, l1 = attention_f64(q, k, v, causal=causal)
    o2, l2, _ = blockwise_f64(q, k, v, causal=causal, block=block, tau=tau)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_blockwise_equals_one_shot_lecture_shape(tau):
    # the lecture's own check: H=2, N=1024, d=64, block 64, fp64 ~ 1e-13
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 2, 1024, 64))
    k = rng.standard_normal((1, 2, 1024, 64))
    v = rng.standard_normal((1, 2, 1024, 64))
    o1, l1 = attention_f64(q, k, v)
    o2, l2, _ = blockwise_f64(q, k, v, block=64, tau=tau)
    assert np.abs(o2 - o1).max() < 1e-12
    assert np.abs(l2 - l1).max() < 1e-12


def test_lagging_max_skips_small_growth():
    # tau in log2 units of the scaled scores: a growth of exactly tau is kept
    # (>= -tau keeps the stale max), a growth just above tau commits
    scores = np.zeros((1, 4))
    scores[0, 2:] = 8.0                       # block 2 raises the max by exactly 8
    _, _, st = blockwise_f64(None, None, None, block=2, tau=8.0, group=1, scores_log2=scores)
    assert st["rows"].tolist() == [[False, False]]
    scores[0, 2:] = 8.0 + 1e-9
    _, _, st = blockwise_f64(None, None, None, block=2, tau=8.0, group=1, scores_log2=scores)
    assert st["rows"].tolist() == [[False, True]]
    _, _, st = blockwise_f64(None, None, None, block=2, tau=0.0, group=1, scores_log2=scores)
    assert st["rows"].tolist() == [[False, True]]


def test_rescale_frequency_table(golden_dir):
    # the first page's simulation: 256 rows x 8192 keys, 128-key blocks
    gold = json.load(open(os.path.join(golden_dir, "rescale_frequency.json")))
    R, N, blk = gold["rows"], gold["keys"], gold["block"]
    rng = np.random.default_rng(2024)
    for row in gold["table"]:
        s = rng.normal(0.0, row["sigma"], (R, N)) + np.linspace(0.0, row["rise"], N)
        for tau in (0, 8):
            _, _, st = blockwise_f64(None, None, None, block=blk, tau=float(tau), group=gold["group"],
                                     scores_log2=s)
            rows_pct = 100.0 * st["rows"][:, 1:].mean()
            warps_pct = 100.0 * st["groups"][:, 1:].mean()
            exp_rows, exp_warps = row[f"tau{tau}_rows"], row[f"tau{tau}_warps"]
            # sampling noise: about 0.2 points on rows, 3 points on warps
            assert abs(rows_pct - exp_rows) <= max(0.6, 0.03 * exp_rows), (row["scores"], tau, rows_pct)
            assert abs(warps_pct - exp_warps) <= 5.0, (row["scores"], tau, warps_pct)


# --- causal alignment when Nq != Nk ------------------------------------------
@pytest.mark.parametrize("nq,nk", [(37, 37), (11, 37), (37, 11), (1, 20), (20, 1)])
def test_bottom_right_equal_scores(nq, nk):
    # Q = 0: row i sees keys 0 .. i + Nk - Nq (bottom-right alignment), so O_i is
    # their mean and LSE_i = ln(count); a row that sees none gets O = 0, LSE = -inf
    q = np.zeros((1, 2, nq, 8))
    k = _rand((1, 2, nk, 8), 3)
    v = _rand((1, 2, nk, 5), 4)
    o, lse = attention_f64(q, k, v, causal="bottom_right", scale=0.9)
    for i in range(nq):
        n = min(nk, max(0, i + nk - nq + 1))
        if n == 0:
            assert np.all(o[:, :, i] == 0.0) and np.all(lse[:, :, i] == -np.inf)
        else:
            np.testing.assert_allclose(o[:, :, i], v[:, :, :n].mean(axis=2), rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14)


def test_bottom_right_equals_top_left_when_square_and_last_row_sees_all():
    q, k, v = _rand((2, 2, 24, 16), 5), _rand((2, 2, 24, 16), 6), _rand((2, 2, 24, 16), 7)
    o1, l1 = attention_f64(q, k, v, causal=True)
    o2, l2 = attention_f64(q, k, v, causal="bottom_right")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    q = _rand((1, 2, 9, 16), 8)
    k, v = _rand((1, 2, 30, 16), 9), _rand((1, 2, 30, 16), 10)
    on, ln_ = attention_f64(q, k, v, causal=False)
    ob, lb = attention_f64(q, k, v, causal="bottom_right")
    np.testing.assert_allclose(ob[:, :, -1], on[:, :, -1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lb[:, :, -1], ln_[:, :, -1], rtol=0, atol=1e-14)
    # and the top-left mask keeps the first row to key 0 only
    ot, _ = attention_f64(q, k, v, causal=True)
    np.testing.assert_allclose(ot[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("nq,nk", [(13, 40), (40, 13)])
def test_bottom_right_brute_force_and_blockwise(nq, nk):
    q, k, v = _rand((1, 1, nq, 6), 11), _rand((1, 1, nk, 6), 12), _rand((1, 1, nk, 3), 13)
    o, lse = attention_f64(q, k, v, causal="bottom_right", scale=0.5)
    for i in range(nq):
        keys = [j for j in range(nk) if j <= i + nk - nq]
        if not keys:
            continue
        sc = [0.5 * float(np.dot(q[0, 0, i], k[0, 0, j])) for j in keys]
        np.testing.assert_allclose(lse[0, 0, i], scipy.special.logsumexp(sc), rtol=0, atol=1e-13)
        w = scipy.special.softmax(sc)
        np.testing.assert_allclose(o[0, 0, i], w @ v[0, 0, keys], rtol=0, atol=1e-13)
    for tau in (0.0, 8.0):
        ob, lb, _ = blockwise_f64(q, k, v, causal="bottom_right", scale=0.5, block=8, tau=tau)
        fin = np.isfinite(lse)
        np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
        assert np.array_equal(np.isfinite(lb), fin)
        np.testing.assert_allclose(lb[fin], lse[fin], rtol=0, atol=1e-12)
