"""GPU parity of the key-split forward (attn_fwd_split) against the float64
oracle.

Each row's keys are cut into chunks run by separate workgroups and merged
exactly ("Lecture 2 -- Online Softmax and Numerical Correctness", section
"Combining two blocks exactly"). The merged O and LSE are the same
attention, so the tolerances are the stated ones: max abs error of O 2e-2
(bf16), LSE 1e-3.
"""
import math

import numpy as np
import pytest

from attn_inputs import WORKLOADS, make_inputs
from oracle import attention_f64

from _gpu import TOL_LSE, TOL_O, announce, attn_module, host64, to_device

pytestmark = pytest.mark.gpu

BF16_BY_D = {64: "bf16_b2h32_n8192_d64_causal_spiky", 128: "bf16_b4h16_n4096_d128",
             192: "bf16_b4h16_n4096_d192", 256: "bf16_b4h16_n4096_d256"}


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return attn_module()


def _check(o, lse, o_ref, lse_ref, what):
    o_h, l_h = host64(o), host64(lse)
    fin = np.isfinite(lse_ref)
    err_o = np.abs(o_h - o_ref).max()
    err_l = np.abs(l_h[fin] - lse_ref[fin]).max(initial=0.0)
    announce(f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert np.isfinite(err_o) and err_o <= TOL_O["bf16"], (what, err_o)
    assert err_l <= TOL_LSE, (what, err_l)
    assert np.array_equal(np.isneginf(l_h), ~fin), what   # rows without keys: LSE = -inf


def _split(attn, dev, causal, mode, tau, key_chunk):
    return attn.fwd_split(dev["q"], dev["k"], dev["v"], causal=causal, exp2_mode=mode, tau=tau, key_chunk=key_chunk)


@pytest.mark.parametrize("d", [64, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, "top_left", "bottom_right"])
@pytest.mark.parametrize("key_chunk", [64, 128, 320])
def test_split_small_ragged(attn, d, causal, key_chunk):
    """Explicit chunk sizes on ragged shapes (300 query rows, 1100 keys:
    tails in both, 4 to 18 chunks per tile), each head against the oracle."""
    w = WORKLOADS[BF16_BY_D[d]]
    x = make_inputs(w, B=1, H=2, Nq=300, Nk=1100)
    dev = to_device(x)
    o, lse = _split(attn, dev, causal, "hw", 8.0, key_chunk)
    o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
    _check(o, lse, o_ref, lse_ref, f"split d={d} causal={causal} chunk={key_chunk}")


@pytest.mark.parametrize("mode", ["emu", "mix2", "emu4"])
@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_split_exp2_modes_and_tau(attn, mode, tau):
    """Software exp2 paths and both lagging-max settings inside the chunks."""
    x = make_inputs(WORKLOADS[BF16_BY_D[128]], B=1, H=2, Nq=300, Nk=1100)
    dev = to_device(x)
    o, lse = _split(attn, dev, True, mode, tau, 128)
    o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=True)
    _check(o, lse, o_ref, lse_ref, f"split {mode} tau={tau}")


@pytest.mark.parametrize("nq,nk", [(600, 100), (100, 600), (1, 5000), (257, 64), (128, 1)])
def test_split_edge_shapes(attn, nq, nk):
    """Bottom-right causal with rows that see no key (Nq > Nk), single rows,
    one key, tiles that fit one chunk next to tiles cut into many."""
    x = make_inputs(WORKLOADS[BF16_BY_D[128]], B=2, H=3, Nq=nq, Nk=nk)
    dev = to_device(x)
    for causal in (False, "bottom_right"):
        o, lse = _split(attn, dev, causal, "hw", 8.0, 64)
        o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
        _check(o, lse, o_ref, lse_ref, f"split edge {nq}x{nk} causal={causal}")


@pytest.mark.parametrize("key_chunk", [128, 192])
def test_split_small_causal_workload(attn, key_chunk):
    """The B=2 H=8 N=1024 d=128 causal workload cut into 128- and 192-key
    chunks (the library itself runs it whole), every element against the
    oracle, and bitwise the same on a second call."""
    w = WORKLOADS["bf16_b2h8_n1024_d128_causal"]
    x = make_inputs(w)
    dev = to_device(x)
    assert attn.split_workspace_bytes(dev["q"], dev["k"], causal=True) == 0
    o, lse = _split(attn, dev, True, w.exp2_mode, w.tau, key_chunk)
    o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=True)
    _check(o, lse, o_ref, lse_ref, f"split B2 H8 N1024 causal chunk={key_chunk}")
    o2, lse2 = _split(attn, dev, True, w.exp2_mode, w.tau, key_chunk)
    assert np.array_equal(host64(o), host64(o2)) and np.array_equal(host64(lse), host64(lse2))


def test_split_decoding_like(attn):
    """One query row per head against 32768 keys: the library cuts the keys
    over the whole chip."""
    x = make_inputs(WORKLOADS[BF16_BY_D[128]], B=1, H=8, Nq=1, Nk=32768)
    dev = to_device(x)
    assert attn.split_workspace_bytes(dev["q"], dev["k"]) > 0
    o, lse = _split(attn, dev, False, "hw", 8.0, 0)
    o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"])
    _check(o, lse, o_ref, lse_ref, "split decoding-like Nq=1 Nk=32768")


def test_split_other_dtypes_run_whole(attn):
    """float32 launches are not split: attn_fwd_split gives attn_fwd_ex's
    bits and needs no workspace."""
    x = make_inputs(WORKLOADS["fp32_b1h1_n128_d64"], B=1, H=2, Nq=200, Nk=300)
    dev = to_device(x)
    assert attn.split_workspace_bytes(dev["q"], dev["k"], key_chunk=64) == 0
    o1, l1 = attn.fwd(dev["q"], dev["k"], dev["v"], causal=True, exp2_mode="hw")
    o2, l2 = attn.fwd_split(dev["q"], dev["k"], dev["v"], causal=True, exp2_mode="hw", key_chunk=64)
    assert np.array_equal(host64(o1), host64(o2)) and np.array_equal(host64(l1), host64(l2))


def test_split_rows_of_one_chunk_match_the_streaming_kernel(attn):
    """A chunk longer than every row leaves one chunk per tile: the split
    kernel then writes O and LSE itself, with the streaming kernel's bits
    (d = 64 is always on the streaming kernel)."""
    x = make_inputs(WORKLOADS[BF16_BY_D[64]], B=1, H=2, Nq=300, Nk=333)
    dev = to_device(x)
    o1, l1 = attn.fwd(dev["q"], dev["k"], dev["v"], causal=True, exp2_mode="hw")
    o2, l2 = _split(attn, dev, True, "hw", 8.0, 384)
    assert np.array_equal(host64(o1), host64(o2)) and np.array_equal(host64(l1), host64(l2))
    scale = 1.0 / math.sqrt(64)
    o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=True, scale=scale)
    _check(o2, l2, o_ref, lse_ref, "split one chunk per tile")
