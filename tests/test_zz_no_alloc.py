"""The no-allocation entry point (attn_fwd_split_noalloc) against the entry
point it varies (attn_fwd_split with a caller workspace), through the C ABI:
two calls in a row on the device's shared scratch, the second smaller, each
bitwise equal to attn_fwd_split for the same chunk and within the stated
tolerances of the float64 oracle (O 2e-2, LSE 1e-3)."""
import ctypes
import math

import numpy as np
import pytest

from attn_inputs import WORKLOADS, make_inputs
from oracle import attention_f64

from _gpu import TOL_LSE, TOL_O, announce, attn_module, host64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return attn_module()


def _noalloc(attn, dev, causal, key_chunk, torch):
    lib = attn.load_library()
    fn = lib.attn_fwd_split_noalloc
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.argtypes = [vp] * 5 + [ci] * 6 + [cf, ci, cf, ci, vp, vp, vp, ci, vp]
    fn.restype = ci
    q, k = dev["q"], dev["k"]
    B, H, Nq, d = q.shape
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    rc = fn(q.data_ptr(), k.data_ptr(), dev["v"].data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq, k.shape[2], d,
            {False: 0, True: 1, "bottom_right": 2}[causal], 1.0 / math.sqrt(d), 0, 8.0, 1, None, None, None,
            key_chunk, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.attn_last_error()
    return o, lse


@pytest.mark.parametrize("key_chunk", [0, 512])
def test_noalloc_matches_split_on_two_calls(attn, key_chunk):
    import torch
    w = WORKLOADS["bf16_b4h16_n4096_d128"]
    # first call: a decoding-like launch the library splits; second, smaller
    cases = [(dict(B=1, H=8, Nq=1, Nk=32768), False), (dict(B=1, H=2, Nq=300, Nk=1100), "bottom_right")]
    for shape, causal in cases:
        x = make_inputs(w, **shape)
        dev = to_device(x)
        assert attn.split_workspace_bytes(dev["q"], dev["k"], causal=causal, key_chunk=key_chunk) > 0
        announce(f"noalloc {shape} causal={causal} key_chunk={key_chunk}")
        o_n, l_n = _noalloc(attn, dev, causal, key_chunk, torch)
        o_s, l_s = attn.fwd_split(dev["q"], dev["k"], dev["v"], causal=causal, exp2_mode="hw", tau=8.0,
                                  key_chunk=key_chunk)
        torch.cuda.synchronize()
        assert np.array_equal(host64(o_n), host64(o_s)) and np.array_equal(host64(l_n), host64(l_s))
        o_ref, lse_ref = attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
        fin = np.isfinite(lse_ref)
        err_o = np.abs(host64(o_n) - o_ref).max()
        err_l = np.abs(host64(l_n)[fin] - lse_ref[fin]).max()
        announce(f"  max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
        assert err_o <= TOL_O["bf16"] and err_l <= TOL_LSE


def test_noalloc_rejects_a_chunk_beyond_the_scratch(attn):
    """An explicit chunk whose partials exceed the scratch is refused before
    any launch; the library's chunk is grown to fit instead."""
    import torch
    lib = attn.load_library()
    w = WORKLOADS["bf16_b4h16_n4096_d128"]
    x = make_inputs(w, B=1, H=64, Nq=128, Nk=16384)
    dev = to_device(x)
    need = attn.split_workspace_bytes(dev["q"], dev["k"], key_chunk=64)
    assert need > 64 * 1024 * 1024
    with pytest.raises(AssertionError, match="scratch"):
        _noalloc(attn, dev, False, 64, torch)
    assert lib.attn_fwd_split_noalloc is not None
    o, lse = _noalloc(attn, dev, False, 0, torch)
    o_ref, lse_ref = attention_f64(x["q64"][:, :4], x["k64"][:, :4], x["v64"][:, :4])
    assert np.abs(host64(o)[:, :4] - o_ref).max() <= TOL_O["bf16"]
    assert np.abs(host64(lse)[:, :4] - lse_ref).max() <= TOL_LSE
