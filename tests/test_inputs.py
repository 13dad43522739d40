"""CPU checks of the seeded input generators (bf16 cast, e4m3, E8M0)."""
import numpy as np
import pytest
import torch

from attn_inputs import (WORKLOADS, bf16_bits, bf16_bits_to_f32, e4m3_decode_table, e4m3_encode,
                         e8m0_for_amax, make_inputs, mx_dequantize, mx_quantize)


def test_bf16_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32) * 1e3
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]          # exact ties both ways
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = e4m3_decode_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_encode_matches_torch_in_range():
    x = np.random.default_rng(1).standard_normal(1 << 16) * 60.0
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3_encode(x)
    # torch keeps the sign of zero; the encoder here writes +0
    diff = ours != ref
    assert np.all((ref[diff] == 0x80) & (ours[diff] == 0))
    assert np.array_equal(e4m3_encode(np.array([1e6, -1e6])), np.array([0x7E, 0xFE], np.uint8))


def test_e8m0_is_the_smallest_non_saturating_power_of_two():
    amax = np.abs(np.random.default_rng(2).standard_normal(10000).astype(np.float32)) * 37 + 1e-3
    amax[:3] = [448.0, 1.75, 1.7500001]
    x = np.ldexp(1.0, e8m0_for_amax(amax).astype(np.int64) - 127)
    assert np.all(amax / x <= 448.0)
    assert np.all(amax / (x / 2) > 448.0)


def test_mx_roundtrip_error_bound():
    x = np.random.default_rng(3).standard_normal((2, 64, 96)).astype(np.float32)
    q, s = mx_quantize(x)
    assert q.shape == x.shape and s.shape == (2, 2, 3)
    xd = mx_dequantize(q, s)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normal codes
    big = np.abs(x) > 2.0 ** -6 * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, 1).repeat(32, 2)
    assert np.all(np.abs(xd - x)[big] <= np.abs(x)[big] * 2.0 ** -4 + 1e-12)


def test_workload_inputs_are_deterministic_and_spiked():
    w = WORKLOADS["bf16_b2h32_n8192_d64_causal_spiky"]
    a = make_inputs(w, B=1, H=2, Nq=256, Nk=256)
    b = make_inputs(w, B=1, H=2, Nq=256, Nk=256)
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["q64"], b["q64"])
    assert a["q"].dtype == np.uint16
    norms = np.linalg.norm(a["k64"], axis=-1)
    n_big = (norms > 4 * np.median(norms)).sum(axis=-1)
    assert np.all(n_big == round(0.01 * 256))
    np.testing.assert_array_equal(a["k64"], bf16_bits_to_f32(a["k"]).astype(np.float64))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_small_draw_of_each_workload(name):
    w = WORKLOADS[name]
    x = make_inputs(w, B=1, H=1, Nq=64, Nk=96)
    assert x["q64"].shape == (1, 1, 64, w.d) and x["v64"].shape == (1, 1, 96, w.d)
    if w.dtype == "mxfp8":
        assert x["qs"].shape == (1, 1, 2, w.d // 32) and x["vs"].shape == (1, 1, 3, w.d // 32)
