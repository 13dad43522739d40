"""Pins for the CPU model of the degree-3 software exp2 (CPU only).

The model is pinned to the error table printed on the first page (4M
inputs, float64 reference), to an exhaustive sweep of every float32
fraction in [0, 1), and to exact values the construction fixes (integers
map to exact powers of two because p(0) = 1; the clamp sends -inf to 0).
"""
import json
import os

import numpy as np
import pytest

from attn_inputs import bf16_bits
from oracle import ex2_emu_deg3


def _bf16_rne(x32):
    return bf16_bits(np.asarray(x32, dtype=np.float32))


def test_error_table_degree3(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "ex2_deg3_error_table.json")))
    lo, hi = gold["range"]
    x = np.random.default_rng(7).uniform(lo, hi, gold["inputs"]).astype(np.float32)
    y = ex2_emu_deg3(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    g = gold["degree3"]
    assert round(rel.max(), 7) == pytest.approx(g["fp32_max_rel"], abs=0.6e-7)
    assert round(rel.mean(), 7) == pytest.approx(g["fp32_mean_rel"], abs=0.6e-7)
    eb = _bf16_rne(y.astype(np.float32)).astype(np.int32)
    rb = _bf16_rne(ref.astype(np.float32)).astype(np.int32)
    same = 100.0 * np.mean(eb == rb)
    within1 = 100.0 * np.mean(np.abs(eb - rb) <= 1)
    assert same == pytest.approx(g["bf16_bit_identical_pct"], abs=0.05)
    assert within1 == g["bf16_within_1ulp_pct"]


def test_every_fraction_in_unit_interval():
    # x in [1, 2) walks every float32 fraction of that binade once; the
    # relative error depends only on the fraction, so this is the max over
    # the whole domain: the printed 8.77e-5
    x = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    y = ex2_emu_deg3(x).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert round(rel.max(), 7) == pytest.approx(8.77e-5, abs=0.6e-7)


def test_integers_are_exact_powers_of_two():
    # frac = 0 leaves p(0) = 1 exactly, so 2^n comes out exact
    n = np.arange(-126, 128, dtype=np.float32)
    assert np.array_equal(ex2_emu_deg3(n), np.exp2(n.astype(np.float64)).astype(np.float32))


def test_clamp_and_masked_scores():
    # the clamp at -127 puts -inf (a masked score) and anything below at 2^-127
    # with a zero fraction, whose bit pattern is exactly 0.0
    x = np.array([-np.inf, -1e30, -127.0, -200.0], dtype=np.float32)
    assert np.array_equal(ex2_emu_deg3(x), np.zeros(4, np.float32))


def test_tiny_negative_fraction_rounds_up_but_stays_within_table():
    # for x in [-2^-25, 0) the fraction x - floor(x) rounds to 1.0 in float32;
    # the result is then 2^-1 * p(1), still within the printed max error
    x = np.array([-2.0 ** -26, -2.0 ** -30], dtype=np.float32)
    y = ex2_emu_deg3(x).astype(np.float64)
    assert np.all(np.abs(y - 1.0) < 8.77e-5 + 1e-7)
