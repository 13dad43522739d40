"""Pins for the P-cast simulation of the oracle (oracle/p_cast.py).

The cast is checked against torch's own bf16 / float8 conversions and the
format limits; the simulation against the rel-L2 table the page prints for
P in FP8 (and its bf16 values), averaged over eight seeded draws because the
page's own draw is not given (the printed values are one draw, to two
significant digits; seed-to-seed spread is up to 10 % on the saturated
entries)."""
import json
import os

import numpy as np
import pytest
import torch

from attn_inputs import make_score_inputs
from oracle import lagging_max_p_cast_f64, rel_l2, round_to_format

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_p_saturation.json")))
TORCH = {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
VMAX = {"bf16": 3.3895313892515355e38, "e4m3": 448.0, "e5m2": 57344.0}


@pytest.mark.parametrize("fmt", sorted(TORCH))
def test_round_to_format_matches_torch_casts(fmt):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-24, 17, 200000))
    # float32 inputs: torch narrows float64 through float32, which double-rounds
    x = x[np.abs(x) <= VMAX[fmt]].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(TORCH[fmt]).to(torch.float64).numpy()
    assert np.array_equal(round_to_format(x, fmt), ref)


def test_round_to_format_limits():
    # saturation at the largest finite value (the FP8 path's satfinite cast)
    assert round_to_format(1e6, "e4m3") == 448.0 and round_to_format(-1e6, "e4m3") == -448.0
    assert round_to_format(500.0, "e4m3") == 448.0
    assert round_to_format(1e9, "e5m2") == 57344.0
    # smallest subnormals: 2^-9 (e4m3), 2^-16 (e5m2); half of them ties to even (0)
    assert round_to_format(2.0 ** -9, "e4m3") == 2.0 ** -9
    assert round_to_format(2.0 ** -10, "e4m3") == 0.0
    assert round_to_format(1.5 * 2.0 ** -10, "e4m3") == 2.0 ** -9
    assert round_to_format(2.0 ** -16, "e5m2") == 2.0 ** -16
    # three fraction bits: 1 + 1/16 is a tie between 1 and 1.125 -> 1 (even)
    assert round_to_format(1.0625, "e4m3") == 1.0
    assert round_to_format(1.1875, "e4m3") == 1.25


def test_uncast_simulation_is_the_exact_softmax():
    s, v = make_score_inputs(1.5, 3001, rows=64, keys=1024, d=16)
    p = np.exp2(s - s.max(axis=1, keepdims=True))
    exact = (p @ v) / p.sum(axis=1, keepdims=True)
    for tau in (0.0, 4.0, 8.0):
        assert rel_l2(lagging_max_p_cast_f64(s, v, tau=tau), exact) < 1e-13


def _table_means(seeds=range(3001, 3009)):
    out = {}
    for sigma in (1.5, 6.0):
        for seed in seeds:
            s, v = make_score_inputs(sigma, seed)
            exact = lagging_max_p_cast_f64(s, v)
            for row in GOLD["table"]:
                if row["sigma"] != sigma:
                    continue
                mo = 0 if row["fmt"] == "bf16" else GOLD["max_offset"]
                err = rel_l2(lagging_max_p_cast_f64(s, v, tau=row["tau"], fmt=row["fmt"], max_offset=mo), exact)
                out.setdefault((sigma, row["fmt"], row["tau"]), []).append(err)
    return {k: float(np.mean(v)) for k, v in out.items()}


@pytest.fixture(scope="module")
def means():
    return _table_means()


@pytest.mark.parametrize("row", GOLD["table"], ids=lambda r: f"s{r['sigma']}-{r['fmt']}-tau{r['tau']}")
def test_printed_rel_l2(means, row):
    got = means[(row["sigma"], row["fmt"], row["tau"])]
    assert abs(got / row["rel_l2"] - 1.0) <= 0.12, (row, got)


def test_e4m3_saturates_and_e5m2_does_not(means):
    # E4M3's largest finite value is 448 < 2^(8+4): with max_offset 8 and tau 4
    # the cast clamps and the error grows by an order of magnitude; E5M2
    # (57344 > 2^12) keeps its tau-0 error
    for sigma in (1.5, 6.0):
        assert means[(sigma, "e4m3", 4)] > 5 * means[(sigma, "e4m3", 0)]
        assert means[(sigma, "e5m2", 4)] < 2.5 * means[(sigma, "e5m2", 0)]
    # the bound max_offset + tau < log2(max) separates the two
    assert 8 + 4 >= np.log2(448.0) and 8 + 4 < np.log2(57344.0)
