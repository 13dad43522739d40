"""Pins for the degree-4 and degree-5 software exp2 (CPU only).

Their coefficients are not printed on the pages, only their measured errors:
the float32 model with our fitted coefficients must reproduce that error
table (4M inputs over the softmax range, float64 reference). The fit itself
(oracle/fit_ex2_poly.py) is re-run and must give the coefficients the model
uses; the construction's exact values (integers map to exact powers of two,
the clamp sends -inf to 0) hold at every degree, and the error shrinks with
the degree as the table says.
"""
import json
import os
import re

import numpy as np
import pytest

from attn_inputs import bf16_bits
from oracle import ex2_emu, ex2_emu_deg3, fit_ex2_poly

HERE = os.path.dirname(os.path.abspath(__file__))


def _stats(y, x):
    y = y.astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    eb = bf16_bits(y.astype(np.float32)).astype(np.int32)
    rb = bf16_bits(ref.astype(np.float32)).astype(np.int32)
    return rel.max(), rel.mean(), 100.0 * np.mean(eb == rb), 100.0 * np.mean(np.abs(eb - rb) <= 1)


@pytest.mark.parametrize("degree", [4, 5])
def test_error_table(golden_dir, degree):
    gold = json.load(open(os.path.join(golden_dir, "ex2_deg45_error_table.json")))
    lo, hi = gold["range"]
    x = np.random.default_rng(7).uniform(lo, hi, gold["inputs"]).astype(np.float32)
    mx, mean, same, within1 = _stats(ex2_emu(x, degree), x)
    g = gold[f"degree{degree}"]
    # our coefficients are a fit of the same kind, not the page's own numbers:
    # the maximum within 7 %, the mean within 2 %, bf16 agreement to 0.005 points
    assert mx == pytest.approx(g["fp32_max_rel"], rel=0.07)
    assert mean == pytest.approx(g["fp32_mean_rel"], rel=0.02)
    assert same == pytest.approx(g["bf16_bit_identical_pct"], abs=0.005)
    assert within1 == g["bf16_within_1ulp_pct"]


def test_error_drops_with_degree():
    x = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)   # every fraction
    ref = np.exp2(x.astype(np.float64))
    errs = [np.abs(f(x).astype(np.float64) / ref - 1.0).max()
            for f in (ex2_emu_deg3, lambda t: ex2_emu(t, 4), lambda t: ex2_emu(t, 5))]
    assert errs[0] > 20 * errs[1] and errs[1] > 15 * errs[2]     # 8.8e-5 > 3.0e-6 > 1.5e-7
    assert errs[1] < 3.2e-6 and errs[2] < 1.6e-7
    assert np.array_equal(ex2_emu(x, 3), ex2_emu_deg3(x))


@pytest.mark.parametrize("degree", [4, 5])
def test_exact_values(degree):
    n = np.arange(-126, 128, dtype=np.float32)
    assert np.array_equal(ex2_emu(n, degree), np.exp2(n.astype(np.float64)).astype(np.float32))
    x = np.array([-np.inf, -1e30, -127.0, -200.0], dtype=np.float32)
    assert np.array_equal(ex2_emu(x, degree), np.zeros(4, np.float32))


@pytest.mark.parametrize("degree", [4, 5])
def test_model_uses_the_fitted_coefficients(degree):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "ex2_emu.c")).read()
    table = re.search(rf"kDeg{degree}\[{degree + 1}\] = \{{(.*?)\}};", src, flags=re.S).group(1)
    committed = np.array([float(t.strip().rstrip("f")) for t in table.split(",")], dtype=np.float32)
    fitted = fit_ex2_poly(degree)
    # the same float32 values (at most 2 float32 steps apart on another BLAS)
    steps = np.abs(committed.view(np.int32).astype(np.int64) - fitted.view(np.int32).astype(np.int64))
    assert steps.max() <= 2, (committed, fitted)
