"""bench.py's host side on the CPU: its arguments, the metric name, the
roofline's byte counts and the refusal of more than one GPU (no GPU work)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attn_inputs import WORKLOADS  # noqa: E402


def test_parse_defaults(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.workload) == (1, 100, 300, bench.DEFAULT_WORKLOAD)
    assert a.key_chunk == 0 and not a.no_split and a.tau is None


def test_parse_driver_flags(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "1", "--steps", "20", "--warmup", "5",
                                      "--key-chunk", "192", "--tau", "0"])
    a = bench.parse()
    assert (a.steps, a.warmup, a.key_chunk, a.tau) == (20, 5, 192, 0.0)


def test_metric_names_the_workload():
    assert bench.metric_of(WORKLOADS["bf16_b4h16_n4096_d128"]) == \
        "attn fwd TFLOP/s, bf16 d=128 N=4096 (causal & non), % of MFMA peak"
    assert "Nq=1 Nk=32768" in bench.metric_of(WORKLOADS["bf16_b1h8_nq1_nk32768_d128"])


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_algorithmic_bytes(name):
    """Q, K, V once plus O and LSE once, against a direct count."""
    w = WORKLOADS[name]
    e = {"bf16": 2, "f32": 4, "mxfp8": 1}[w.dtype]
    per_head = w.Nq * w.d * e + 2 * w.Nk * w.d * e + w.Nq * w.d * (4 if w.dtype == "f32" else 2) + 4 * w.Nq
    if w.dtype == "mxfp8":   # one E8M0 byte per 32 x 32 block of Q, K and V
        per_head += (w.Nq // 32) * (w.d // 32) + 2 * (w.Nk // 32) * (w.d // 32)
    assert bench.algorithmic_bytes(w) == w.B * w.H * per_head


def test_roofline_bound_choice():
    """The headline launch sits far above the ridge point, a decoding step far below."""
    ridge = bench.PEAK_TFLOPS["bf16"] * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    head = WORKLOADS["bf16_b4h16_n4096_d128"]
    dec = WORKLOADS["bf16_b1h8_nq1_nk32768_d128"]
    assert bench.flops_of(head, False) / bench.algorithmic_bytes(head) > 5 * ridge
    assert bench.flops_of(dec, False) / bench.algorithmic_bytes(dec) < ridge / 100


def test_traffic_entries_name_existing_sources():
    for name, t in bench.TRAFFIC.items():
        assert name in WORKLOADS
        for rel in t["sources"]:
            assert os.path.exists(os.path.join(ROOT, rel)), rel
        b = bench.traffic_bytes(WORKLOADS[name])
        assert b is None or b > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
