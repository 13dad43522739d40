"""Helpers for the GPU tests: build-if-missing, host -> device copies of the
seeded inputs, and the comparison against the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

TOL_O = {"f32": 1e-4, "bf16": 2e-2, "mxfp8": 6e-2}   # max abs error of O vs the float64 oracle
TOL_LSE = 1e-3                                         # max abs error of LSE


def attn_module():
    from online_softmax_fwd_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build_library(verbose=False)
    import online_softmax_fwd_amd as attn
    attn.load_library()
    return attn


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x: dict):
    """Device tensors for the dict make_inputs returns."""
    import torch
    dev = torch.device("cuda", 0)
    out = {}
    if x["dtype"] == "f32":
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(dev)
    elif x["dtype"] == "bf16":
        for n in ("q", "k", "v"):
            out[n] = torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        for n in ("q", "k", "v", "qs", "ks", "vs"):
            out[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(dev)
    return out


def run_fwd(attn, dev, causal, exp2_mode, tau, scale=None, **kw):
    extra = {}
    if "qs" in dev:
        extra = dict(q_scale=dev["qs"], k_scale=dev["ks"], v_scale=dev["vs"])
    return attn.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, exp2_mode=exp2_mode, tau=tau,
                    **extra, **kw)


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)
