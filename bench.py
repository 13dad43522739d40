#!/usr/bin/env python3
"""Attention-forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole hot path over one batch of synthetic input: for the
default workload (bf16, B=4 H=16 Nq=Nk=4096 d=128, mixed hardware/software
exp2, tau=8) a non-causal launch followed by a causal launch, each a full
pass of load -> QK^T -> mask -> lagging-max softmax -> PV -> epilogue.
Inputs are resident in HBM before timing starts. Throughput counts
4*B*H*Nq*Nk*d FLOPs per non-causal launch and half that per causal launch.

Prints ONE JSON line. Besides the contract fields it carries
  roofline      for the dominant kernel (the non-causal launch): algorithmic
                FLOPs per launch / its mean duration from HIP events recorded
                on the launch stream inside the timed region, against the
                dense MFMA peak of MI355X for the dtype (bf16 2.5 PFLOP/s);
                a launch below the ridge point (a decoding step: about one
                FLOP per byte) reports algorithmic HBM bytes (Q, K, V read
                once, O and LSE written once) per second against 8 TB/s
                instead; "traffic" is the calibrated HBM byte count per launch
                from rocprofv3 counters (null when no counter run covers these
                kernel sources)
  rescale       lagging-max rescale counts per mode, from one counting launch
                (attn_fwd_stats) outside the timed region
  backward      bf16 workloads at d 64 and 128 and the MXFP8 workload: the backward pass (attn_bwd) on the same
                inputs with the forward's O and LSE and a seeded dO, timed
                after the forward's timed region (HIP events per call on the
                launch stream); FLOPs counted as 2.5 x the forward's (the five
                products S, dP, dV, dK, dQ); not part of "value"
  cpu_baseline  the float64 oracle timed on a bounded sample of the same
                workload on the host cores (rank 0, N=1 only)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "mxfp8": 5000.0}   # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0                                              # MI355X HBM3E, published
MODE_CODES = {"hw": 0, "emu": 1, "mix": 2}
DEFAULT_WORKLOAD = "bf16_b4h16_n4096_d128"
# HBM traffic of one non-causal launch, from two rocprofv3 --pmc runs of this
# script per workload (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch,
# --calib-copy-mib 256). Calibrated on a plain 256 MiB device copy in the
# same runs: FETCH_SIZE read 131088 KiB for 262144 KiB moved (x2.0),
# WRITE_SIZE read 262144 KiB (x1.0). Valid only for the kernel sources a
# count was taken on (first 16 hex digits of their SHA-256); any edit turns
# it off.
TRAFFIC = {
    "bf16_b4h16_n4096_d128": {
        "sources": {"online_softmax_fwd_amd/csrc/attn_fwd_bf16.hip": "2cf0f9c0887dc927",
                    "online_softmax_fwd_amd/csrc/attn_fwd_bf16_kernels.h": "ed434fc3a23e1aa4",
                    "online_softmax_fwd_amd/csrc/attn_device.h": "29e06bec4380ef33",
                    "online_softmax_fwd_amd/csrc/attn_bf16_common.h": "1249699229bb3642"},
        "fetch_kib_raw": 98476.0, "fetch_scale": 2.0,
        "write_kib_raw": 66560.0, "write_scale": 1.0,
    },
    "mxfp8_b2h16_n8192_d128": {
        "sources": {"online_softmax_fwd_amd/csrc/attn_fwd_mxfp8.hip": "280fe15064e37a4a",
                    "online_softmax_fwd_amd/csrc/attn_mx_common.h": "3ff9393404d4e1ce",
                    "online_softmax_fwd_amd/csrc/attn_device.h": "29e06bec4380ef33",
                    "online_softmax_fwd_amd/csrc/attn_bf16_common.h": "1249699229bb3642"},
        "fetch_kib_raw": 53544.7, "fetch_scale": 2.0,
        "write_kib_raw": 66560.0, "write_scale": 1.0,
    },
}


def traffic_bytes(w):
    """Calibrated HBM bytes per launch of the dominant kernel, or None when no
    counter run covers this workload and these kernel sources."""
    import hashlib
    t = TRAFFIC.get(w.name)
    if t is None:
        return None
    for rel, digest in t["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    kib = t["fetch_kib_raw"] * t["fetch_scale"] + t["write_kib_raw"] * t["write_scale"]
    return int(round(kib * 1024))


def algorithmic_bytes(w) -> int:
    """HBM bytes one launch must move at the least: Q, K, V read once, O and
    LSE written once (MXFP8: one E8M0 scale byte per 32x32 block of Q, K, V)."""
    e = {"bf16": 2, "f32": 4, "mxfp8": 1}[w.dtype]
    inp = (w.Nq + 2 * w.Nk) * w.d * e
    if w.dtype == "mxfp8":
        inp += (w.Nq + 2 * w.Nk) * w.d // 1024
    out = w.Nq * w.d * (4 if w.dtype == "f32" else 2) + w.Nq * 4
    return w.B * w.H * (inp + out)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--exp2-mode", default=None, help="override the workload's exp2 mode (hw, emu, mix, mixK)")
    p.add_argument("--tau", type=float, default=None)
    p.add_argument("--fp8-p", default="block", choices=["block", "e4m3", "e5m2"],
                   help="MXFP8 workloads: P scaled per 32-key block, or times 2^8 with one fixed scale as E4M3 or E5M2")
    p.add_argument("--no-split", action="store_true",
                   help="run every launch whole (attn_fwd_ex) instead of letting the library cut small launches "
                        "into key chunks (attn_fwd_split)")
    p.add_argument("--key-chunk", type=int, default=0,
                   help="cut every bf16 launch into key chunks of this many keys (a multiple of 64; 0: the "
                        "library's choice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bwd", action="store_true", help="skip the backward-pass section")
    p.add_argument("--bwd-steps", type=int, default=50)
    p.add_argument("--bwd-warmup", type=int, default=50)
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (HBM counter calibration)")
    return p.parse_args()


def metric_of(w) -> str:
    """The metric's name for a workload: dtype, head dim, length and the
    causal settings one step runs."""
    causal = "causal & non" if len(w.causal) == 2 else ("causal" if w.causal[0] else "non-causal")
    n = f"N={w.Nq}" if w.Nq == w.Nk else f"Nq={w.Nq} Nk={w.Nk}"
    return f"attn fwd TFLOP/s, {w.dtype} d={w.d} {n} ({causal}), % of MFMA peak"


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def flops_of(w, causal: bool) -> float:
    f = 4.0 * w.B * w.H * w.Nq * w.Nk * w.d
    return f / 2 if causal else f


def cpu_baseline(w, causal_modes, flop_budget=1.2e12):
    """The float64 oracle, untuned, on the workload's (batch, head) slices, as
    many of them as fit a FLOP budget of about 10-30 s of host time (all of
    them for the default workload)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from attn_inputs import make_inputs
    from oracle import attention_f64

    per_slice = sum(4.0 * w.Nq * w.Nk * w.d for _ in causal_modes)   # the oracle forms the full S either way
    n_bh = int(min(w.B * w.H, max(1, flop_budget // per_slice)))
    if n_bh == w.B * w.H:
        x, what = make_inputs(w), f"the whole workload (B={w.B} H={w.H})"
    else:
        x, what = make_inputs(w, B=1, H=n_bh), f"{n_bh} of its {w.B * w.H} (batch, head) slices"
    flops = 0.0
    t0 = time.perf_counter()
    for causal in causal_modes:
        attention_f64(x["q64"], x["k64"], x["v64"], causal=causal)
        flops += n_bh * 4.0 * w.Nq * w.Nk * w.d / (2 if causal else 1)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what}, {f'Nq=Nk={w.Nq}' if w.Nq == w.Nk else f'Nq={w.Nq} Nk={w.Nk}'} d={w.d}, causal modes {list(causal_modes)}; float64 numpy one-shot "
                  f"softmax (it forms the full S even when causal; FLOPs counted as for the GPU); {dt:.1f} s on "
                  f"{threads} BLAS threads of {len(os.sched_getaffinity(0))} usable cores, {cpu_model()}",
        "cpu_model": cpu_model(),
        "seconds": round(dt, 2),
    }


def fwd_kernel_name(w, causal: bool, split: bool = False, hw_exp2: bool = True) -> str:
    """The kernel a launch of this workload runs (the bf16 path has a
    ping-pong kernel for d = 128 and 192, causal only with at least 256 query
    tiles of 256 rows, at d = 128 with hardware exp2 also for launches of at
    most 256 workgroups of 128 rows, with key parities; and a streaming kernel
    for everything else; a split launch runs the streaming kernel over key
    chunks, then a merge kernel). hw_exp2: the launch computes every
    exponential in hardware (exp2 mode "hw", or "mix" at 0 sixteenths)."""
    if split:
        return "fwd_bf16_stream_kernel (key chunks) + fwd_split_merge_kernel"
    if w.dtype == "bf16":
        bh = w.B * w.H
        if w.d == 128 and hw_exp2:
            if bh * -(-w.Nq // 64) <= 256:
                return "fwd_bf16_kernel (4 key parities)"
            if bh * -(-w.Nq // 128) <= 256:
                return "fwd_bf16_kernel (2 key parities)"
        pingpong = w.d in (128, 192) and ((not causal) or bh * -(-w.Nq // 256) >= 256)
        return "fwd_bf16_kernel" if pingpong else "fwd_bf16_stream_kernel"
    return f"fwd_{w.dtype}_kernel"


def bench_backward(attn, w, q, k, v, outs, stream, args, scales=None):
    import numpy as np
    import torch
    from attn_inputs import make_grad_output
    bits, _ = make_grad_output((w.B, w.H, w.Nq, w.d), w.seed + 1)
    do = torch.from_numpy(bits.view(np.int16)).to(q.device).view(torch.bfloat16)
    extra = {}
    if w.dtype == "mxfp8":  # dO in square 32x32 blocks, quantised once outside the timed calls
        do, dos = attn.mx_quantize(do, stream=stream)
        extra = dict(scales, do_scale=dos)
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.bfloat16, device=q.device) for t in (q, k, v))
    ws = torch.empty(2 * w.B * w.H * w.Nq, dtype=torch.float32, device=q.device)
    res = {}
    for c in w.causal:
        o, lse = outs[c]

        def call():
            attn.bwd(q, k, v, o, do, lse, causal=c, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream, **extra)
        for _ in range(args.bwd_warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.bwd_steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        fl = 2.5 * flops_of(w, c)
        res["causal" if c else "noncausal"] = {
            "ms_mean": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[w.dtype], 2)}
    res["flops_note"] = ("2.5 x the forward's FLOPs per call; kernels: prep, dK/dV, dQ" +
                         ("; dO quantised once outside the timed calls" if w.dtype == "mxfp8" else ""))
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the attention forward "
              f"shards over (batch, head) with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import online_softmax_fwd_amd as attn
    from attn_inputs import WORKLOADS, make_inputs

    if not os.path.exists(attn.lib_path()):
        from online_softmax_fwd_amd import build
        build.build_library(verbose=False)
    lib = attn.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = WORKLOADS[args.workload]
    mode = args.exp2_mode or w.exp2_mode
    tau = w.tau if args.tau is None else args.tau
    if w.dtype == "mxfp8" and args.fp8_p != "block" and args.tau is None:
        tau = 0.0  # a fixed-offset P admits only tau < log2(fmt max) - 8 (0.81 for E4M3, 7.81 for E5M2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    x = make_inputs(w)
    if w.dtype == "bf16":
        q, k, v = (torch.from_numpy(x[n].view(np.int16)).to(dev).view(torch.bfloat16) for n in ("q", "k", "v"))
        scales = {}
    elif w.dtype == "f32":
        q, k, v = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v"))
        scales = {}
    else:
        q, k, v = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v"))
        scales = dict(q_scale=torch.from_numpy(x["qs"]).to(dev), k_scale=torch.from_numpy(x["ks"]).to(dev),
                      v_scale=torch.from_numpy(x["vs"]).to(dev))
    del x
    fp8 = dict(fp8_p=args.fp8_p) if w.dtype == "mxfp8" else {}
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    outs = {c: (torch.empty((w.B, w.H, w.Nq, w.d), dtype=odt, device=dev),
                torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)) for c in w.causal}
    stream = torch.cuda.current_stream(dev)
    # key-split workspaces (allocated before timing; none when the library
    # runs a launch whole, as it does for launches that fill the chip)
    ws = {}
    for c in w.causal:
        n = 0 if args.no_split else attn.split_workspace_bytes(q, k, causal=c, key_chunk=args.key_chunk,
                                                               fp8_p=args.fp8_p)
        ws[c] = torch.empty(-(-n // 4), dtype=torch.float32, device=dev) if n > 0 else None

    def launch(causal):
        o, l = outs[causal]
        if args.no_split:
            attn.fwd(q, k, v, causal=causal, exp2_mode=mode, tau=tau, out=o, lse=l, stream=stream, **scales, **fp8)
        else:
            attn.fwd_split(q, k, v, causal=causal, exp2_mode=mode, tau=tau, out=o, lse=l, stream=stream,
                           key_chunk=args.key_chunk, workspace=ws[causal], **scales, **fp8)

    for _ in range(args.warmup):
        for c in w.causal:
            launch(c)
    torch.cuda.synchronize()

    # timed region: K steps; per-launch event pairs on the launch stream
    ev = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for c in w.causal}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        for c in w.causal:
            ev[c][i][0].record(stream)
            launch(c)
            ev[c][i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per = {c: [a.elapsed_time(b) for a, b in ev[c]] for c in w.causal}

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    step_flops = sum(flops_of(w, c) for c in w.causal)
    ms_per_step = total_ms / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    dom = False if False in w.causal else w.causal[0]
    dom_ms = float(np.mean(per[dom]))
    achieved = flops_of(w, dom) / (dom_ms * 1e-3) / 1e12
    per_mode = {("causal" if c else "noncausal"): {
        "ms_mean": round(float(np.mean(per[c])), 4), "ms_min": round(float(np.min(per[c])), 4),
        "ms_median": round(float(np.median(per[c])), 4),
        "tflops": round(flops_of(w, c) / (float(np.mean(per[c])) * 1e-3) / 1e12, 2),
        "pct_of_peak": round(100.0 * flops_of(w, c) / (float(np.mean(per[c])) * 1e-3) / 1e12 / peak, 2),
    } for c in w.causal}

    mix16 = None
    if mode == "mix":
        dcode = {"f32": 0, "bf16": 1, "mxfp8": 2}[w.dtype]
        mix16 = {("causal" if c else "noncausal"): lib.attn_mix_sixteenths(dcode, w.d, int(c)) for c in w.causal}
    hw_exp2 = mode == "hw" or (mode == "mix" and mix16["causal" if dom else "noncausal"] == 0)

    # The bound: matrix core when the launch's FLOPs per algorithmic byte
    # exceed the ridge point (peak FLOP/s / peak HBM B/s), else HBM.
    kname = (f"{fwd_kernel_name(w, dom, ws[dom] is not None, hw_exp2)} "
             f"(d={w.d}, {'causal' if dom else 'non-causal'})")
    abytes = algorithmic_bytes(w)
    if flops_of(w, dom) / abytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        gbs = abytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": abytes}
    roofline.update({"traffic": traffic_bytes(w), "traffic_unit": "bytes per launch (HBM read + write)"})

    result = {
        "metric": metric_of(w),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "mxfp8": "e4m3+e8m0"}[w.dtype],
        "data": "synthetic",
        "config": {
            "workload": f"attention forward {w.name}: {w.dtype} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d}, "
                        f"{' + '.join('causal' if c else 'non-causal' for c in w.causal)} per step, "
                        f"exp2 {mode}, tau={tau}",
            "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": list(w.causal),
            "exp2_mode": mode, "mix_sixteenths": mix16, "tau": tau, "seed": w.seed,
            "key_split": {("causal" if c else "noncausal"): (ws[c] is not None) for c in w.causal},
            **({"fp8_p": args.fp8_p} if w.dtype == "mxfp8" else {}),
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "per_mode": per_mode,
        "roofline": roofline,
    }
    # lagging-max rescales, one extra launch per mode outside the timed region
    rescale = {}
    for c in w.causal:
        _, _, st = attn.fwd_stats(q, k, v, causal=c, exp2_mode=mode, tau=tau, stream=stream, **scales, **fp8)
        rescale["causal" if c else "noncausal"] = {
            "row_tile_steps": st[0], "row_rescales": st[1], "wave_tile_steps": st[2], "wave_rescales": st[3],
            "row_frac": round(st[1] / max(st[0], 1), 6), "wave_frac": round(st[3] / max(st[2], 1), 6)}
    result["rescale"] = rescale
    if not args.no_bwd and ((w.dtype == "bf16" and w.d in (64, 128)) or (w.dtype == "mxfp8" and args.fp8_p == "block")):
        result["backward"] = bench_backward(attn, w, q, k, v, outs, stream, args, scales)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, w.causal)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
