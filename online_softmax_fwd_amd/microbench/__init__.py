"""gfx950 issue-rate microbenchmark (measurement tool; the library does not use it).

    python -m online_softmax_fwd_amd.microbench --build   # compile (hipcc, gfx950), on any host
    python -m online_softmax_fwd_amd.microbench           # run the built binary on the GPU
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "issue_rates.hip")
BINARY = os.path.join(HERE, "issue_rates")


def build(verbose: bool = True) -> str:
    """Compile issue_rates.hip for gfx950 next to its source; always rebuilds."""
    from online_softmax_fwd_amd.build import hipcc
    cmd = [hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument", SOURCE, "-o", BINARY + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(BINARY + ".tmp", BINARY)
    if verbose:
        print(f"built {BINARY}")
    return BINARY


def run() -> int:
    if not os.path.exists(BINARY):
        raise RuntimeError(f"{BINARY} is not built: run python -m online_softmax_fwd_amd.microbench --build first")
    return subprocess.run([BINARY]).returncode
