"""ctypes loader for the C model of the software exp2 (ex2_emu.c; degrees 3, 4, 5).

Test infrastructure only (see the package docstring). The shared object is
built with gcc next to this file; ``build_ex2_emu()`` always rebuilds it,
and ``ex2_emu_deg3`` builds it on first use if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ex2_emu.c")
_LIB = os.path.join(_HERE, "libex2emu.so")
_handle = None


def build_ex2_emu() -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(_LIB):
            build_ex2_emu()
        h = ctypes.CDLL(_LIB)
        h.ex2_emu_deg3.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        h.ex2_emu_deg3.restype = None
        h.ex2_emu_poly.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_int]
        h.ex2_emu_poly.restype = None
        _handle = h
    return _handle


def ex2_emu_deg3(x: np.ndarray) -> np.ndarray:
    """Degree-3 emulated exp2 of a float32 array (float32 result)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _lib().ex2_emu_deg3(x.ctypes.data, y.ctypes.data, x.size)
    return y


def ex2_emu(x: np.ndarray, degree: int = 3) -> np.ndarray:
    """Emulated exp2 of a float32 array with the degree-3, -4 or -5
    polynomial (float32 result)."""
    if degree not in (3, 4, 5):
        raise ValueError(f"degree {degree} is not 3, 4 or 5")
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _lib().ex2_emu_poly(x.ctypes.data, y.ctypes.data, x.size, degree)
    return y
