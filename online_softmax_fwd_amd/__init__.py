"""Python binding of libattn.so, the gfx950 attention forward library.

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI of ``include/attn.h``. torch is used to allocate
device memory and to name the stream. There is no CPU path: if libattn.so is
missing or cannot be loaded, every call raises.

    O, LSE = fwd(q, k, v, causal=False, scale=None, exp2_mode="hw", tau=8.0)

q, k, v: contiguous CUDA (HIP) tensors [B, H, N, d], float32 or bfloat16,
or uint8 e4m3 bytes with ``q_scale``/``k_scale``/``v_scale`` E8M0 bytes
[B, H, N/32, d/32] for the MXFP8 path. O has q's dtype (bfloat16 for MXFP8);
LSE is float32 [B, H, Nq], natural log. For MXFP8, ``fp8_p`` picks how P is
cast before the PV MFMA: "block" (one E8M0 scale per 32 keys), "e4m3" or
"e5m2" (P times 2^8 with one fixed scale; tau is then bounded by the
format's range).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "fwd_split", "split_workspace_bytes", "fwd_varlen", "fwd_stats", "bwd", "mx_quantize", "mx_scale_offsets", "mx_scale_scatter", "exp2", "mix_sixteenths", "AttnError", "lib_path", "load_library",
           "ATTN_F32", "ATTN_BF16", "ATTN_MXFP8_E4M3", "ATTN_MXFP8_E4M3_PFIX_E4M3", "ATTN_MXFP8_E4M3_PFIX_E5M2",
           "EXP2_MODES", "STATUS"]

ATTN_F32, ATTN_BF16, ATTN_MXFP8_E4M3 = 0, 1, 2
ATTN_MXFP8_E4M3_PFIX_E4M3, ATTN_MXFP8_E4M3_PFIX_E5M2 = 3, 4
FP8_P = {"block": ATTN_MXFP8_E4M3, "e4m3": ATTN_MXFP8_E4M3_PFIX_E4M3, "e5m2": ATTN_MXFP8_E4M3_PFIX_E5M2}
EXP2_MODES = {"hw": 0, "emu": 1, "mix": 2, "emu4": 3, "emu5": 4}
MIX_BASE = 16
STATUS = {0: "ATTN_OK", -1: "ATTN_E_NULLPTR", -2: "ATTN_E_SHAPE", -3: "ATTN_E_HEADDIM", -4: "ATTN_E_DTYPE",
          -5: "ATTN_E_EXP2MODE", -6: "ATTN_E_TAU", -7: "ATTN_E_SCALE", -8: "ATTN_E_ALIGN", -9: "ATTN_E_HIP"}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libattn.so (built by online_softmax_fwd_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m online_softmax_fwd_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd_args = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, cf]
    lib.attn_fwd.argtypes = fwd_args
    lib.attn_fwd.restype = ci
    lib.attn_fwd_ex.argtypes = fwd_args + [ci, vp, vp, vp, vp]
    lib.attn_fwd_ex.restype = ci
    lib.attn_fwd_stats.argtypes = fwd_args + [ci, vp, vp, vp, vp, vp]
    lib.attn_fwd_split_workspace_bytes.argtypes = [ci] * 8
    lib.attn_fwd_split_workspace_bytes.restype = ctypes.c_longlong
    lib.attn_fwd_split.argtypes = fwd_args + [ci, vp, vp, vp, ci, vp, ctypes.c_longlong, vp]
    lib.attn_fwd_split.restype = ci
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, cf, ci, vp]
    lib.attn_fwd_varlen.restype = ci
    lib.attn_fwd_varlen_ex.argtypes = [vp] * 12 + [ci] * 9 + [cf, ci, cf, ci, vp]
    lib.attn_fwd_varlen_ex.restype = ci
    lib.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_longlong
    lib.attn_bwd.argtypes = [vp] * 10 + [ctypes.c_longlong, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.attn_bwd.restype = ci
    lib.attn_bwd_ex.argtypes = [vp] * 10 + [ctypes.c_longlong, ci, ci, ci, ci, ci, ci, cf, ci, vp, vp, vp, vp, vp]
    lib.attn_bwd_ex.restype = ci
    lib.attn_mx_quantize.argtypes = [vp, vp, vp, ctypes.c_longlong, ci, vp]
    lib.attn_mx_quantize.restype = ci
    lib.attn_mx_scale_offsets.argtypes = [vp, ci, ci, ci, vp, vp]
    lib.attn_mx_scale_offsets.restype = ci
    lib.attn_mx_scale_scatter.argtypes = [vp, vp, ci, vp, vp, ci, vp, ci, ci, ci, ci, vp]
    lib.attn_mx_scale_scatter.restype = ci
    lib.attn_fwd_stats.restype = ci
    lib.attn_exp2.argtypes = [vp, vp, ctypes.c_long, ci, vp]
    lib.attn_exp2.restype = ci
    lib.attn_mix_sixteenths.argtypes = [ci, ci, ci]
    lib.attn_mix_sixteenths.restype = ci
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise AttnError(rc, load_library().attn_last_error().decode())


def _mode(exp2_mode) -> int:
    if isinstance(exp2_mode, int):
        return exp2_mode
    if exp2_mode.startswith("mix") and exp2_mode[3:].isdigit():   # "mix3" = 3/16 emulated
        return MIX_BASE + int(exp2_mode[3:])
    return EXP2_MODES[exp2_mode]


def _causal(causal) -> int:
    """False/0: no mask; True/1/"top_left": key j > query i removed;
    2/"bottom_right": key j > i + Nk - Nq removed."""
    if causal in ("top_left",):
        return 1
    if causal in ("bottom_right",):
        return 2
    if isinstance(causal, (bool, int)) and int(causal) in (0, 1, 2):
        return int(causal)
    raise ValueError(f"causal={causal!r}: use False, True / 'top_left' or 'bottom_right'")


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _prepare(q, k, v, out, lse, q_scale, k_scale, v_scale, fp8_p="block"):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d]")
    if q.dtype == torch.float32:
        dtype, odt = ATTN_F32, torch.float32
    elif q.dtype == torch.bfloat16:
        dtype, odt = ATTN_BF16, torch.bfloat16
    elif q.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        if fp8_p not in FP8_P:
            raise ValueError(f"fp8_p must be one of {sorted(FP8_P)}")
        dtype, odt = FP8_P[fp8_p], torch.bfloat16
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, Nq, d) or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse has the wrong shape, dtype or layout")
    scales = [0, 0, 0]
    if dtype in FP8_P.values():
        for i, (name, s, n) in enumerate((("q_scale", q_scale, Nq), ("k_scale", k_scale, k.shape[2]),
                                          ("v_scale", v_scale, k.shape[2]))):
            if s is None or s.dtype != torch.uint8 or not s.is_contiguous() or \
                    tuple(s.shape) != (B, H, n // 32, d // 32):
                raise ValueError(f"{name} must be contiguous uint8 [B, H, N/32, d/32]")
            scales[i] = s.data_ptr()
    return dtype, out, lse, scales


def fwd(q, k, v, causal: bool = False, scale=None, exp2_mode="hw", tau: float = 8.0, out=None, lse=None,
        q_scale=None, k_scale=None, v_scale=None, stream=None, fp8_p="block"):
    """Attention forward through attn_fwd_ex. Returns (O, LSE); asynchronous on `stream`."""
    lib = load_library()
    dtype, out, lse, scales = _prepare(q, k, v, out, lse, q_scale, k_scale, v_scale, fp8_p)
    B, H, Nq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, Nq, k.shape[2], d, _causal(causal), scale, _mode(exp2_mode), float(tau),
                           dtype, scales[0], scales[1], scales[2], _stream_ptr(stream, q.device)))
    return out, lse


def split_workspace_bytes(q, k, causal=False, key_chunk: int = 0, fp8_p="block") -> int:
    """Workspace bytes attn_fwd_split needs for these tensors (0: not split)."""
    import torch
    lib = load_library()
    B, H, Nq, d = q.shape
    dtype = ATTN_F32 if q.dtype == torch.float32 else ATTN_BF16 if q.dtype == torch.bfloat16 else FP8_P[fp8_p]
    n = int(lib.attn_fwd_split_workspace_bytes(B, H, Nq, k.shape[2], d, _causal(causal), dtype, int(key_chunk)))
    if n < 0:
        raise AttnError(-2, lib.attn_last_error().decode())
    return n


def fwd_split(q, k, v, causal: bool = False, scale=None, exp2_mode="hw", tau: float = 8.0, out=None, lse=None,
              q_scale=None, k_scale=None, v_scale=None, stream=None, fp8_p="block", key_chunk: int = 0,
              workspace=None):
    """fwd through attn_fwd_split: launches with too few query tiles to fill
    the GPU are cut into key chunks run by separate workgroups and merged
    exactly. key_chunk 0 lets the library choose (no split for large
    launches); a positive multiple of 64 forces that chunk (bf16). The float32
    workspace is allocated here unless given. Returns (O, LSE)."""
    import torch
    lib = load_library()
    dtype, out, lse, scales = _prepare(q, k, v, out, lse, q_scale, k_scale, v_scale, fp8_p)
    B, H, Nq, d = q.shape
    nbytes = split_workspace_bytes(q, k, causal, key_chunk, fp8_p)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(-(-nbytes // 4), dtype=torch.float32, device=q.device)
    wptr, wbytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                      workspace.numel() * workspace.element_size())
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, Nq, k.shape[2], d, _causal(causal), scale, _mode(exp2_mode), float(tau),
                              dtype, scales[0], scales[1], scales[2], int(key_chunk), wptr, wbytes,
                              _stream_ptr(stream, q.device)))
    return out, lse


def _int32_vec(name, c, n=None):
    import torch
    if not c.is_cuda or c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor [B+1]")
    if n is not None and c.shape[0] != n:
        raise ValueError(f"{name} must have {n} entries")


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal=False, scale=None,
               exp2_mode="hw", tau: float = 8.0, out=None, lse=None, stream=None, q_scale=None, k_scale=None,
               v_scale=None, scale_offsets_q=None, scale_offsets_k=None, fp8_p="block"):
    """Packed batch of sequences of different lengths through attn_fwd_varlen_ex.

    q: [total_q, H, d], k, v: [total_k, H, d] (float32, bfloat16, or uint8 e4m3
    bytes for MXFP8; contiguous); cu_seqlens_q / cu_seqlens_k: int32 GPU
    tensors [B+1] of sequence starts. MXFP8 also takes q_scale [rows_q, H, d/32]
    and k_scale / v_scale [rows_k, H, d/32] uint8 E8M0 with each sequence's
    first scale row in scale_offsets_q / scale_offsets_k (int32 [B+1], e.g.
    from mx_scale_offsets). Returns O [total_q, H, d] (bfloat16 for MXFP8) and
    LSE [H, total_q]."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D GPU tensor [total, H, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    if q.dtype == torch.float32:
        dtype, odt = ATTN_F32, torch.float32
    elif q.dtype == torch.bfloat16:
        dtype, odt = ATTN_BF16, torch.bfloat16
    elif q.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        if fp8_p not in FP8_P:
            raise ValueError(f"fp8_p must be one of {sorted(FP8_P)}")
        dtype, odt = FP8_P[fp8_p], torch.bfloat16
    else:
        raise ValueError(f"unsupported dtype {q.dtype} for packed batches")
    total_q, H, d = q.shape
    total_k = k.shape[0]
    if k.shape[1:] != (H, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _int32_vec("cu_seqlens_q", cu_seqlens_q)
    B = cu_seqlens_q.shape[0] - 1
    _int32_vec("cu_seqlens_k", cu_seqlens_k, B + 1)
    out = torch.empty((total_q, H, d), dtype=odt, device=q.device) if out is None else out
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse has the wrong shape, dtype or layout")
    ptrs, rows = [0] * 5, [0, 0]
    if dtype in FP8_P.values():
        for i, (name, t) in enumerate((("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale))):
            if t is None or t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 3 or \
                    tuple(t.shape[1:]) != (H, d // 32):
                raise ValueError(f"{name} must be contiguous uint8 [rows, H, d/32]")
            ptrs[i] = t.data_ptr()
        if v_scale.shape != k_scale.shape:
            raise ValueError("k_scale and v_scale must have the same shape")
        for i, (name, t) in enumerate((("scale_offsets_q", scale_offsets_q), ("scale_offsets_k", scale_offsets_k))):
            if t is None:
                raise ValueError(f"MXFP8 needs {name}")
            _int32_vec(name, t, B + 1)
            ptrs[3 + i] = t.data_ptr()
        rows = [q_scale.shape[0], k_scale.shape[0]]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.attn_fwd_varlen_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  ptrs[0], ptrs[1], ptrs[2], cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                  ptrs[3], ptrs[4], rows[0], rows[1], B, H, int(max_seqlen_q), total_q, total_k, d,
                                  _causal(causal), scale, _mode(exp2_mode), float(tau), dtype,
                                  _stream_ptr(stream, q.device)))
    return out, lse


def bwd(q, k, v, o, do, lse, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
        q_scale=None, k_scale=None, v_scale=None, do_scale=None):
    """Attention backward through attn_bwd_ex: (dQ, dK, dV) from dO and the
    forward pass's O and LSE. bf16: q, o, do bfloat16 [B, H, Nq, d]; k, v
    bfloat16 [B, H, Nk, d]. MXFP8: q, k, v, do uint8 e4m3 bytes with
    q_scale / k_scale / v_scale / do_scale uint8 [B, H, N/32, 4] (see
    mx_quantize), o bfloat16. lse: float32 [B, H, Nq]. dQ, dK, dV are
    bfloat16. The float32 workspace (8*B*H*Nq bytes) is allocated here unless
    given."""
    import torch
    lib = load_library()
    mx = q.dtype == torch.uint8
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.dtype != (torch.uint8 if mx else torch.bfloat16):
            raise ValueError(f"{name} must be a contiguous {'uint8' if mx else 'bfloat16'} GPU tensor [B, H, N, d]")
    if not o.is_cuda or not o.is_contiguous() or o.dtype != torch.bfloat16:
        raise ValueError("o must be a contiguous bfloat16 GPU tensor [B, H, Nq, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or o.shape != q.shape or do.shape != q.shape:
        raise ValueError("shape mismatch")
    if not lse.is_cuda or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 GPU tensor [B, H, Nq]")
    sptr = [0, 0, 0, 0]
    if mx:
        for i, (name, t, n) in enumerate((("q_scale", q_scale, Nq), ("k_scale", k_scale, Nk), ("v_scale", v_scale, Nk),
                                          ("do_scale", do_scale, Nq))):
            if t is None or t.dtype != torch.uint8 or not t.is_contiguous() or tuple(t.shape) != (B, H, n // 32, d // 32):
                raise ValueError(f"{name} must be contiguous uint8 [B, H, N/32, d/32]")
            sptr[i] = t.data_ptr()
    dq = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.bfloat16, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.bfloat16, device=q.device) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} has the wrong shape, dtype or layout")
    nbytes = int(lib.attn_bwd_workspace_bytes(B, H, Nq))
    if workspace is None:
        workspace = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), B, H, Nq, Nk, d, _causal(causal), scale,
                           ATTN_MXFP8_E4M3 if mx else ATTN_BF16, sptr[0], sptr[1], sptr[2], sptr[3],
                           _stream_ptr(stream, q.device)))
    return dq, dk, dv


def mx_quantize(x, out=None, scale=None, stream=None):
    """bf16 [..., N, 128] (N a multiple of 32) to e4m3 bytes of the same shape
    and one E8M0 byte per 32x32 block [..., N/32, 4] (attn_mx_quantize)."""
    import torch
    lib = load_library()
    if not x.is_cuda or x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous bfloat16 GPU tensor [..., N, d]")
    *lead, n, d = x.shape
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    scale = torch.empty((*lead, n // 32, d // 32), dtype=torch.uint8, device=x.device) if scale is None else scale
    if out.shape != x.shape or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if tuple(scale.shape) != (*lead, n // 32, d // 32) or scale.dtype != torch.uint8 or not scale.is_contiguous():
        raise ValueError("scale has the wrong shape, dtype or layout")
    _check(lib.attn_mx_quantize(x.data_ptr(), out.data_ptr(), scale.data_ptr(), x.numel() // d, d,
                                _stream_ptr(stream, x.device)))
    return out, scale


def mx_scale_offsets(cu_seqlens, total: int, align: int = 32, out=None, stream=None):
    """First scale row of each packed sequence (attn_mx_scale_offsets): int32
    GPU tensor [B+1]; entry B is the number of scale rows. align 32 gives the
    compact layout, 128 the padded one."""
    import torch
    lib = load_library()
    _int32_vec("cu_seqlens", cu_seqlens)
    B = cu_seqlens.shape[0] - 1
    out = torch.empty(B + 1, dtype=torch.int32, device=cu_seqlens.device) if out is None else out
    _int32_vec("out", out, B + 1)
    _check(lib.attn_mx_scale_offsets(cu_seqlens.data_ptr(), B, int(total), int(align), out.data_ptr(),
                                     _stream_ptr(stream, cu_seqlens.device)))
    return out


def mx_scale_scatter(src, src_offsets, dst_offsets, dst_rows: int, cu_seqlens, total: int, out=None, stream=None):
    """Copy packed MX scales [src_rows, H, d/32] into the layout given by
    dst_offsets (attn_mx_scale_scatter); padding rows get 127 (scale 1).
    Returns the [dst_rows, H, d/32] uint8 GPU tensor."""
    import torch
    lib = load_library()
    if not src.is_cuda or src.dtype != torch.uint8 or src.dim() != 3 or not src.is_contiguous():
        raise ValueError("src must be a contiguous uint8 GPU tensor [rows, H, d/32]")
    _int32_vec("cu_seqlens", cu_seqlens)
    B = cu_seqlens.shape[0] - 1
    _int32_vec("src_offsets", src_offsets, B + 1)
    _int32_vec("dst_offsets", dst_offsets, B + 1)
    H, w = src.shape[1], src.shape[2]
    out = torch.empty((int(dst_rows), H, w), dtype=torch.uint8, device=src.device) if out is None else out
    if tuple(out.shape) != (int(dst_rows), H, w) or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    _check(lib.attn_mx_scale_scatter(src.data_ptr(), src_offsets.data_ptr(), src.shape[0], out.data_ptr(),
                                     dst_offsets.data_ptr(), int(dst_rows), cu_seqlens.data_ptr(), B, int(total), H,
                                     32 * w, _stream_ptr(stream, src.device)))
    return out


def fwd_stats(q, k, v, causal: bool = False, scale=None, exp2_mode="hw", tau: float = 8.0,
              q_scale=None, k_scale=None, v_scale=None, stream=None, fp8_p="block"):
    """fwd plus the rescale counters: returns (O, LSE, stats[4] uint64 on the host)."""
    import torch
    lib = load_library()
    dtype, out, lse, scales = _prepare(q, k, v, None, None, q_scale, k_scale, v_scale, fp8_p)
    B, H, Nq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = torch.zeros(4, dtype=torch.int64, device=q.device)
    _check(lib.attn_fwd_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, Nq, k.shape[2], d, _causal(causal), scale, _mode(exp2_mode), float(tau),
                              dtype, scales[0], scales[1], scales[2], st.data_ptr(),
                              _stream_ptr(stream, q.device)))
    return out, lse, st.cpu().tolist()


def exp2(x, exp2_mode="emu", out=None, stream=None):
    """The kernels' device exp2 applied to a float32 GPU tensor."""
    import torch
    lib = load_library()
    if not x.is_cuda or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    y = torch.empty_like(x) if out is None else out
    _check(lib.attn_exp2(x.data_ptr(), y.data_ptr(), x.numel(), _mode(exp2_mode), _stream_ptr(stream, x.device)))
    return y


def mix_sixteenths(dtype: int, d: int, causal: bool) -> int:
    return load_library().attn_mix_sixteenths(dtype, d, int(bool(causal)))
