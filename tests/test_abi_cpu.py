"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/attn.h declares, and rejects bad arguments before any HIP call.

No call here reaches a kernel launch: every call is either invalid (the
validation returns first) or has nothing to do (B*H*Nq == 0)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from online_softmax_fwd_amd import build, load_library
    if not os.path.exists(build.LIB_PATH):
        build.build_library(verbose=False)
    return load_library()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|long long|const char\*)\s+(attn_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names == sorted(["attn_bwd", "attn_bwd_ex", "attn_bwd_workspace_bytes", "attn_exp2", "attn_fwd",
                            "attn_fwd_ex", "attn_fwd_split", "attn_fwd_split_noalloc", "attn_fwd_split_workspace_bytes",
                            "attn_mx_quantize",
                            "attn_fwd_stats", "attn_fwd_varlen",
                            "attn_fwd_varlen_ex", "attn_last_error", "attn_mix_sixteenths",
                            "attn_mx_scale_offsets", "attn_mx_scale_scatter"])
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {lib._name}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


FAKE = 0x10000            # 16-byte aligned, never dereferenced: validation fails first
GOOD = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, B=1, H=1, Nq=128, Nk=128, d=128, causal=0,
            scale=0.088, mode=0, tau=8.0, dtype=1, qs=None, ks=None, vs=None)


def _call(lib, **kw):
    a = dict(GOOD)
    a.update(kw)
    return lib.attn_fwd_ex(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                           a["causal"], a["scale"], a["mode"], a["tau"], a["dtype"], a["qs"], a["ks"], a["vs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -4),
    (dict(B=-1), -2),
    (dict(Nk=0), -2),
    (dict(d=96), -3),
    (dict(d=256, dtype=0), -3),       # f32: d 64, 128
    (dict(d=192, dtype=2, qs=FAKE, ks=FAKE, vs=FAKE), -3),   # MXFP8: d 128
    (dict(d=320), -3),
    (dict(causal=3), -2),
    (dict(causal=-1), -2),
    (dict(scale=0.0), -7),
    (dict(scale=-1.0), -7),
    (dict(scale=float("nan")), -7),
    (dict(scale=float("inf")), -7),
    (dict(tau=-1.0), -6),
    (dict(tau=float("nan")), -6),
    (dict(tau=65.0), -6),
    (dict(mode=5), -5),
    (dict(mode=3, dtype=2, qs=FAKE, ks=FAKE, vs=FAKE), -5),   # degree-4/5 software exp2 is f32/bf16 only
    (dict(mode=4, dtype=4, qs=FAKE, ks=FAKE, vs=FAKE, tau=0.0), -5),
    (dict(mode=16 + 5), -5),          # no instance emulates 5/16
    (dict(mode=16 + 17), -5),
    (dict(Q=None), -1),
    (dict(LSE=None), -1),
    (dict(O=FAKE + 4), -8),
    (dict(dtype=2, Nq=100), -2),      # MXFP8 needs multiples of 32
    (dict(dtype=2), -1),              # MXFP8 needs scales
    (dict(Nq=1 << 31 - 1, B=1 << 20), -2),
    (dict(dtype=5), -4),
    (dict(dtype=3, tau=0.81), -6),    # E4M3 P times 2^8: 8 + tau must stay below log2(448) = 8.807
    (dict(dtype=3, tau=8.0), -6),
    (dict(dtype=4, tau=7.81), -6),    # E5M2 P: below log2(57344) = 15.807
    (dict(dtype=3, tau=0.5), -1),     # tau accepted; fails later on the missing MX scales
    (dict(dtype=4, tau=7.5), -1),
    (dict(dtype=3, tau=0.0, d=64), -1),
    (dict(Nk=1 << 23), -2),           # one bf16 d=128 K/V slice of 2 GiB or more
    (dict(Nq=1 << 24, d=64, dtype=0), -2),  # f32 Q slice of 4 GiB
])
def test_validation_errors(lib, kw, code):
    assert _call(lib, **kw) == code
    assert lib.attn_last_error().decode() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0), dict(Nq=0, Nk=0)])
def test_nothing_to_do_is_ok_without_touching_memory(lib, kw):
    assert _call(lib, Q=None, K=None, V=None, O=None, LSE=None, **kw) == 0


def test_attn_fwd_is_bf16_on_the_null_stream(lib):
    assert lib.attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 16, 100, 0, 0.1, 0, 8.0) == -3
    assert lib.attn_fwd(None, None, None, None, None, 0, 1, 16, 16, 64, 0, 0.1, 0, 8.0) == 0


def test_exp2_validation(lib):
    assert lib.attn_exp2(FAKE, FAKE, 10, 2, None) == -5
    assert lib.attn_exp2(FAKE, FAKE, -1, 0, None) == -2
    assert lib.attn_exp2(None, None, 0, 1, None) == 0
    assert lib.attn_exp2(None, FAKE, 5, 1, None) == -1
    assert lib.attn_exp2(FAKE + 2, FAKE, 5, 1, None) == -8
    assert lib.attn_exp2(None, None, 0, 3, None) == 0      # degree-4 and degree-5 software exp2
    assert lib.attn_exp2(None, None, 0, 4, None) == 0
    assert lib.attn_exp2(FAKE, FAKE, 10, 5, None) == -5


def test_stats_validation(lib):
    a = GOOD
    args = [a["Q"], a["K"], a["V"], a["O"], a["LSE"], 1, 1, 128, 128, 128, 0, 0.1, 0, 8.0, 1, None, None, None]
    assert lib.attn_fwd_stats(*args, None, None) == -1
    assert lib.attn_fwd_stats(*args, FAKE + 4, None) == -8


def _split_ws(lib, B=2, H=8, Nq=1024, Nk=1024, d=128, causal=1, dtype=1, key_chunk=0):
    return lib.attn_fwd_split_workspace_bytes(B, H, Nq, Nk, d, causal, dtype, key_chunk)


def _split_units(n_qt, BM, Nq, Nk, chunk, causal, diag=0):
    """Units of a split launch per head, counted the way the planner
    describes them: query tile qt needs the keys below its end (causal) or
    all Nk, cut into ceil(keys / chunk) chunks, at least one."""
    units = 0
    for qt in range(n_qt):
        kend = min(Nk, (qt + 1) * BM + diag) if causal else Nk
        units += max(1, -(-kend // chunk)) if kend > 0 else 1
    return units


def test_split_workspace_sizes(lib):
    # the library splits launches that would occupy under a quarter of the
    # 256 compute units: B2 H8 N1024 causal (128 workgroups) runs whole
    assert _split_ws(lib) == 0
    assert _split_ws(lib, B=1, H=2) > 0                      # 16 workgroups: split
    assert _split_ws(lib, key_chunk=128) == 2 * 8 * _split_units(8, 128, 1024, 1024, 128, True) * 128 * 129 * 4
    assert _split_units(8, 128, 1024, 1024, 128, True) == 36
    # explicit chunks, non-causal, ragged
    assert _split_ws(lib, B=1, H=2, Nq=300, Nk=333, causal=0, key_chunk=64) == 2 * 3 * 6 * 128 * 129 * 4
    assert _split_ws(lib, B=1, H=2, Nq=300, Nk=333, causal=1, key_chunk=64) == \
        2 * _split_units(3, 128, 300, 333, 64, True) * 128 * 129 * 4
    # d = 64 runs 256-row tiles of 64-key blocks
    assert _split_ws(lib, B=1, H=1, Nq=100, Nk=4096, d=64, causal=0, key_chunk=128) == 32 * 256 * 65 * 4
    # a launch that fills the chip is not split; nor are other dtypes or empty launches
    assert _split_ws(lib, B=4, H=16, Nq=4096, Nk=4096) == 0
    assert _split_ws(lib, dtype=0, d=64) == 0
    assert _split_ws(lib, B=0) == 0
    # rows too short to cut
    assert _split_ws(lib, B=1, H=1, Nq=64, Nk=100, causal=0) == 0
    # decoding-like: one query row, long keys
    assert _split_ws(lib, B=1, H=8, Nq=1, Nk=32768, causal=0) > 0
    # invalid input
    assert _split_ws(lib, key_chunk=100) == -1
    assert _split_ws(lib, key_chunk=-64) == -1
    assert _split_ws(lib, d=96) == -1
    assert _split_ws(lib, B=-1) == -1


def test_split_validation(lib):
    a = GOOD
    base = [a["Q"], a["K"], a["V"], a["O"], a["LSE"], 2, 8, 1024, 1024, 128, 1, 0.088, 0, 8.0, 1, None, None, None]
    need = _split_ws(lib, key_chunk=128)
    assert lib.attn_fwd_split(*base, 128, FAKE, need - 4, None) == -2       # workspace too small
    assert lib.attn_fwd_split(*base, 128, None, need, None) == -1           # no workspace
    assert lib.attn_fwd_split(*base, 128, FAKE + 4, need, None) == -8       # unaligned workspace
    assert lib.attn_fwd_split(*base, 96, FAKE, 1 << 40, None) == -2         # chunk not a multiple of 64
    assert "key_chunk" in lib.attn_last_error().decode()
    bad = list(base)
    bad[9] = 100
    assert lib.attn_fwd_split(*bad, 0, FAKE, need, None) == -3
    empty = list(base)
    empty[5] = 0
    assert lib.attn_fwd_split(*empty, 0, None, 0, None) == 0


def test_split_noalloc_validation(lib):
    """attn_fwd_split_noalloc checks everything attn_fwd_split checks, and an
    explicit chunk whose partials exceed its 64 MiB scratch, before it
    touches a device."""
    import ctypes
    fn = lib.attn_fwd_split_noalloc
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.argtypes = [vp] * 5 + [ci] * 6 + [cf, ci, cf, ci, vp, vp, vp, ci, vp]
    a = GOOD
    ptrs = [a["Q"], a["K"], a["V"], a["O"], a["LSE"]]
    # B=1 H=64 Nq=128 Nk=16384 cut into 64-key chunks: 64 * 256 partial slots of 128 x 129 floats
    assert _split_ws(lib, B=1, H=64, Nq=128, Nk=16384, causal=0, key_chunk=64) == 64 * 256 * 128 * 129 * 4
    assert fn(*ptrs, 1, 64, 128, 16384, 128, 0, 0.088, 0, 8.0, 1, None, None, None, 64, None) == -2
    assert "scratch" in lib.attn_last_error().decode()
    assert fn(*ptrs, 1, 64, 128, 16384, 128, 0, 0.088, 0, 8.0, 1, None, None, None, 96, None) == -2
    assert fn(*ptrs, 1, 64, 128, 16384, 100, 0, 0.088, 0, 8.0, 1, None, None, None, 0, None) == -3
    assert fn(None, None, None, None, None, 1, 64, 0, 16384, 128, 0, 0.088, 0, 8.0, 1, None, None, None, 0,
              None) == 0


def test_mix_table(lib):
    for dtype in (0, 1, 2, 3, 4):
        for d in (64, 128):
            for causal in (0, 1):
                k = lib.attn_mix_sixteenths(dtype, d, causal)
                assert 0 <= k <= 16
    for d in (192, 256):                       # bf16 only
        assert 0 <= lib.attn_mix_sixteenths(1, d, 1) <= 16
        assert lib.attn_mix_sixteenths(0, d, 1) < 0
    assert lib.attn_mix_sixteenths(1, 96, 0) < 0
    assert lib.attn_mix_sixteenths(9, 128, 0) < 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import online_softmax_fwd_amd as attn
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd(x, x, x)


def _varlen(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, cq=FAKE, ck=FAKE, B=2, H=4, maxq=100, tq=150, tk=170,
             d=128, causal=0, scale=0.088, mode=0, tau=8.0, dtype=1)
    a.update(kw)
    return lib.attn_fwd_varlen(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["cq"], a["ck"], a["B"], a["H"],
                               a["maxq"], a["tq"], a["tk"], a["d"], a["causal"], a["scale"], a["mode"], a["tau"],
                               a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -4),              # packed batches take f32 or bf16
    (dict(dtype=3), -4),
    (dict(B=-1), -2),
    (dict(tq=-5), -2),
    (dict(maxq=200), -2),             # longer than the whole packed Q
    (dict(d=96), -3),
    (dict(causal=3), -2),
    (dict(scale=0.0), -7),
    (dict(tau=-1.0), -6),
    (dict(mode=99), -5),
    (dict(cq=None), -1),
    (dict(ck=None), -1),
    (dict(cq=FAKE + 2), -8),
    (dict(O=FAKE + 4), -8),
    (dict(tq=1 << 22, maxq=1 << 20), -2),   # packed Q of 2 GiB or more
])
def test_varlen_validation_errors(lib, kw, code):
    assert _varlen(lib, **kw) == code
    assert lib.attn_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(maxq=0), dict(tq=0, maxq=0)])
def test_varlen_nothing_to_do(lib, kw):
    assert _varlen(lib, Q=None, K=None, V=None, O=None, LSE=None, cq=None, ck=None, **kw) == 0


def _varlen_ex(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=FAKE, qs=FAKE, ks=FAKE, vs=FAKE, cq=FAKE, ck=FAKE, sq=FAKE,
             sk=FAKE, rq=10, rk=12, B=2, H=4, maxq=100, tq=150, tk=170, d=128, causal=0, scale=0.088, mode=0,
             tau=0.0, dtype=2)
    a.update(kw)
    return lib.attn_fwd_varlen_ex(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["qs"], a["ks"], a["vs"], a["cq"],
                                  a["ck"], a["sq"], a["sk"], a["rq"], a["rk"], a["B"], a["H"], a["maxq"], a["tq"],
                                  a["tk"], a["d"], a["causal"], a["scale"], a["mode"], a["tau"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -4),
    (dict(d=64), -3),                 # MXFP8 is d = 128 only
    (dict(rq=-1), -2),
    (dict(qs=None), -1),
    (dict(vs=None), -1),
    (dict(sk=None), -1),
    (dict(ks=FAKE + 2), -8),          # scale and offset pointers 4-byte aligned
    (dict(sq=FAKE + 1), -8),
    (dict(tau=1.0, dtype=3), -6),     # fixed-scale E4M3 P: 8 + tau < log2(448)
    (dict(maxq=200), -2),
    (dict(dtype=1, d=96), -3),        # bf16 keeps its own checks
    (dict(dtype=1, cq=None), -1),
])
def test_varlen_ex_validation_errors(lib, kw, code):
    assert _varlen_ex(lib, **kw) == code
    assert lib.attn_last_error()


def test_varlen_ex_ignores_scales_for_bf16(lib):
    # bf16 with NULL scale arguments passes validation; nothing to do (B = 0)
    assert _varlen_ex(lib, dtype=1, qs=None, ks=None, vs=None, sq=None, sk=None, rq=-1, rk=-1, B=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(total=-1), -2), (dict(align=48), -2), (dict(align=0), -2), (dict(align=8192), -2),
    (dict(cu=None), -1), (dict(off=None), -1), (dict(off=FAKE + 2), -8),
    (dict(B=1 << 28, align=4096), -2),       # row count could overflow int32
])
def test_mx_scale_offsets_validation(lib, kw, code):
    a = dict(cu=FAKE, B=3, total=100, align=128, off=FAKE)
    a.update(kw)
    assert lib.attn_mx_scale_offsets(a["cu"], a["B"], a["total"], a["align"], a["off"], None) == code
    assert lib.attn_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(src_rows=-1), -2), (dict(d=64), -3), (dict(src=None), -1), (dict(cu=None), -1),
    (dict(dst=FAKE + 2), -8), (dict(dst_off=FAKE + 1), -8), (dict(dst_rows=1 << 28, H=4), -2),
])
def test_mx_scale_scatter_validation(lib, kw, code):
    a = dict(src=FAKE, src_off=FAKE, src_rows=8, dst=FAKE, dst_off=FAKE, dst_rows=16, cu=FAKE, B=3, total=100,
             H=2, d=128)
    a.update(kw)
    assert lib.attn_mx_scale_scatter(a["src"], a["src_off"], a["src_rows"], a["dst"], a["dst_off"], a["dst_rows"],
                                     a["cu"], a["B"], a["total"], a["H"], a["d"], None) == code
    assert lib.attn_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(dst_rows=0)])
def test_mx_scale_scatter_nothing_to_do(lib, kw):
    a = dict(B=3, H=2, dst_rows=16)
    a.update(kw)
    assert lib.attn_mx_scale_scatter(None, None, 8, None, None, a["dst_rows"], None, a["B"], 100, a["H"], 128,
                                     None) == 0


def _bwd(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, ws=FAKE, wsb=1 << 20,
             B=2, H=3, Nq=100, Nk=120, d=128, causal=0, scale=0.088, dtype=1)
    a.update(kw)
    return lib.attn_bwd(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"], a["ws"],
                        a["wsb"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"], None)


def test_bwd_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(2, 3, 100) == 8 * 2 * 3 * 100
    assert lib.attn_bwd_workspace_bytes(0, 3, 100) == 0
    assert lib.attn_bwd_workspace_bytes(-1, 3, 100) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), -4), (dict(dtype=2), -4),
    (dict(B=-1), -2), (dict(Nk=-1), -2), (dict(causal=3), -2), (dict(causal=-1), -2),
    (dict(d=96), -3), (dict(scale=0.0), -7), (dict(scale=float("nan")), -7),
    (dict(wsb=8 * 2 * 3 * 100 - 4), -2),          # workspace one float short
    (dict(Q=None), -1), (dict(dK=None), -1), (dict(ws=None), -1), (dict(LSE=None), -1),
    (dict(dV=FAKE + 8), -8), (dict(ws=FAKE + 4), -8),
    (dict(Nq=1 << 24, Nk=1 << 24), -2),           # a slice of 2 GiB or more
])
def test_bwd_validation_errors(lib, kw, code):
    assert _bwd(lib, **kw) == code
    assert lib.attn_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0, Nk=0)])
def test_bwd_nothing_to_do(lib, kw):
    assert _bwd(lib, Q=None, K=None, V=None, O=None, dO=None, LSE=None, dQ=None, dK=None, dV=None, ws=None,
                wsb=0, **kw) == 0


def _bwd_ex(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, ws=FAKE, wsb=1 << 20,
             B=2, H=3, Nq=96, Nk=128, d=128, causal=0, scale=0.088, dtype=2, qs=FAKE, ks=FAKE, vs=FAKE, ds=FAKE)
    a.update(kw)
    return lib.attn_bwd_ex(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"], a["ws"],
                           a["wsb"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"],
                           a["qs"], a["ks"], a["vs"], a["ds"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -4),                  # the backward pass takes the per-block MXFP8 code
    (dict(dtype=0), -4),
    (dict(d=64), -3),                     # MXFP8 is d = 128 only
    (dict(Nq=100), -2), (dict(Nk=40), -2),  # multiples of 32
    (dict(qs=None), -1), (dict(ds=None), -1), (dict(vs=None), -1),
    (dict(ks=FAKE + 2), -8), (dict(ds=FAKE + 1), -8),
    (dict(wsb=8 * 2 * 3 * 96 - 8), -2),
    (dict(dtype=1, d=192), -3),           # bf16 keeps its own checks
])
def test_bwd_ex_validation_errors(lib, kw, code):
    assert _bwd_ex(lib, **kw) == code
    assert lib.attn_last_error()


def test_bwd_ex_bf16_ignores_scales(lib):
    assert _bwd_ex(lib, dtype=1, qs=None, ks=None, vs=None, ds=None, B=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), -3), (dict(rows=33), -2), (dict(rows=-32), -2), (dict(x=None), -1), (dict(sc=None), -1),
    (dict(x=FAKE + 2), -8), (dict(q=FAKE + 8), -8),
])
def test_mx_quantize_validation(lib, kw, code):
    a = dict(x=FAKE, q=FAKE, sc=FAKE, rows=64, d=128)
    a.update(kw)
    assert lib.attn_mx_quantize(a["x"], a["q"], a["sc"], a["rows"], a["d"], None) == code
    assert lib.attn_last_error()


def test_mx_quantize_nothing_to_do(lib):
    assert lib.attn_mx_quantize(None, None, None, 0, 128, None) == 0
