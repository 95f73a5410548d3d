"""CPU tests of the C ABI: the library loads, exports every function the header declares,
validates descriptors on the host (gemm_create makes no HIP call) and reports the
schedule; its FastDivmod constants equal the oracle's for every divisor below 2^16."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from gemm_epilogue_persistent_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from gemm_epilogue_persistent_amd import build
        build.build()
    return _abi.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gemm_mi355x.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(gemm_[a-z_]+)\s*\(", text, flags=re.M))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gemm_create", "gemm_run", "gemm_run_ex", "gemm_destroy", "gemm_run_logged", "gemm_run_dynamic",
            "gemm_plan_grid",
            "gemm_fastdivmod_params", "gemm_fastdivmod_check", "gemm_status_string",
            "gemm_last_error"} <= names
    for n in names:
        assert hasattr(lib, n), n


def base_desc(**kw):
    d = _abi.GemmDesc()
    d.M, d.N, d.K, d.L = 256, 256, 256, 1
    d.a = d.b = _abi.DT["bf16"]
    d.d = _abi.DT["bf16"]
    d.lda = d.ldb = 256
    d.ldd = 256
    d.alpha, d.beta = 1.0, 1.0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def create(lib, d):
    h = ctypes.c_void_p()
    st = lib.gemm_create(ctypes.byref(d), ctypes.byref(h))
    if st == _abi.OK:
        lib.gemm_destroy(h)
    else:
        assert not h.value
        assert lib.gemm_last_error()  # a message explains the failure
    return st


def test_create_accepts_valid(lib):
    assert create(lib, base_desc()) == _abi.OK
    assert create(lib, base_desc(K=0)) == _abi.OK  # empty K: product is zero
    assert create(lib, base_desc(d=_abi.DT["e4m3"], post=_abi.DT["e5m2"], ldp=256)) == _abi.OK  # fp8 outputs
    assert create(lib, base_desc(M=0)) == _abi.OK  # empty output
    d = base_desc(a=_abi.DT["e4m3"], b=_abi.DT["e5m2"])
    assert create(lib, d) == _abi.OK
    d = base_desc(a_major=_abi.COL, b_major=_abi.COL, a=_abi.DT["f16"], b=_abi.DT["f16"])
    assert create(lib, d) == _abi.OK
    d = base_desc(c=_abi.DT["f32"], ldc=256, post=_abi.DT["bf16"], ldp=256, act=_abi.ACT["gelu_tanh"])
    assert create(lib, d) == _abi.OK
    # C in the other major mode than D (either way round), dact included
    assert create(lib, base_desc(c=_abi.DT["bf16"], ldc=256, c_major=_abi.COL)) == _abi.OK
    assert create(lib, base_desc(c=_abi.DT["f32"], ldc=256, d_major=_abi.COL)) == _abi.OK
    assert create(lib, base_desc(c=_abi.DT["f16"], ldc=256, c_major=_abi.COL, dact=1)) == _abi.OK
    # varlen-K: A (M, K) M-major, B (N, K) N-major, D (L, M, N); M-major D as well
    d = base_desc(varlen_k=1, L=4, a_major=_abi.COL, b_major=_abi.COL, sd=65536)
    assert create(lib, d) == _abi.OK
    assert create(lib, base_desc(varlen_k=1, L=4, sd=65536, d_major=_abi.COL)) == _abi.OK
    assert create(lib, base_desc(varlen_k=1, L=3, a=_abi.DT["e4m3"], b=_abi.DT["e5m2"], sd=65536)) == _abi.OK
    # gathered A rows: A (gather_rows, K) K-major
    assert create(lib, base_desc(varlen_m=1, L=2, sb=65536, gather_a=1, gather_rows=1000)) == _abi.OK
    assert create(lib, base_desc(varlen_m=1, L=2, sb=65536, gather_a=1, gather_rows=10, b_major=_abi.COL)) == _abi.OK
    # gathered k-rows of an M-major A (varlen-K)
    d = base_desc(varlen_k=1, L=3, sd=65536, gather_a=1, gather_rows=1000, a_major=_abi.COL, b_major=_abi.COL)
    assert create(lib, d) == _abi.OK


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), _abi.INVALID_ARG),
    (dict(K=-5), _abi.INVALID_ARG),
    (dict(a=_abi.DT["f16"]), _abi.UNSUPPORTED),  # f16 x bf16
    (dict(a=_abi.DT["e4m3"]), _abi.UNSUPPORTED),  # 8-bit x 16-bit
    (dict(a=_abi.DT["e4m3"], b=_abi.DT["e4m3"], a_major=_abi.COL), _abi.UNSUPPORTED),
    (dict(a=_abi.DT["f32"], b=_abi.DT["f32"]), _abi.UNSUPPORTED),
    (dict(a=9), _abi.INVALID_ARG),
    (dict(c=_abi.DT["e4m3"], ldc=256), _abi.UNSUPPORTED),  # fp8 C
    (dict(d=_abi.DT["e4m3"], N=264, ldd=264), _abi.ALIGNMENT),  # 264 fp8 bytes: not whole chunks
    (dict(d=0), _abi.INVALID_ARG),  # neither D nor PostAct
    (dict(act=_abi.ACT["relu"]), _abi.INVALID_ARG),  # activation without PostAct
    (dict(act=7, post=2, ldp=256), _abi.INVALID_ARG),
    (dict(a_major=3), _abi.INVALID_ARG),
    (dict(K=250, lda=256, ldb=256), _abi.ALIGNMENT),  # 500 bytes is not a multiple of 16
    (dict(lda=260), _abi.ALIGNMENT),
    (dict(lda=128), _abi.INVALID_ARG),  # leading dimension below K
    (dict(N=100, ldd=256), _abi.ALIGNMENT),
    (dict(post=_abi.DT["bf16"], ldp=256, post_major=_abi.COL), _abi.UNSUPPORTED),  # D and PostAct majors differ
    (dict(varlen_m=1, L=2, sb=65536, c=_abi.DT["bf16"], ldc=256, c_major=_abi.COL), _abi.UNSUPPORTED),
    (dict(tile_m=64, tile_n=64), _abi.UNSUPPORTED),
    (dict(lda=1 << 49), _abi.UNSUPPORTED),  # stride beyond 2^48 elements
    (dict(L=1 << 15, sa=65536, sb=65536, sd=(1 << 48) - 8), _abi.UNSUPPORTED),  # D spans 2^64 bytes
    (dict(M=1 << 30, ldd=1 << 33, K=16, lda=16), _abi.UNSUPPORTED),  # D spans 2^64 bytes
    (dict(group_m=3), _abi.INVALID_ARG),
    (dict(group_m=32), _abi.INVALID_ARG),
    (dict(xcd_remap=2), _abi.INVALID_ARG),
    (dict(tail_split=2), _abi.INVALID_ARG),
    (dict(tail_split=-2), _abi.INVALID_ARG),
    (dict(raster_order=3), _abi.INVALID_ARG),
    (dict(dact=1), _abi.INVALID_ARG),  # dact without C
    (dict(dact=1, c=2, ldc=256, beta=0.5), _abi.INVALID_ARG),  # dact takes no beta
    (dict(dact=2, c=2, ldc=256), _abi.INVALID_ARG),
    (dict(varlen_m=1, L=2, sb=65536, raster_order=2), _abi.UNSUPPORTED),
    (dict(varlen_m=1, L=2000, sb=65536), _abi.UNSUPPORTED),
    (dict(varlen_m=1, L=2, sb=65536, d_major=_abi.COL), _abi.UNSUPPORTED),
    (dict(L=2, sa=65536, sb=65536, sd=65536 + 4), _abi.ALIGNMENT),
    (dict(L=2, sa=65536, sb=65536, sd=65536 - 256), _abi.INVALID_ARG),  # D batches overlap
    (dict(varlen_k=2), _abi.INVALID_ARG),
    (dict(varlen_k=1, varlen_m=1, L=2, sb=65536), _abi.INVALID_ARG),  # exclusive modes
    (dict(varlen_k=1, L=2, sd=65536, dact=1, c=2, ldc=256, sc=65536), _abi.UNSUPPORTED),
    (dict(gather_a=1, gather_rows=10), _abi.INVALID_ARG),  # gather without varlen
    (dict(gather_a=1, gather_rows=10, varlen_k=1, L=2, sd=65536), _abi.UNSUPPORTED),  # gathered columns of a K-major A
    (dict(gather_a=1, gather_rows=300, varlen_k=1, L=2, sd=65536, a_major=_abi.COL, d_major=_abi.COL), _abi.UNSUPPORTED),
    (dict(gather_a=1, gather_rows=1 << 22, varlen_k=1, L=2, sd=65536, a_major=_abi.COL), _abi.UNSUPPORTED),  # >= 2^31 B
    (dict(gather_a=2, varlen_m=1, L=2, sb=65536), _abi.INVALID_ARG),
    (dict(gather_a=1, gather_rows=-1, varlen_m=1, L=2, sb=65536), _abi.INVALID_ARG),
    (dict(gather_a=1, gather_rows=10, varlen_m=1, L=2, sb=65536, a_major=_abi.COL), _abi.UNSUPPORTED),
    (dict(gather_a=1, gather_rows=10, varlen_m=1, L=2, sb=65536, a=4, b=4), _abi.UNSUPPORTED),  # fp8
    (dict(gather_a=1, gather_rows=1 << 23, varlen_m=1, L=2, sb=65536), _abi.UNSUPPORTED),  # >= 2^31 bytes
    (dict(gather_a=1, gather_rows=10, varlen_m=1, L=2, sb=65536, dact=1, c=2, ldc=256), _abi.UNSUPPORTED),
])
def test_create_rejects(lib, kw, status):
    assert create(lib, base_desc(**kw)) == status


def test_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.gemm_create(None, ctypes.byref(h)) == _abi.INVALID_ARG
    d = base_desc()
    assert lib.gemm_create(ctypes.byref(d), None) == _abi.INVALID_ARG
    assert lib.gemm_destroy(None) == _abi.OK
    assert lib.gemm_plan_grid(None, 256, None, None, None, None, None, None) == _abi.INVALID_ARG


def grid_of(lib, d, cus=256):
    h = ctypes.c_void_p()
    assert lib.gemm_create(ctypes.byref(d), ctypes.byref(h)) == _abi.OK
    o = [ctypes.c_int32() for _ in range(4)]
    T = ctypes.c_int64()
    P = ctypes.c_int32()
    assert lib.gemm_plan_grid(h, cus, *(ctypes.byref(x) for x in o), ctypes.byref(T), ctypes.byref(P)) == 0
    lib.gemm_destroy(h)
    return tuple(x.value for x in o) + (T.value, P.value)


def test_plan_grid(lib):
    big = base_desc(M=8192, N=8192, K=8192, lda=8192, ldb=8192, ldd=8192)
    assert grid_of(lib, big) == (256, 256, 8, 1, 1024, 256)
    small = base_desc()
    tm, tn, G, x, T, P = grid_of(lib, small)
    assert (tm, tn, T, P) == (128, 128, 4, 4)
    assert grid_of(lib, base_desc(M=8192, N=8192, K=64, lda=64, ldb=64, ldd=8192, group_m=4,
                                  max_ctas=100, xcd_remap=-1)) == (256, 256, 4, 0, 1024, 100)
    v = base_desc(varlen_m=1, L=8, M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096,
                  sb=4096 * 4096)
    assert grid_of(lib, v)[4:] == (-1, 256)
    # a 128x128 plan holds two workgroups per CU
    assert grid_of(lib, base_desc(M=2048, N=2048, K=64, lda=64, ldb=64, ldd=2048))[5] == 256


def raster_of(lib, d):
    h = ctypes.c_void_p()
    assert lib.gemm_create(ctypes.byref(d), ctypes.byref(h)) == _abi.OK
    v = ctypes.c_int32(-1)
    assert lib.gemm_plan_raster(h, ctypes.byref(v)) == _abi.OK
    lib.gemm_destroy(h)
    return v.value


def test_default_raster_order():
    """Along N only for a single dense GEMM that reads C; an explicit order always wins."""
    lib = _abi.load()
    big = dict(M=8192, N=8192, K=8192, lda=8192, ldb=8192, ldd=8192)
    assert raster_of(lib, base_desc(**big)) == 0
    assert raster_of(lib, base_desc(**big, c=_abi.DT["bf16"], ldc=8192)) == 1
    assert raster_of(lib, base_desc(**big, c=_abi.DT["bf16"], ldc=8192, raster_order=1)) == 0
    assert raster_of(lib, base_desc(**big, raster_order=2)) == 1
    assert raster_of(lib, base_desc(**big, c=_abi.DT["bf16"], ldc=8192, L=2, sa=8192 * 8192,
                                    sb=8192 * 8192, sc=8192 * 8192, sd=8192 * 8192)) == 0


def test_fastdivmod_constants_match_oracle(lib):
    m = ctypes.c_uint32()
    s = ctypes.c_uint32()
    for d in list(range(1, 1 << 16)) + [2 ** 31 - 1, 2 ** 30 + 1, 123456789]:
        assert lib.gemm_fastdivmod_params(d, ctypes.byref(m), ctypes.byref(s)) == 0
        assert (m.value, s.value) == oracle.fdm_create(d), d
    assert lib.gemm_fastdivmod_params(0, ctypes.byref(m), ctypes.byref(s)) == _abi.INVALID_ARG


def test_status_strings(lib):
    for st in range(6):
        assert lib.gemm_status_string(st)
    assert lib.gemm_status_string(99) == b"unknown status"


def test_f32_output_granularity(lib):
    """f32-only outputs need their contiguous extent in whole 16-byte chunks, i.e. a multiple
    of 4 elements (not 8): N = 260 is accepted for N-major f32 outputs and M = 260 for
    M-major ones; the kernel then stores the last 4-column half of the right-edge tile only
    where it exists. 16-bit outputs at the same extent, and f32 at 258, are rejected."""
    f32 = _abi.DT["f32"]
    assert create(lib, base_desc(N=260, d=f32, ldd=260)) == _abi.OK
    assert create(lib, base_desc(N=260, c=f32, ldc=272, d=f32, ldd=264, post=f32, ldp=260,
                                 act=_abi.ACT["relu"])) == _abi.OK
    assert create(lib, base_desc(M=260, d=f32, ldd=260, d_major=_abi.COL)) == _abi.OK
    assert create(lib, base_desc(N=260, ldd=264)) == _abi.ALIGNMENT  # bf16 D: 520 bytes
    assert create(lib, base_desc(N=260, d=f32, ldd=264, post=_abi.DT["bf16"], ldp=264)) == _abi.ALIGNMENT
    assert create(lib, base_desc(N=258, d=f32, ldd=260)) == _abi.ALIGNMENT
