"""CPU oracle for D = act(alpha * A x B + beta * C): test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the GPU library and never calls it.

Every function follows a plain definition (see oracle.c for the passages cited):
exact decode of the stored codes, a k-ascending fp64 dot product per output, alpha then
beta*C then the activation on the unrounded value, round-to-nearest-even to the output type,
and a tile map computed with '/' and '%'.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"none": 0, "f16": 1, "bf16": 2, "f32": 3, "e4m3": 4, "e5m2": 5}
ACTS = {"none": 0, "relu": 1, "relu_sq": 2, "gelu_tanh": 3, "silu": 4}
_CODE_NP = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32, "e4m3": np.uint8,
            "e5m2": np.uint8}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("L", ctypes.c_int64),
        ("a_dt", ctypes.c_int32), ("b_dt", ctypes.c_int32), ("c_dt", ctypes.c_int32),
        ("a_kmajor", ctypes.c_int32), ("b_kmajor", ctypes.c_int32), ("c_nmajor", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("sa", ctypes.c_int64), ("sb", ctypes.c_int64), ("sc", ctypes.c_int64),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
        ("has_c", ctypes.c_int32), ("act", ctypes.c_int32), ("varlen", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("dact", ctypes.c_int32),
        ("varlen_k", ctypes.c_int32),
        ("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32)),
        ("a_idx", ctypes.POINTER(ctypes.c_int32)),
        ("a_rows", ctypes.c_int64),
    ]


_ERRORS = {-1: "cu_seqlens must start at 0, never decrease and end at M",
           -2: "cu_seqlens_k must start at 0, never decrease and end at most at K",
           -3: "requested output coordinates lie outside the output"}


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_decode.restype = ctypes.c_double
        lib.orc_decode.argtypes = [ctypes.c_int, ctypes.c_uint32]
        lib.orc_encode.restype = ctypes.c_uint32
        lib.orc_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        lib.orc_act.restype = ctypes.c_double
        lib.orc_act.argtypes = [ctypes.c_int, ctypes.c_double]
        lib.orc_dact.restype = ctypes.c_double
        lib.orc_dact.argtypes = [ctypes.c_int, ctypes.c_double]
        vp = ctypes.c_void_p
        for name in ("orc_gemm_points", "orc_gemm_rows"):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, ctypes.c_int64, vp, vp, vp,
                          ctypes.c_int]
        lib.orc_gemm_all.restype = ctypes.c_int
        lib.orc_gemm_all.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp, vp, ctypes.c_int]
        lib.orc_encode_array.restype = None
        lib.orc_encode_array.argtypes = [ctypes.c_int, ctypes.c_int64, vp, vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.orc_raster.restype = None
        lib.orc_raster.argtypes = [ctypes.c_int64] * 4 + [i64p, i64p]
        lib.orc_tile_dense.restype = None
        lib.orc_tile_dense.argtypes = [ctypes.c_int64] * 4 + [i64p, i64p, i64p]
        lib.orc_tile_dense_n.restype = None
        lib.orc_tile_dense_n.argtypes = [ctypes.c_int64] * 4 + [i64p, i64p, i64p]
        lib.orc_tile_varlen.restype = None
        lib.orc_tile_varlen.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)] + \
            [ctypes.c_int64] * 4 + [i64p, i64p, i64p]
        lib.orc_wg_tile.restype = ctypes.c_int64
        lib.orc_wg_tile.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.orc_fdm_create.restype = None
        lib.orc_fdm_create.argtypes = [ctypes.c_uint32, u32p, u32p]
        lib.orc_fdm_divmod.restype = None
        lib.orc_fdm_divmod.argtypes = [ctypes.c_uint32] * 4 + [u32p, u32p]
        lib.orc_fdm_exhaustive.restype = ctypes.c_uint64
        lib.orc_fdm_exhaustive.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                           ctypes.c_int]
        lib.orc_fdm_edges.restype = ctypes.c_uint64
        lib.orc_fdm_edges.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        lib.orc_fdm_random.restype = ctypes.c_uint64
        lib.orc_fdm_random.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _lib = lib
    return _lib


def lib_path() -> str:
    return _LIB_PATH


# ---------------------------------------------------------------------------------------
# scalar helpers
# ---------------------------------------------------------------------------------------

def decode(dtype: str, code: int) -> float:
    return _load().orc_decode(DTYPES[dtype], int(code))


def decode_array(dtype: str, codes) -> np.ndarray:
    codes = np.asarray(codes).ravel()
    f = _load().orc_decode
    d = DTYPES[dtype]
    return np.array([f(d, int(c)) for c in codes], dtype=np.float64)


def encode(dtype: str, x: float) -> int:
    return int(_load().orc_encode(DTYPES[dtype], float(x)))


def encode_array(dtype: str, x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=_CODE_NP[dtype])
    _load().orc_encode_array(DTYPES[dtype], x.size, x.ctypes.data, out.ctypes.data)
    return out


def act(name: str, x: float) -> float:
    return _load().orc_act(ACTS[name], float(x))


def dact(name: str, x: float) -> float:
    """act'(x), the factor the activation-backward epilogue applies to the incoming gradient."""
    return _load().orc_dact(ACTS[name], float(x))


# ---------------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------------

class Problem:
    """Description of one GEMM for the oracle; operands are numpy arrays of stored codes
    (uint16 for f16/bf16, uint8 for fp8, uint32 for f32), flat, addressed by the strides."""

    def __init__(self, M, N, K, L, a_dt, b_dt, a_kmajor=True, b_kmajor=True, lda=None, ldb=None,
                 sa=0, sb=0, c_dt="none", c_nmajor=True, ldc=None, sc=0, alpha=1.0, beta=1.0,
                 act="none", cu_seqlens=None, dact=False, cu_seqlens_k=None, a_idx=None,
                 a_rows=None):
        """Varlen-K: cu_seqlens_k (L+1 entries) splits K into groups, A (M, K) and B (N, K)
        have no batch index, K is A's and B's total K extent. a_idx (varlen-M or varlen-K
        only): the A row of each global output row, or the A column of each global k;
        a_rows: the number of rows (varlen-M) or columns (varlen-K) of A an index may name
        (an index outside [0, a_rows) reads zeros). Invalid cu_seqlens / cu_seqlens_k raise
        ValueError when the problem is evaluated."""
        assert a_idx is None or a_rows is not None, "a gathered A needs its row (column) count"
        assert cu_seqlens is None or cu_seqlens_k is None, "varlen in M or in K, not both"
        assert a_idx is None or cu_seqlens is not None or cu_seqlens_k is not None, \
            "gathered A needs varlen-M or varlen-K"
        self.M, self.N, self.K, self.L = M, N, K, L
        self.dact = bool(dact)
        assert not self.dact or c_dt != "none", "the activation-backward epilogue reads C"
        self.a_dt, self.b_dt, self.c_dt = a_dt, b_dt, c_dt
        self.a_kmajor, self.b_kmajor, self.c_nmajor = a_kmajor, b_kmajor, c_nmajor
        self.lda = lda if lda is not None else (K if a_kmajor else M)
        self.ldb = ldb if ldb is not None else (K if b_kmajor else N)
        self.ldc = ldc if ldc is not None else (N if c_nmajor else M)
        self.sa, self.sb, self.sc = sa, sb, sc
        self.alpha, self.beta, self.act = alpha, beta, act
        self.cu_seqlens = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        self.cu_seqlens_k = None if cu_seqlens_k is None else np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
        self.a_idx = None if a_idx is None else np.ascontiguousarray(a_idx, dtype=np.int32)
        self.a_rows = 0 if a_rows is None else int(a_rows)

    def _struct(self):
        s = _Problem()
        s.M, s.N, s.K, s.L = self.M, self.N, self.K, self.L
        s.a_dt, s.b_dt, s.c_dt = DTYPES[self.a_dt], DTYPES[self.b_dt], DTYPES[self.c_dt]
        s.a_kmajor, s.b_kmajor, s.c_nmajor = int(self.a_kmajor), int(self.b_kmajor), int(self.c_nmajor)
        s.lda, s.ldb, s.ldc = self.lda, self.ldb, self.ldc
        s.sa, s.sb, s.sc = self.sa, self.sb, self.sc
        s.alpha, s.beta = float(self.alpha), float(self.beta)
        s.has_c = int(self.c_dt != "none")
        s.act = ACTS[self.act]
        s.varlen = int(self.cu_seqlens is not None)
        s.dact = int(self.dact)
        if self.cu_seqlens is not None:
            assert len(self.cu_seqlens) == self.L + 1
            s.cu_seqlens = self.cu_seqlens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        s.varlen_k = int(self.cu_seqlens_k is not None)
        if self.cu_seqlens_k is not None:
            assert len(self.cu_seqlens_k) == self.L + 1
            s.cu_seqlens_k = self.cu_seqlens_k.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        if self.a_idx is not None:
            s.a_idx = self.a_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        s.a_rows = self.a_rows
        return s

    @staticmethod
    def _ptr(a):
        if a is None:
            return None
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data

    def points(self, A, B, C, pts, nthreads=0):
        """pre, post (fp64) at (l, m, n) triples; for varlen, m is the global row."""
        pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
        pre = np.empty(len(pts)); post = np.empty(len(pts))
        s = self._struct()
        _check(_load().orc_gemm_points(ctypes.byref(s), self._ptr(A), self._ptr(B), self._ptr(C),
                                len(pts), pts.ctypes.data, pre.ctypes.data, post.ctypes.data,
                                nthreads))
        return pre, post

    def rows(self, A, B, C, rows, nthreads=0):
        """pre, post (fp64) of whole rows given as (l, m) pairs: shape [nrows, N]."""
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
        pre = np.empty((len(rows), self.N)); post = np.empty((len(rows), self.N))
        s = self._struct()
        _check(_load().orc_gemm_rows(ctypes.byref(s), self._ptr(A), self._ptr(B), self._ptr(C),
                              len(rows), rows.ctypes.data, pre.ctypes.data, post.ctypes.data,
                              nthreads))
        return pre, post

    def all(self, A, B, C, nthreads=0):
        """pre, post (fp64): [L, M, N], or [M, N] over global rows in varlen-M mode."""
        shape = (self.M, self.N) if self.cu_seqlens is not None else (self.L, self.M, self.N)
        pre = np.empty(shape); post = np.empty(shape)
        s = self._struct()
        _check(_load().orc_gemm_all(ctypes.byref(s), self._ptr(A), self._ptr(B), self._ptr(C),
                             pre.ctypes.data, post.ctypes.data, nthreads))
        return pre, post


def problem_from(inp, act=None, alpha=None, beta=None):
    """Problem for a workload description (duck-typed: M, N, K, a_dt, b_dt, A, B, C, c_dt,
    alpha, beta, act, cu_seqlens, with A / B / C torch views whose strides give the layout)."""
    A, B = inp.A, inp.B
    varlen = inp.cu_seqlens is not None
    cu_k = getattr(inp, "cu_seqlens_k", None)
    a_idx = getattr(inp, "a_idx", None)
    if varlen or cu_k is not None:  # A is (rows, K) with no batch index
        a_k = A.stride(1) == 1
        lda = A.stride(0) if a_k else A.stride(1)
        sa = 0
        L = B.shape[0] if varlen else len(cu_k) - 1
    else:
        a_k = A.stride(2) == 1
        lda = A.stride(1) if a_k else A.stride(2)
        sa, L = A.stride(0), A.shape[0]
    if cu_k is not None:  # B is (N, K) with no batch index
        b_k = B.stride(1) == 1
        ldb = B.stride(0) if b_k else B.stride(1)
        sb = 0
    else:
        b_k = B.stride(2) == 1
        ldb = B.stride(1) if b_k else B.stride(2)
        sb = B.stride(0)
    kw = {}
    if inp.C is not None:
        C = inp.C if inp.C.dim() == 3 else inp.C.unsqueeze(0)
        c_n = C.stride(2) == 1
        kw = dict(c_dt=inp.c_dt, c_nmajor=c_n, ldc=C.stride(1) if c_n else C.stride(2),
                  sc=0 if varlen else C.stride(0))
    a_rows = None
    if a_idx is not None:  # the rows (varlen-M) or columns (varlen-K) an index may name
        a_rows = A.shape[0] if varlen else A.shape[1]
    return Problem(inp.M, inp.N, inp.K, L, inp.a_dt, inp.b_dt, a_kmajor=a_k, b_kmajor=b_k,
                   lda=lda, ldb=ldb, sa=sa, sb=sb, a_rows=a_rows,
                   alpha=inp.alpha if alpha is None else alpha,
                   beta=inp.beta if beta is None else beta,
                   act=inp.act if act is None else act, cu_seqlens=inp.cu_seqlens,
                   dact=getattr(inp, "dact", False), cu_seqlens_k=cu_k, a_idx=a_idx, **kw)


# ---------------------------------------------------------------------------------------
# tile map and fast divmod
# ---------------------------------------------------------------------------------------

def raster(r, tm, tn, G):
    m = ctypes.c_int64(); n = ctypes.c_int64()
    _load().orc_raster(r, tm, tn, G, ctypes.byref(m), ctypes.byref(n))
    return m.value, n.value


def tile_dense(t, tm, tn, G, along_n=False):
    m = ctypes.c_int64(); n = ctypes.c_int64(); l = ctypes.c_int64()
    f = _load().orc_tile_dense_n if along_n else _load().orc_tile_dense
    f(t, tm, tn, G, ctypes.byref(m), ctypes.byref(n), ctypes.byref(l))
    return m.value, n.value, l.value


def tile_varlen(t, cu, TM, tn, G):
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    m = ctypes.c_int64(); n = ctypes.c_int64(); l = ctypes.c_int64()
    _load().orc_tile_varlen(t, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(cu) - 1,
                            TM, tn, G, ctypes.byref(m), ctypes.byref(n), ctypes.byref(l))
    return m.value, n.value, l.value


def wg_tile(b, i, P, xcd_remap):
    return int(_load().orc_wg_tile(b, i, P, int(xcd_remap)))


def tile_count_dense(M, N, L, TM, TN):
    return -(-M // TM) * -(-N // TN) * L


def tile_count_varlen(cu, TM, TN, N):
    tn = -(-N // TN)
    return sum(-(-(int(cu[g + 1]) - int(cu[g])) // TM) * tn for g in range(len(cu) - 1))


def tile_schedule(P, T, tile_fn, xcd_remap):
    """Expected per-workgroup sequence: list over b of [(m, n, l), ...] for t = b' + i*P < T."""
    out = []
    for b in range(P):
        seq = []
        i = 0
        while True:
            t = wg_tile(b, i, P, xcd_remap)
            if t >= T:
                break
            seq.append(tile_fn(t))
            i += 1
        out.append(seq)
    return out


def fdm_create(d):
    m = ctypes.c_uint32(); s = ctypes.c_uint32()
    _load().orc_fdm_create(d, ctypes.byref(m), ctypes.byref(s))
    return m.value, s.value


def fdm_divmod(n, d):
    mult, shift = fdm_create(d)
    q = ctypes.c_uint32(); r = ctypes.c_uint32()
    _load().orc_fdm_divmod(n, d, mult, shift, ctypes.byref(q), ctypes.byref(r))
    return q.value, r.value


def fdm_exhaustive(d_lo, d_hi, n_count, nthreads=0):
    return int(_load().orc_fdm_exhaustive(d_lo, d_hi, n_count, nthreads))


def fdm_edges(d_lo, d_hi):
    return int(_load().orc_fdm_edges(d_lo, d_hi))


def fdm_random(count, seed):
    return int(_load().orc_fdm_random(count, seed))
