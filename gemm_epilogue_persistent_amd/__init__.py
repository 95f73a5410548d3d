"""Python binding of the MI355X GEMM-with-epilogue library (argument marshalling only).

    D       = alpha * A x B + beta * C
    PostAct = act(alpha * A x B + beta * C)

Every step runs in the HIP kernels of libgemm_mi355x.so, reached through its C ABI
(include/gemm_mi355x.h); torch supplies device memory and the current stream. There is no
fallback path: if the library is missing, importing the binding's entry points raises.

Tensors follow the wrapper convention of quack-kernels (0.1.10 -> 0.2.0 diff, page 5,
quack/dense_gemm_sm90.py, gemm_sm90): A (l, m, k), B (l, n, k), C / D / PostAct (l, m, n),
with the major mode of each read from its strides; 2-D tensors mean l = 1. In varlen-M
mode (cu_seqlens_m given) A is (M, K), B is (G, N, K), C / D / PostAct are (M, N); with
a_idx (gathered A) A is (rows, K) and output row r reads A row a_idx[r]. In varlen-K mode
(cu_seqlens_k given; the same pages' grouped K) A is (M, K), B is (N, K) and C / D /
PostAct are (G, M, N), group g summing k over [cu_seqlens_k[g], cu_seqlens_k[g+1]); with
a_idx, A is M-major (M, cols) and global k reads A column a_idx[k].
"""
import ctypes

import torch

from . import _abi
from ._abi import GemmError, DT, ACT, ROW, COL

_TORCH_DT = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32",
             torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2"}

__all__ = ["Plan", "gemm", "gemm_dact", "gemm_create", "gemm_run", "plan_grid", "configs", "tune", "fastdivmod_params",
           "fastdivmod_check", "check_cu_seqlens", "tuned_config", "GemmError", "library_path"]


def library_path():
    return _abi.LIB_PATH


def _dt(t):
    if t is None:
        return "none"
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}")


def _as3(t):
    return None if t is None else (t if t.dim() == 3 else t.unsqueeze(0))


def _major_ld(t, first_major_name):
    """(major, ld) of a (.., X, Y) tensor: ROW if Y is contiguous, else COL if X is.
    Zero-element tensors have no meaningful strides: they are described as packed rows."""
    if t.numel() == 0:
        return ROW, t.shape[-1]
    if t.stride(-1) == 1 and (t.shape[-2] <= 1 or t.stride(-2) >= t.shape[-1] or t.stride(-2) != 1):
        return ROW, (t.stride(-2) if t.shape[-2] > 1 else max(t.shape[-1], 1))
    if t.stride(-2) == 1:
        return COL, (t.stride(-1) if t.shape[-1] > 1 else max(t.shape[-2], 1))
    raise ValueError(f"{first_major_name}: one of the last two dimensions must be contiguous")


def _bstride(t):
    return t.stride(0) if (t.dim() == 3 and t.shape[0] > 1 and t.numel() > 0) else 0


def describe(A, B, C=None, D=None, PostAct=None, alpha=1.0, beta=1.0, act="none",
             varlen=False, tile=None, group_m=0, max_ctas=0, xcd_remap=0,
             tail_split=0, raster_order=0, dact=False, varlen_k=0, gather=False):
    """Build the gemm_desc for these tensors (no GPU work). varlen_k: the number of K groups
    (len(cu_seqlens_k) - 1), or 0. gather: A rows are read through a_idx (varlen-M)."""
    d = _abi.GemmDesc()
    if varlen_k:
        M, K = A.shape
        N, K2 = B.shape
        if gather:  # gathered k-rows: A's K extent is its own; the groups index B's K
            K = K2
        L = varlen_k
        A3, B3 = A.unsqueeze(0), B.unsqueeze(0)
        C3, D3, P3 = (_as3(x) for x in (C, D, PostAct))
        for name, x in (("C", C3), ("D", D3), ("PostAct", P3)):
            if x is not None and x.shape[0] != L:
                raise ValueError(f"{name}: expected {L} batches (one per K group)")
    elif varlen:
        rows_a, K = A.shape
        G, N, K2 = B.shape
        L = G
        out = D if D is not None else PostAct
        M = out.shape[0] if gather else rows_a
        A3, B3 = A.unsqueeze(0), B
        C3, D3, P3 = (None if x is None else x.unsqueeze(0) for x in (C, D, PostAct))
    else:
        A3, B3, C3, D3, P3 = (_as3(x) for x in (A, B, C, D, PostAct))
        L, M, K = A3.shape
        L2, N, K2 = B3.shape
        if L2 != L:
            raise ValueError("A and B batch counts differ")
    if K2 != K:
        raise ValueError("A and B disagree on K")
    for name, x in (("C", C3), ("D", D3), ("PostAct", P3)):
        if x is not None and tuple(x.shape[-2:]) != (M, N):
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected (.., {M}, {N})")
    d.M, d.N, d.K, d.L = M, N, K, L
    d.a, d.b, d.c, d.d, d.post = (DT[_dt(x)] for x in (A, B, C, D, PostAct))
    d.a_major, d.lda = _major_ld(A3, "A")
    d.b_major, d.ldb = _major_ld(B3, "B")
    d.sa, d.sb = (0 if (varlen or varlen_k) else _bstride(A3)), (0 if varlen_k else _bstride(B3))
    for x, mf, lf, sf in ((C3, "c_major", "ldc", "sc"), (D3, "d_major", "ldd", "sd"),
                          (P3, "post_major", "ldp", "sp")):
        if x is not None:
            mj, ld = _major_ld(x, mf)
            setattr(d, mf, mj)
            setattr(d, lf, ld)
            setattr(d, sf, 0 if varlen else _bstride(x))
    d.alpha, d.beta = float(alpha), float(beta)
    d.act = ACT[act]
    d.varlen_m = int(varlen)
    if tile is not None:
        d.tile_m, d.tile_n = tile
    d.group_m, d.max_ctas, d.xcd_remap, d.tail_split = group_m, max_ctas, xcd_remap, tail_split
    d.raster_order = raster_order
    d.dact = 1 if dact else 0
    d.varlen_k = 1 if varlen_k else 0
    d.gather_a = 1 if gather else 0
    d.gather_rows = (A.shape[1] if varlen_k else A.shape[0]) if gather else 0
    return d


def gemm_create(desc):
    lib = _abi.load()
    h = ctypes.c_void_p()
    _abi.check(lib.gemm_create(ctypes.byref(desc), ctypes.byref(h)))
    return h


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Plan:
    """A validated plan for one problem shape (host memory; reusable across calls).
    cu_seqlens_k / a_idx select varlen-K / gathered A (their values are read at run time;
    only their presence and, for varlen-K, the group count matter to the plan)."""

    def __init__(self, A, B, C=None, D=None, PostAct=None, alpha=1.0, beta=1.0, act="none",
                 cu_seqlens_m=None, cu_seqlens_k=None, a_idx=None, **tuning):
        self.varlen = cu_seqlens_m is not None
        self.varlen_k = cu_seqlens_k is not None
        self.gather = a_idx is not None
        self.desc = describe(A, B, C, D, PostAct, alpha, beta, act, self.varlen, **tuning,
                             varlen_k=(cu_seqlens_k.numel() - 1) if self.varlen_k else 0,
                             gather=self.gather)
        self.handle = gemm_create(self.desc)
        self._lib = _abi.load()

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self._lib.gemm_destroy(h)
            self.handle = None

    def run(self, A, B, C=None, D=None, PostAct=None, alpha_dev=None, beta_dev=None,
            cu_seqlens_m=None, stream=None, tile_log=None, max_iters=0, tile_counters=None,
            cu_seqlens_k=None, a_idx=None):
        """Enqueue on `stream` (default: torch's current stream). alpha_dev / beta_dev:
        optional fp32 device tensors of one element, read by the kernel. tile_counters: an
        int32 device tensor of 8 zeros selects the dynamic schedule (gemm_run_dynamic; the
        kernel leaves it zero again). Varlen-K and gathered-A plans run through gemm_run_ex
        with cu_seqlens_k / a_idx (int32 device tensors)."""
        if tile_counters is not None:
            if tile_counters.dtype != torch.int32 or tile_counters.numel() < 8 or not tile_counters.is_cuda:
                raise ValueError("tile_counters: int32 device tensor of at least 8 elements")
        for name, x in (("cu_seqlens_m", cu_seqlens_m), ("cu_seqlens_k", cu_seqlens_k), ("a_idx", a_idx)):
            if x is not None and (x.dtype != torch.int32 or not x.is_cuda or not x.is_contiguous()):
                raise ValueError(f"{name}: contiguous int32 device tensor expected")
        if self.varlen_k or self.gather:
            if tile_log is not None:
                raise ValueError("the tile log is not offered for varlen-K / gathered-A plans")
            a = _abi.GemmArgs()
            a.A, a.B, a.C, a.D, a.PostAct = (None if t is None else t.data_ptr() for t in (A, B, C, D, PostAct))
            a.alpha_dev, a.beta_dev = (None if t is None else t.data_ptr() for t in (alpha_dev, beta_dev))
            a.cu_seqlens_m, a.cu_seqlens_k, a.a_idx, a.tile_counters = (
                None if t is None else t.data_ptr() for t in (cu_seqlens_m, cu_seqlens_k, a_idx, tile_counters))
            _abi.check(self._lib.gemm_run_ex(self.handle, ctypes.byref(a), _stream(stream)))
            return
        args = [self.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(PostAct), _ptr(alpha_dev),
                _ptr(beta_dev), _ptr(cu_seqlens_m)]
        if tile_counters is not None:
            st = self._lib.gemm_run_dynamic(*args, _ptr(tile_counters), _ptr(tile_log), int(max_iters),
                                            _stream(stream))
        elif tile_log is not None:
            st = self._lib.gemm_run_logged(*args, _ptr(tile_log), int(max_iters), _stream(stream))
        else:
            st = self._lib.gemm_run(*args, _stream(stream))
        _abi.check(st)

    def run_noalloc(self, A, B, C=None, D=None, PostAct=None, alpha_dev=None, beta_dev=None,
                    cu_seqlens_m=None, stream=None):
        """Enqueue with the dynamic schedule on the library's own per-device counters
        (gemm_run_dynamic_noalloc): no device memory is allocated by the call. Calls that
        may overlap on one GPU race on those counters."""
        _abi.check(self._lib.gemm_run_dynamic_noalloc(self.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                                      _ptr(PostAct), _ptr(alpha_dev), _ptr(beta_dev),
                                                      _ptr(cu_seqlens_m), _stream(stream)))

    def grid(self, num_cus=None):
        """(tile_m, tile_n, group_m, xcd_remap, tiles, grid) for a device with num_cus CUs."""
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(0).multi_processor_count
        out = [ctypes.c_int32() for _ in range(4)]
        T = ctypes.c_int64()
        P = ctypes.c_int32()
        _abi.check(self._lib.gemm_plan_grid(self.handle, int(num_cus), *(ctypes.byref(o) for o in out),
                                            ctypes.byref(T), ctypes.byref(P)))
        return tuple(o.value for o in out) + (T.value, P.value)

    def raster_along_n(self):
        """True when the plan's tile map rasters along N (gemm_plan_raster)."""
        v = ctypes.c_int32()
        _abi.check(self._lib.gemm_plan_raster(self.handle, ctypes.byref(v)))
        return bool(v.value)


def gemm(A, B, D=None, C=None, PostAct=None, alpha=1.0, beta=1.0, act="none", cu_seqlens_m=None,
         alpha_dev=None, beta_dev=None, stream=None, cu_seqlens_k=None, a_idx=None, autotune=False, **tuning):
    """One-shot call: plan (validated on the host) and enqueue. Outputs are written in place.
    autotune=True (dense and varlen-M plans): the configuration tune() found fastest for this
    problem signature, timed once per process and cached (see tuned_config)."""
    if autotune and not tuning and cu_seqlens_k is None and a_idx is None:
        tuning = tuned_config(A, B, C, D, PostAct, alpha, beta, act, cu_seqlens_m)
    p = Plan(A, B, C, D, PostAct, alpha, beta, act, cu_seqlens_m, cu_seqlens_k, a_idx, **tuning)
    p.run(A, B, C, D, PostAct, alpha_dev, beta_dev, cu_seqlens_m, stream, cu_seqlens_k=cu_seqlens_k,
          a_idx=a_idx)
    return D if D is not None else PostAct


def gemm_dact(A, B, PreAct, D, PostAct=None, act="none", alpha=1.0, cu_seqlens_m=None, alpha_dev=None,
              stream=None, **tuning):
    """Activation backward (page 6, gemm_dact_sm90): D = (alpha * A x B) * act'(PreAct) and,
    if given, PostAct = act(PreAct). Outputs are written in place; returns D."""
    p = Plan(A, B, PreAct, D, PostAct, alpha, 1.0, act, cu_seqlens_m, dact=True, **tuning)
    p.run(A, B, PreAct, D, PostAct, alpha_dev, None, cu_seqlens_m, stream)
    return D


gemm_run = Plan.run
plan_grid = Plan.grid


def configs(varlen=False):
    """The tuning space on MI355X: the page 6 quack/gemm_config.py space (tile shape, raster
    order, swizzle size) with this library's tiles (256x256 with one workgroup per CU, 128x128
    with two), the raster group size G in {1, 2, 4, 8, 16}, the raster order (along N is dense
    only) and the XCD remap on or off. Every configuration computes the same bits."""
    out = []
    for tile in ((256, 256), (128, 128)):
        for g in (1, 2, 4, 8, 16):
            for raster in ((1,) if varlen else (1, 2)):
                for xcd in (1, -1):
                    out.append(dict(tile=tile, group_m=g, raster_order=raster, xcd_remap=xcd))
    return out


def tune(A, B, C=None, D=None, PostAct=None, alpha=1.0, beta=1.0, act="none", cu_seqlens_m=None,
         candidates=None, steps=10, warmup=3):
    """Time each candidate configuration (default: configs()) on these operands through
    gemm_run on the current stream and return (fastest tuning dict, [(ms, tuning), ...] sorted).
    The outputs are overwritten by the runs."""
    cands = candidates if candidates is not None else configs(cu_seqlens_m is not None)
    stream = torch.cuda.current_stream()
    timed = []
    for tun in cands:
        p = Plan(A, B, C, D, PostAct, alpha, beta, act, cu_seqlens_m, **tun)
        for _ in range(warmup):
            p.run(A, B, C, D, PostAct, None, None, cu_seqlens_m)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            p.run(A, B, C, D, PostAct, None, None, cu_seqlens_m)
        end.record(stream)
        end.synchronize()
        timed.append((start.elapsed_time(end) / steps, tun))
    timed.sort(key=lambda x: x[0])
    return timed[0][1], timed


_TUNED = {}


def _signature(A, B, C, D, PostAct, act, cu_seqlens_m):
    """What a configuration's speed depends on: shapes, strides, types, epilogue kind and, for
    varlen-M, the group sizes (the tile count and balance follow from them)."""
    sig = [act, None if cu_seqlens_m is None else tuple(cu_seqlens_m.tolist())]
    for t in (A, B, C, D, PostAct):
        sig.append(None if t is None else (tuple(t.shape), tuple(t.stride()), str(t.dtype)))
    return tuple(sig)


def tuned_config(A, B, C=None, D=None, PostAct=None, alpha=1.0, beta=1.0, act="none", cu_seqlens_m=None,
                 candidates=None, steps=10, warmup=3):
    """The fastest configuration for this problem signature: timed with tune() on the first call
    (the outputs are overwritten then), looked up afterwards. Every configuration computes the
    same bits, so the choice changes only the speed."""
    key = _signature(A, B, C, D, PostAct, act, cu_seqlens_m)
    if key not in _TUNED:
        best, _ = tune(A, B, C, D, PostAct, alpha, beta, act, cu_seqlens_m, candidates, steps, warmup)
        _TUNED[key] = best
    return dict(_TUNED[key])


def fastdivmod_params(d):
    lib = _abi.load()
    m = ctypes.c_uint32()
    s = ctypes.c_uint32()
    _abi.check(lib.gemm_fastdivmod_params(d, ctypes.byref(m), ctypes.byref(s)))
    return m.value, s.value


def fastdivmod_check(d_lo, d_hi, n_count, bad_dev, stream=None):
    """Enqueue the device FastDivmod self-check; adds mismatches to bad_dev (uint64)."""
    lib = _abi.load()
    _abi.check(lib.gemm_fastdivmod_check(d_lo, d_hi, n_count, _ptr(bad_dev), _stream(stream)))


def check_cu_seqlens(cu, total, exact_end=True, stream=None):
    """Enqueue the library's cu_seqlens check (gemm_check_cu_seqlens) and return a one-element
    int32 device tensor: 0 if valid, else 1 + the index of the first bad entry."""
    if cu.dtype != torch.int32 or not cu.is_cuda or not cu.is_contiguous():
        raise ValueError("cu: contiguous int32 device tensor expected")
    status = torch.empty(1, dtype=torch.int32, device=cu.device)
    _abi.check(_abi.load().gemm_check_cu_seqlens(_ptr(cu), cu.numel() - 1, int(total), int(bool(exact_end)),
                                                 _ptr(status), _stream(stream)))
    return status
