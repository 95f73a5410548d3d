"""ctypes view of include/gemm_mi355x.h (argument marshalling only)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gemm_mi355x.h")

OK, INVALID_ARG, UNSUPPORTED, ALIGNMENT, HIP_ERROR, NO_MEMORY = range(6)
DT = {"none": 0, "f16": 1, "bf16": 2, "f32": 3, "e4m3": 4, "e5m2": 5}
ROW, COL = 0, 1
ACT = {"none": 0, "relu": 1, "relu_sq": 2, "gelu_tanh": 3, "silu": 4}


class GemmDesc(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("L", ctypes.c_int32),
        ("a", ctypes.c_int32), ("b", ctypes.c_int32), ("c", ctypes.c_int32), ("d", ctypes.c_int32),
        ("post", ctypes.c_int32),
        ("a_major", ctypes.c_int32), ("b_major", ctypes.c_int32), ("c_major", ctypes.c_int32),
        ("d_major", ctypes.c_int32), ("post_major", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("ldd", ctypes.c_int64), ("ldp", ctypes.c_int64),
        ("sa", ctypes.c_int64), ("sb", ctypes.c_int64), ("sc", ctypes.c_int64),
        ("sd", ctypes.c_int64), ("sp", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
        ("act", ctypes.c_int32), ("varlen_m", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("group_m", ctypes.c_int32), ("max_ctas", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
        ("tail_split", ctypes.c_int32), ("raster_order", ctypes.c_int32), ("dact", ctypes.c_int32),
        ("varlen_k", ctypes.c_int32), ("gather_a", ctypes.c_int32), ("gather_rows", ctypes.c_int64),
    ]


class GemmArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("A", "B", "C", "D", "PostAct", "alpha_dev", "beta_dev",
                                               "cu_seqlens_m", "cu_seqlens_k", "a_idx", "tile_counters")]


class GemmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load():
    """Load the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with gemm_epilogue_persistent_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        lib.gemm_create.restype = ctypes.c_int
        lib.gemm_create.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(vp)]
        lib.gemm_run.restype = ctypes.c_int
        lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gemm_run_logged.restype = ctypes.c_int
        lib.gemm_run_logged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        lib.gemm_run_dynamic.restype = ctypes.c_int
        lib.gemm_run_dynamic.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        lib.gemm_run_dynamic_noalloc.restype = ctypes.c_int
        lib.gemm_run_dynamic_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gemm_check_cu_seqlens.restype = ctypes.c_int
        lib.gemm_check_cu_seqlens.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.gemm_run_ex.restype = ctypes.c_int
        lib.gemm_run_ex.argtypes = [vp, ctypes.POINTER(GemmArgs), vp]
        lib.gemm_destroy.restype = ctypes.c_int
        lib.gemm_destroy.argtypes = [vp]
        lib.gemm_plan_grid.restype = ctypes.c_int
        lib.gemm_plan_grid.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(i64), ctypes.POINTER(i32)]
        lib.gemm_plan_raster.restype = ctypes.c_int
        lib.gemm_plan_raster.argtypes = [vp, ctypes.POINTER(i32)]
        lib.gemm_fastdivmod_params.restype = ctypes.c_int
        lib.gemm_fastdivmod_params.argtypes = [u32, ctypes.POINTER(u32), ctypes.POINTER(u32)]
        lib.gemm_fastdivmod_check.restype = ctypes.c_int
        lib.gemm_fastdivmod_check.argtypes = [u32, u32, u32, vp, vp]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_status_string.argtypes = [ctypes.c_int]
        lib.gemm_last_error.restype = ctypes.c_char_p
        lib.gemm_last_error.argtypes = []
        _lib = lib
    return _lib


def check(status):
    if status != OK:
        lib = load()
        msg = lib.gemm_last_error().decode() or lib.gemm_status_string(status).decode()
        raise GemmError(status, msg)
