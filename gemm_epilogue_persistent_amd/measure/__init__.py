"""Measurement support for the benchmark, apart from the GEMM library: the MFMA rate probe
(libmfma_probe.so, built from mfma_probe.hip), which measures the MFMA rate and clock the chip
sustains on full-entropy operands with no memory traffic."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmfma_probe.so")
_DT = {"bf16": 0, "e4m3": 1, "bf16_16x16": 2, "e4m3_16x16": 3}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with gemm_epilogue_persistent_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        lib.mfma_probe_run.restype = ctypes.c_int
        lib.mfma_probe_run.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def probe_mfma(dtype, iters, seed, blocks, out_dev, stream=None):
    """Launch the MFMA rate probe: out_dev is a device int64 tensor of 2 * blocks elements
    receiving {shader cycles, 100 MHz ticks} per workgroup. Raises ValueError for a bad
    argument and RuntimeError if the launch fails."""
    if dtype not in _DT:
        raise ValueError(f"probe dtype must be one of {sorted(_DT)}")
    s = torch.cuda.current_stream() if stream is None else stream
    rc = _load().mfma_probe_run(_DT[dtype], int(iters), int(seed) & 0xFFFFFFFF, int(blocks),
                                ctypes.c_void_p(out_dev.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    if rc == 1:
        raise ValueError("probe: iters and blocks must be positive and a buffer given")
    if rc != 0:
        raise RuntimeError("probe launch failed")
