"""gemm_run_dynamic_noalloc (the dynamic schedule on the library's own per-device counters,
for callers that cannot allocate) against gemm_run_dynamic with caller-provided counters:
the outputs must be identical bit for bit, on two calls in a row with the second smaller,
for a dense and a varlen-M problem. Both are called through the C ABI."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W
from gemm_epilogue_persistent_amd import Plan, _abi
from parity import check_close, oracle_codes, problem_of, to_dev, out_like, tol_for

pytestmark = pytest.mark.gpu


def announce(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(inp):
    """(outputs of gemm_run_dynamic_noalloc, outputs of gemm_run_dynamic) as float64 arrays."""
    lib = _abi.load()
    A, B, C = to_dev(inp.A), to_dev(inp.B), to_dev(inp.C)
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda") if inp.varlen else None
    res = []
    for noalloc in (True, False):
        D = out_like(inp, inp.d_dt) if inp.d_dt != "none" else None
        P = out_like(inp, inp.post_dt) if inp.post_dt != "none" else None
        plan = Plan(A, B, C, D, P, inp.alpha, inp.beta, inp.act, cu)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = [plan.handle, _p(A), _p(B), _p(C), _p(D), _p(P), None, None, _p(cu)]
        if noalloc:
            st = lib.gemm_run_dynamic_noalloc(*args, stream)
        else:
            ctr = torch.zeros(8, dtype=torch.int32, device="cuda")
            st = lib.gemm_run_dynamic(*args, _p(ctr), None, 0, stream)
        assert st == _abi.OK, lib.gemm_last_error()
        torch.cuda.synchronize()
        if not noalloc:
            assert (ctr.cpu() == 0).all()
        res.append(tuple(None if x is None else x.double().cpu().numpy() for x in (D, P)))
    return res


def check(inp):
    (d0, p0), (d1, p1) = both(inp)
    for a, b in ((d0, d1), (p0, p1)):
        if a is not None:
            assert np.isfinite(a).all()
            assert np.array_equal(a, b)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    if d0 is not None:
        check_close(d0, pre, tol, rms, "D")
    if p0 is not None:
        check_close(p0, post, tol, rms, "PostAct")


def dense(M, N, K, seed):
    A = W.normal(seed, (1, M, K), "bf16", 0.5)
    B = W.normal(seed + 1, (1, N, K), "bf16", 0.5)
    C = W.normal(seed + 2, (1, M, N), "bf16")
    return W.Inputs("noalloc_dense", M, N, K, 1, "bf16", "bf16", A, B, C=C, c_dt="bf16", d_dt="bf16",
                    post_dt="bf16", alpha=0.5, beta=0.25, act="gelu_tanh")


def varlen(sizes, N, K, seed):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G, M = len(sizes), int(cu[-1])
    A = W.normal(seed, (M, K), "bf16", 0.5)
    B = W.normal(seed + 1, (G, N, K), "bf16", 0.5)
    return W.Inputs("noalloc_varlen", M, N, K, G, "bf16", "bf16", A, B, post_dt="bf16", act="silu",
                    cu_seqlens=cu)


def test_noalloc_dense_twice_second_smaller():
    # first call: more tiles than one round of the grid (several claims per queue)
    announce("noalloc dense 4360x4104x200, then 520x392x136")
    check(dense(4360, 4104, 200, 3000))
    check(dense(520, 392, 136, 3010))


def test_noalloc_varlen_twice_second_smaller():
    announce("noalloc varlen, then a smaller one")
    check(varlen([1000, 0, 3000, 129, 2048, 700], 1304, 72, 3020))
    check(varlen([0, 300, 5], 264, 64, 3030))
