"""GPU parity of the grouped modes added to the persistent GEMM: variable-length K (grouped K,
one output batch per group) and gathered A (varlen-M reading A rows, varlen-K reading A columns
through an index).

Small cases span several tiles with ragged M / N and ragged or empty K groups, every major
mode, both tiles, 16-bit and fp8 inputs, C with beta, activations and M-major outputs; they are
compared element by element with the CPU oracle. Small integers must match exactly. The
dynamic schedule must reproduce the static one bit for bit. The grouped workloads run at
full size with sampled outputs.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W
from gemm_epilogue_persistent_amd import GemmError, Plan, _abi
from parity import check_close, oracle_codes, problem_of, run_hip, tol_for
from test_gpu_parity import full_size

pytestmark = pytest.mark.gpu


def announce(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


def a2(M, K, m_major, seed, dt, gen=W.uniform, **kw):
    """Logical (M, K): storage [M][K] (K-major) or [K][M] (M-major)."""
    if m_major:
        return gen(seed, (K, M), dt, **kw).t()
    return gen(seed, (M, K), dt, **kw)


def varlen_k_small(sizes, M=264, N=392, dt="bf16", a_mmaj=False, b_nmaj=False, c_dt="none",
                   act="none", beta=1.0, alpha=1.0, post=False, seed=0, gen=W.uniform, fp8=None):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    K = int(cu[-1])
    G = len(sizes)
    if fp8:
        A, sa = W.quantize_fp8(1200 + seed, (M, K), fp8[0])
        B, sb = W.quantize_fp8(1201 + seed, (N, K), fp8[1])
        alpha = sa * sb
        a_dt, b_dt = fp8
    else:
        A = a2(M, K, a_mmaj, 1200 + seed, dt, gen)
        B = a2(N, K, b_nmaj, 1201 + seed, dt, gen)
        a_dt = b_dt = dt
    C = gen(1202 + seed, (G, M, N), c_dt) if c_dt != "none" else None
    return W.Inputs("varlen_k_small", M, N, K, G, a_dt, b_dt, A, B, C=C, c_dt=c_dt, d_dt="bf16",
                    post_dt="bf16" if post else "none", act=act, alpha=alpha, beta=beta,
                    cu_seqlens_k=cu)


def compare(inp, tile=None, d_major_m=False, **kw):
    announce(f"{inp.name} M={inp.M} N={inp.N} K={inp.K} L={inp.L} tile={tile} mmaj_out={d_major_m} "
             f"cu_k={None if inp.cu_seqlens_k is None else inp.cu_seqlens_k.tolist()} "
             f"gather={inp.a_idx is not None} {kw}")
    d, p, _ = run_hip(inp, d_major_m=d_major_m, tile=tile, **kw)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    if d is not None:
        check_close(d, pre, tol, rms, "D")
    if p is not None:
        check_close(p, post, tol, rms, "PostAct")
    return d, p, pre, post


# ---------------------------------------------------------------------------------------
# varlen-K
# ---------------------------------------------------------------------------------------

# K-major operands need every group to start on a 16-byte chunk (multiples of 8 16-bit
# elements); M/N-major operands take any split
SIZES_ALIGNED = [[64, 0, 200, 8, 520], [0, 0, 136], [1024], [72, 64, 0]]
SIZES_ANY = [[5, 0, 131, 1, 77], [0, 300], [3, 3, 3, 200]]


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("a_mmaj,b_nmaj", [(False, False), (True, False), (False, True), (True, True)])
def test_varlen_k_small_majors(tile, a_mmaj, b_nmaj):
    sets = SIZES_ALIGNED + (SIZES_ANY if (a_mmaj and b_nmaj) else [])
    for i, sizes in enumerate(sets):
        compare(varlen_k_small(sizes, a_mmaj=a_mmaj, b_nmaj=b_nmaj, seed=i), tile=tile)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_varlen_k_f16_epilogue_and_m_major_out(tile):
    inp = varlen_k_small([40, 0, 296], dt="f16", a_mmaj=True, b_nmaj=True, c_dt="f32", beta=-0.5,
                         act="gelu_tanh", post=True, alpha=0.75, seed=5)
    compare(inp, tile=tile)
    compare(inp, tile=tile, d_major_m=False)
    inp2 = varlen_k_small([40, 0, 296], dt="f16", a_mmaj=True, b_nmaj=False, seed=6)
    compare(inp2, tile=tile, d_major_m=True)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("fmt", [("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_varlen_k_fp8(tile, fmt):
    # fp8 operands are K-major: groups start on 16-element chunks
    compare(varlen_k_small([128, 0, 48, 336], fp8=fmt, seed=7), tile=tile)


def test_varlen_k_small_integers_exact():
    def ints(seed, shape, dt):
        r = np.random.Generator(np.random.PCG64(seed))
        return torch.from_numpy(r.integers(-3, 4, size=shape).astype(np.float64)).to(W.TORCH_DT[dt])
    for a_mmaj, b_nmaj in ((False, False), (True, True)):
        inp = varlen_k_small([64, 0, 136, 320], a_mmaj=a_mmaj, b_nmaj=b_nmaj, gen=ints, seed=8)
        inp.d_dt = "f32"
        d, _, _ = run_hip(inp)
        pre, _ = problem_of(inp).all(*oracle_codes(inp))
        assert np.array_equal(d, pre)


def test_varlen_k_dynamic_equals_static():
    inp = varlen_k_small([640, 8, 0, 1024, 72], M=1040, N=1296, a_mmaj=True, b_nmaj=True, seed=9,
                         gen=W.normal)
    d0, _, _ = run_hip(inp)
    ctr = torch.zeros(8, dtype=torch.int32, device="cuda")
    for _ in range(2):
        d1, _, _ = run_hip(inp, tile_counters=ctr)
        assert np.array_equal(d0, d1)
        assert (ctr.cpu() == 0).all()


def test_varlen_k_rejected_by_the_plain_entry_points():
    inp = varlen_k_small([64, 64])
    A, B = inp.A.cuda(), inp.B.cuda()
    D = torch.empty((2, inp.M, inp.N), dtype=torch.bfloat16, device="cuda")
    cuk = torch.from_numpy(inp.cu_seqlens_k).cuda()
    plan = Plan(A, B, None, D, None, cu_seqlens_k=cuk)
    lib = _abi.load()
    st = lib.gemm_run(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()), None,
                      ctypes.c_void_p(D.data_ptr()), None, None, None, None, None)
    assert st == _abi.INVALID_ARG
    with pytest.raises(GemmError):
        plan.run(A, B, None, D, None)  # no cu_seqlens_k
    plan.run(A, B, None, D, None, cu_seqlens_k=cuk)
    torch.cuda.synchronize()
    assert torch.isfinite(D.float()).all()


# ---------------------------------------------------------------------------------------
# gathered A rows (varlen-M)
# ---------------------------------------------------------------------------------------

def gather_small(sizes, rows_a=301, N=264, K=200, dt="bf16", b_nmaj=False, seed=0, bad=False,
                 act="silu"):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(cu[-1]), len(sizes)
    r = np.random.Generator(np.random.PCG64(1300 + seed))
    idx = r.integers(0, rows_a, size=M).astype(np.int32)
    A = W.uniform(1301 + seed, (rows_a, K), dt)
    B = W.make_b(W.uniform, G, N, K, b_nmaj, 1302 + seed, dt)
    inp = W.Inputs("gather_small", M, N, K, G, dt, dt, A, B, d_dt="bf16", post_dt="bf16", act=act,
                   cu_seqlens=cu, a_idx=idx)
    if bad and M > 3:
        # indices outside [0, rows_a) read zeros (the oracle's own reading)
        idx[[0, M // 2, M - 1]] = [-1, rows_a, 1 << 30]
    return inp



@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("b_nmaj", [False, True])
@pytest.mark.parametrize("sizes", [[0, 300, 0, 1, 129, 0], [256, 256, 256], [5], [384, 0, 513, 128, 1, 255]])
def test_gather_small(tile, b_nmaj, sizes):
    inp = gather_small(sizes, b_nmaj=b_nmaj, seed=len(sizes))
    announce(f"gather tile={tile} b_nmaj={b_nmaj} sizes={sizes}")
    d, p, _ = run_hip(inp, tile=tile)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    check_close(d, pre, 2e-2, 1e-2, "D")
    check_close(p, post, 2e-2, 1e-2, "PostAct")


def test_gather_out_of_range_indices_read_zero():
    inp = gather_small([40, 200, 77], bad=True, seed=3, act="none")
    d, _, _ = run_hip(inp)
    pre, _ = problem_of(inp).all(*oracle_codes(inp))  # the oracle reads zero rows there
    check_close(d, pre, 2e-2, 1e-2, "D")
    for r in (0, inp.M // 2, inp.M - 1):
        assert (d[r] == 0).all()


def test_gather_identity_equals_plain_varlen():
    sizes = [136, 0, 264, 16]
    inp = W.varlen_moe(G=4, N=264, K=200, sizes=sizes)
    d_plain, p_plain, _ = run_hip(inp)
    inp.a_idx = np.arange(inp.M, dtype=np.int32)
    d_g, p_g, _ = run_hip(inp)
    assert np.array_equal(p_plain, p_g)


# ---------------------------------------------------------------------------------------
# gathered A columns (varlen-K)
# ---------------------------------------------------------------------------------------

def gather_k_small(sizes, M=264, N=392, cols_a=333, b_nmaj=True, seed=0, bad=False, c=False):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    K, G = int(cu[-1]), len(sizes)
    r = np.random.Generator(np.random.PCG64(1400 + seed))
    idx = r.integers(0, cols_a, size=max(K, 1)).astype(np.int32)[:K]
    A = W.uniform(1401 + seed, (cols_a, M), "bf16").t()  # (M, cols_a), M-major
    B = a2(N, K, b_nmaj, 1402 + seed, "bf16")
    C = W.uniform(1403 + seed, (G, M, N), "f32") if c else None
    if bad and K > 3:
        idx[[0, K // 2, K - 1]] = [-1, cols_a, 1 << 30]
    return W.Inputs("gather_k_small", M, N, K, G, "bf16", "bf16", A, B, C=C, c_dt="f32" if c else "none",
                    d_dt="bf16", beta=0.5, cu_seqlens_k=cu, a_idx=idx)



@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("b_nmaj", [True, False])
@pytest.mark.parametrize("sizes", [[64, 0, 200, 8, 520], [0, 0, 136], [1024], [72, 64, 0]])
def test_gather_k_small(tile, b_nmaj, sizes):
    inp = gather_k_small(sizes, b_nmaj=b_nmaj, seed=len(sizes), c=len(sizes) == 3)
    announce(f"gather-k tile={tile} b_nmaj={b_nmaj} sizes={sizes}")
    d, _, _ = run_hip(inp, tile=tile)
    pre, _ = problem_of(inp).all(*oracle_codes(inp))
    check_close(d, pre, 2e-2, 1e-2, "D")


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_gather_k_any_split_and_bad_indices(tile):
    # an N-major B takes group boundaries at any k; out-of-range indices read zero columns
    inp = gather_k_small([5, 0, 131, 1, 77], bad=True, seed=9)
    announce(f"gather-k bad indices tile={tile}")
    d, _, _ = run_hip(inp, tile=tile)
    pre, _ = problem_of(inp).all(*oracle_codes(inp))  # the oracle reads zero columns there
    check_close(d, pre, 2e-2, 1e-2, "D")


def test_gather_k_identity_equals_plain_varlen_k():
    inp = varlen_k_small([64, 0, 200, 8, 520], a_mmaj=True, b_nmaj=True, seed=11)
    d_plain, _, _ = run_hip(inp)
    inp.a_idx = np.arange(inp.K, dtype=np.int32)
    d_g, _, _ = run_hip(inp)
    assert np.array_equal(d_plain, d_g)


def test_gather_k_dynamic_equals_static():
    inp = gather_k_small([640, 8, 0, 1024, 72], M=1040, N=1296, cols_a=2000, seed=12)
    d0, _, _ = run_hip(inp)
    ctr = torch.zeros(8, dtype=torch.int32, device="cuda")
    d1, _, _ = run_hip(inp, tile_counters=ctr)
    assert np.array_equal(d0, d1)


# ---------------------------------------------------------------------------------------
# the grouped workloads at full size (sampled outputs, whole rows)
# ---------------------------------------------------------------------------------------

def test_workload_varlen_k_moe():
    full_size(W.varlen_k_moe())


def test_workload_varlen_moe_gather():
    full_size(W.varlen_moe_gather(), every_tile_row=True)


def test_workload_varlen_k_moe_gather():
    full_size(W.varlen_k_moe_gather())
