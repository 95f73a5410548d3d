"""GPU parity at the edges of what gemm_create accepts, with guard bands around the outputs.

f32-only outputs need their contiguous extent in whole 16-byte chunks, i.e. a multiple of 4
elements: at N = 260 (N-major) or M = 260 (M-major) the right-edge tile ends half way
through a lane's 8-column group. Every output here lives inside a larger buffer prefilled
with a sentinel: 12 padding elements past each contiguous row (ld = extent + 12) and one
trailing row per batch. After the run the padding must still hold the sentinel and every
output element must match the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from parity import check_close, oracle_codes, problem_of, to_dev, tol_for

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def announce(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


def guarded(L, M, N, dt, m_major):
    """A logical (L, M, N) view into a sentinel-filled buffer with padded rows and a trailing
    guard row; returns (view, buffer, mask of the view's elements inside the buffer)."""
    rows, cols = (N, M) if m_major else (M, N)
    buf = torch.full((L, rows + 1, cols + 12), SENTINEL, dtype=W.TORCH_DT[dt], device="cuda")
    v = buf[:, :rows, :cols]
    view = v.permute(0, 2, 1) if m_major else v
    mask = np.zeros((L, rows + 1, cols + 12), dtype=bool)
    mask[:, :rows, :cols] = True
    return view, buf, mask


def run_guarded(inp, m_major, tile, dact=False):
    from gemm_epilogue_persistent_amd import Plan
    A, B, C = to_dev(inp.A), to_dev(inp.B), to_dev(inp.C)
    D, dbuf, mask = guarded(inp.L, inp.M, inp.N, inp.d_dt, m_major)
    P = pbuf = None
    if inp.post_dt != "none":
        P, pbuf, _ = guarded(inp.L, inp.M, inp.N, inp.post_dt, m_major)
    plan = Plan(A, B, C, D, P, inp.alpha, inp.beta, inp.act, tile=tile, dact=dact)
    plan.run(A, B, C, D, P)
    torch.cuda.synchronize()
    for buf in (dbuf, pbuf):
        if buf is not None:
            pad = buf.cpu().double().numpy()[~mask]
            assert (pad == SENTINEL).all(), f"{(pad != SENTINEL).sum()} guard elements overwritten"
    d = D.double().cpu().numpy()
    p = None if P is None else P.double().cpu().numpy()
    return d, p


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("m_major", [False, True])
@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_f32_outputs_ragged_half_group(tile, m_major, act):
    # the output's contiguous extent is 260 = 8 * 32 + 4 elements
    M, N = (260, 392) if m_major else (392, 260)
    L, K = 2, 136
    A = W.make_a(W.uniform, L, M, K, False, 2100, "bf16")
    B = W.make_b(W.uniform, L, N, K, m_major, 2101, "bf16")  # N-major only where N = 392
    # C with padded rows too (its own leading dimension)
    rows, cols = (N, M) if m_major else (M, N)
    cstore = W.uniform(2102, (L, rows, cols + 8), "f32")[:, :, :cols]
    C = cstore.permute(0, 2, 1) if m_major else cstore
    post = "f32" if act != "none" else "none"
    inp = W.Inputs("f32_edge", M, N, K, L, "bf16", "bf16", A, B, C=C, c_dt="f32", d_dt="f32",
                   post_dt=post, alpha=0.75, beta=-0.5, act=act)
    announce(f"f32 outputs M={M} N={N} tile={tile} m_major={m_major} act={act}")
    d, p = run_guarded(inp, m_major, tile)
    pre, postv = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    if p is not None:
        check_close(p, postv, tol, rms, "PostAct")


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_f32_dact_ragged_half_group(tile):
    M, N, K, L = 200, 260, 72, 1
    A = W.normal(2110, (L, M, K), "bf16", 0.5)
    B = W.normal(2111, (L, N, K), "bf16", 0.5)
    C = W.normal(2112, (L, M, N), "f32", 1.5)
    inp = W.Inputs("f32_dact_edge", M, N, K, L, "bf16", "bf16", A, B, C=C, c_dt="f32", d_dt="f32",
                   post_dt="f32", act="silu", dact=True)
    announce(f"f32 dact N={N} tile={tile}")
    d, p = run_guarded(inp, False, tile, dact=True)
    pre, postv = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    check_close(p, postv, tol, rms, "PostAct")


# ---------------------------------------------------------------------------------------
# malformed cu_seqlens: reported by gemm_check_cu_seqlens; the varlen-M kernels run no tile
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("cu,total,exact,want", [
    ([0, 300, 300, 557], 557, True, 0),
    ([0], 0, True, 0),
    ([1, 300, 557], 557, True, 1),        # does not start at 0
    ([0, 300, 200, 557], 557, True, 3),   # decreases at index 2
    ([0, 300, 556], 557, True, 3),        # ends short of M
    ([0, 300, 600], 557, True, 3),        # ends past M
    ([0, 64, 64, 128], 200, False, 0),    # varlen-K: may end before K
    ([0, 64, 300], 200, False, 3),        # ... but not past it
])
def test_check_cu_seqlens(cu, total, exact, want):
    from gemm_epilogue_persistent_amd import check_cu_seqlens
    st = check_cu_seqlens(torch.tensor(cu, dtype=torch.int32, device="cuda"), total, exact)
    torch.cuda.synchronize()
    assert int(st.item()) == want


@pytest.mark.parametrize("cu_bad", [[0, 300, 200, 520], [0, 256, 520 + 256], [8, 264, 520], [0, 100, 500]])
def test_varlen_bad_cu_seqlens_writes_nothing(cu_bad):
    """M = 520 rows in the plan; each array breaks a rule (decreasing, past M, not from 0, short
    of M). The output buffer holds 512 rows more than M, so that even rows addressed past M
    stay inside it: all of it must still hold the sentinel afterwards."""
    from gemm_epilogue_persistent_amd import Plan
    M, N, K = 520, 264, 64
    G = len(cu_bad) - 1
    A = W.normal(2200, (M, K), "bf16", 0.5).cuda()
    B = W.normal(2201, (G, N, K), "bf16", 0.5).cuda()
    buf = torch.full((M + 512, N), SENTINEL, dtype=torch.float32, device="cuda")
    D = buf[:M]
    cu = torch.tensor(cu_bad, dtype=torch.int32, device="cuda")
    announce(f"varlen bad cu_seqlens {cu_bad}")
    plan = Plan(A, B, None, D, None, cu_seqlens_m=cu)
    plan.run(A, B, None, D, None, cu_seqlens_m=cu)
    torch.cuda.synchronize()
    assert (buf == SENTINEL).all()


# ---------------------------------------------------------------------------------------
# C in the other major mode than D / PostAct (each operand's major from its own strides)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("d_mmaj", [False, True])
@pytest.mark.parametrize("c_dt,out_dt", [("bf16", "bf16"), ("f32", "f16"), ("f16", "f32")])
def test_c_transposed(tile, d_mmaj, c_dt, out_dt):
    from parity import run_hip
    M, N, K, L = 264, 392, 136, 2
    A = W.normal(2300, (L, M, K), "bf16", 0.5)
    B = W.normal(2301, (L, N, K), "bf16", 0.5)
    # C's contiguous dimension is the other one than the outputs'
    C = W.normal(2302, (L, M, N), c_dt) if d_mmaj else W.normal(2302, (L, N, M), c_dt).permute(0, 2, 1)
    inp = W.Inputs("c_trans", M, N, K, L, "bf16", "bf16", A, B, C=C, c_dt=c_dt, d_dt=out_dt,
                   post_dt=out_dt, alpha=0.75, beta=-1.5, act="gelu_tanh")
    announce(f"C transposed tile={tile} d_mmaj={d_mmaj} C={c_dt} out={out_dt}")
    d, p, _ = run_hip(inp, d_major_m=d_mmaj, tile=tile)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    check_close(p, post, tol, rms, "PostAct")


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_c_transposed_dact(tile):
    from parity import run_hip
    M, N, K = 200, 264, 72
    A = W.normal(2310, (1, M, K), "bf16", 0.5)
    B = W.normal(2311, (1, N, K), "bf16", 0.5)
    C = W.normal(2312, (1, N, M), "bf16", 1.5).permute(0, 2, 1)  # M-contiguous pre-activation
    inp = W.Inputs("c_trans_dact", M, N, K, 1, "bf16", "bf16", A, B, C=C, c_dt="bf16", d_dt="bf16",
                   post_dt="bf16", act="silu", dact=True)
    announce(f"C transposed dact tile={tile}")
    d, p, _ = run_hip(inp, tile=tile)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    check_close(p, post, tol, rms, "PostAct")
