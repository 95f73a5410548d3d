"""Seeded random sweep of the GPU path against the CPU oracle: each case draws a mode (dense
batched, varlen-M, varlen-K, with or without gathered A), operand types and major modes,
a tile, output types, a C term, an activation, alpha / beta and ragged sizes within the
alignment rules, runs it through the C ABI and compares every output element with the
oracle (per element |gpu - oracle| <= tol (|oracle| + 1), plus the normalised-RMS guard).
The case description is printed before each GPU call. GEP_SWEEP_CASES sets the number of
cases (default 160; case i draws from seed 9000 + i, so a larger count adds cases).
"""
import os
import sys

import numpy as np
import pytest
import torch

import workloads as W
from parity import check_close, oracle_codes, problem_of, run_hip, tol_for

pytestmark = pytest.mark.gpu

CASES = int(os.environ.get("GEP_SWEEP_CASES", "160"))


def aligned(r, lo, hi, unit):
    return int(r.integers(lo // unit, hi // unit + 1)) * unit


def draw_case(i):
    r = np.random.Generator(np.random.PCG64(9000 + i))
    mode = ["dense", "dense", "varlen_m", "varlen_k"][int(r.integers(0, 4))]
    fp8 = bool(r.random() < 0.2)
    gather = mode != "dense" and not fp8 and bool(r.random() < 0.35)
    dt = "bf16" if r.random() < 0.5 else "f16"
    a_dt = b_dt = dt
    if fp8:
        a_dt, b_dt = [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e4m3", "e4m3"), ("e5m2", "e5m2")][int(r.integers(0, 4))]
    a_mmaj = not fp8 and bool(r.random() < 0.5)
    b_nmaj = not fp8 and bool(r.random() < 0.5)
    if mode == "varlen_m":
        a_mmaj = False  # its A rows are ragged: M-contiguous storage would not be whole chunks
    if gather and mode == "varlen_k":
        a_mmaj = True
    out_dt = ["bf16", "f16", "f32", "f32"][int(r.integers(0, 4))]
    c_dt = "none" if r.random() < 0.5 else ["bf16", "f16", "f32"][int(r.integers(0, 3))]
    if c_dt != "none" and c_dt != "f32" and out_dt != "f32":
        c_dt = out_dt
    act = ["none", "relu", "relu_sq", "gelu_tanh", "silu"][int(r.integers(0, 5))]
    post = act != "none" or bool(r.random() < 0.2)
    has_d = (not post) or bool(r.random() < 0.5)
    alpha = float(r.choice([1.0, 0.5, -1.25, 2.0]))
    beta = float(r.choice([1.0, 0.5, -0.75, 0.0]))
    tile = [None, (128, 128), (256, 256)][int(r.integers(0, 3))]
    m_major_out = mode == "dense" and bool(r.random() < 0.25)
    seed = 9100 + 10 * i
    es = 1 if fp8 else 2
    kunit = 16 // es
    # M and N at the granularity gemm_create accepts: a contiguous extent holds whole
    # 16-byte chunks (4 f32, 8 16-bit elements); extents that are not contiguous anywhere
    # are free
    out_unit = max(16 // W.ELEM_BYTES[t] for t in (out_dt, c_dt) if t != "none")
    n_unit = (out_unit if not m_major_out else 1)
    if b_nmaj:
        n_unit = max(n_unit, 16 // es)
    m_unit = out_unit if m_major_out else 1
    if a_mmaj:
        m_unit = max(m_unit, 16 // es)
    M, N = aligned(r, 16, 560, m_unit), aligned(r, 16, 560, n_unit)
    k_free = mode == "dense" and a_mmaj and b_nmaj  # K contiguous in neither operand

    scales = []  # fp8: per-tensor scales, folded into alpha so outputs stay O(sqrt(K))

    def quant(s, shape, d):
        x, sc = W.quantize_fp8(s, shape, d)
        scales.append(sc)
        return x

    def make2(rows, k, mmaj, s, d):
        if d in ("e4m3", "e5m2"):
            return quant(s, (rows, k), d)
        return W.uniform(s, (k, rows), d).t() if mmaj else W.uniform(s, (rows, k), d)

    if mode == "dense":
        L = int(r.integers(1, 4))
        K = aligned(r, 0, 520, 1 if k_free else kunit) if r.random() < 0.9 else 0
        if fp8:
            K = max(K, kunit)  # per-tensor fp8 scales need a non-empty operand
        if fp8:
            A = quant(seed, (L, M, K), a_dt)
            B = quant(seed + 1, (L, N, K), b_dt)
        else:
            A = W.make_a(W.uniform, L, M, K, a_mmaj, seed, dt)
            B = W.make_b(W.uniform, L, N, K, b_nmaj, seed + 1, dt)
        C = None
        if c_dt != "none":
            C = W.uniform(seed + 2, (L, N, M), c_dt).permute(0, 2, 1) if m_major_out else W.uniform(seed + 2, (L, M, N), c_dt)
        inp = W.Inputs(f"sweep{i}", M, N, K, L, a_dt, b_dt, A, B, C=C, c_dt=c_dt)
    elif mode == "varlen_m":
        G = int(r.integers(1, 5))
        sizes = [int(x) for x in r.integers(0, 300, size=G)]
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        M = int(cu[-1])
        K = aligned(r, 16, 400, kunit)
        rows_a = M if not gather else max(1, int(r.integers(1, 400)))
        A = make2(rows_a, K, a_mmaj, seed, a_dt)
        if fp8:
            B = quant(seed + 1, (G, N, K), b_dt)
        else:
            B = W.make_b(W.uniform, G, N, K, b_nmaj, seed + 1, dt)
        C = W.uniform(seed + 2, (M, N), c_dt) if c_dt != "none" else None
        inp = W.Inputs(f"sweep{i}", M, N, K, G, a_dt, b_dt, A, B, C=C, c_dt=c_dt, cu_seqlens=cu)
        if gather:
            inp.a_idx = r.integers(0, rows_a, size=M).astype(np.int32)
    else:
        G = int(r.integers(1, 5))
        kmaj_any = (not a_mmaj) or (not b_nmaj)  # a K-major operand: groups on 16-byte chunks
        sizes = [aligned(r, 0, 300, kunit) if kmaj_any else int(r.integers(0, 300)) for _ in range(G)]
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        K = int(cu[-1])
        if K % kunit:
            K += kunit - K % kunit  # A / B hold a whole number of chunks; the groups end before
        K = max(K, kunit)
        cols_a = K if not gather else max(1, int(r.integers(1, 400)))
        A = make2(M, cols_a, a_mmaj, seed, a_dt)
        B = make2(N, K, b_nmaj, seed + 1, b_dt)
        C = W.uniform(seed + 2, (G, M, N), c_dt) if c_dt != "none" else None
        inp = W.Inputs(f"sweep{i}", M, N, K, G, a_dt, b_dt, A, B, C=C, c_dt=c_dt, cu_seqlens_k=cu)
        if gather:
            inp.a_idx = r.integers(0, cols_a, size=K).astype(np.int32)
    if scales:
        alpha = alpha * float(np.prod(scales))
    inp.d_dt = out_dt if has_d else "none"
    inp.post_dt = out_dt if post else "none"
    inp.act, inp.alpha, inp.beta = act, alpha, beta
    grouped = mode != "dense"
    # the activation-backward epilogue (C is the pre-activation), where it is built: dense or
    # varlen-M, no gathered rows, N-major outputs (drawn last, so the other draws of a case
    # do not depend on it)
    inp.dact = (mode in ("dense", "varlen_m") and not gather and c_dt != "none"
                and not (m_major_out and not grouped) and bool(r.random() < 0.35))
    if inp.dact:
        inp.beta = beta = 1.0  # beta has no role there, and the boundary asks for 1
        inp.d_dt = out_dt      # D (the gradient) is that epilogue's required output
    desc = (f"case {i}: {mode} gather={gather} {a_dt}x{b_dt} M={inp.M} N={N} K={inp.K} L={inp.L} "
            f"a_mmaj={a_mmaj} b_nmaj={b_nmaj} tile={tile} C={c_dt} D={inp.d_dt} Post={inp.post_dt} "
            f"act={act} alpha={alpha} beta={beta} m_major_out={m_major_out} dact={inp.dact}"
            + (f" cu={inp.cu_seqlens.tolist()}" if inp.cu_seqlens is not None else "")
            + (f" cu_k={inp.cu_seqlens_k.tolist()}" if inp.cu_seqlens_k is not None else ""))
    return inp, tile, m_major_out and not grouped, desc


@pytest.mark.parametrize("i", range(CASES))
def test_sweep(i):
    inp, tile, m_major_out, desc = draw_case(i)
    print(f"[case] {desc}", flush=True)
    sys.stdout.flush()
    d, p, _ = run_hip(inp, d_major_m=m_major_out, tile=tile)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    if d is not None:
        check_close(d, pre, tol, rms, desc + " D")
    if p is not None:
        check_close(p, post, tol, rms, desc + " PostAct")
