"""Pins for the oracle's GEMM and epilogue.

The oracle is checked against: numpy's fp64 einsum on torch-decoded inputs (brute force on
tiny shapes, every major mode, L in {1, 3}); closed forms (identity, permutation, rank-1,
small integers whose products and sums are exact); linearity; the epilogue's special cases
(B = 0, alpha scaling, activation none); torch / scipy activation routines in float64; and
for varlen-M, the equivalence with the batched GEMM and the per-group plain GEMM.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as W

DT16 = ["f16", "bf16"]


def f64(t):
    return t.to(torch.float64).numpy()


def problem_of(inp: W.Inputs, act=None, alpha=None, beta=None, c=True):
    """Oracle Problem for an Inputs (addresses from the logical views' strides)."""
    A, B = inp.A, inp.B
    if inp.varlen:
        a_k = A.stride(1) == 1
        lda = A.stride(0) if a_k else A.stride(1)
        b_k = B.stride(2) == 1
        ldb = B.stride(1) if b_k else B.stride(2)
        sa, sb = 0, B.stride(0)
        L = B.shape[0]
    else:
        a_k = A.stride(2) == 1
        lda = A.stride(1) if a_k else A.stride(2)
        b_k = B.stride(2) == 1
        ldb = B.stride(1) if b_k else B.stride(2)
        sa, sb = A.stride(0), B.stride(0)
        L = A.shape[0]
    kw = {}
    if inp.C is not None and c:
        C = inp.C
        if inp.varlen:
            c_n = C.stride(1) == 1
            kw = dict(c_dt=inp.c_dt, c_nmajor=c_n, ldc=C.stride(0) if c_n else C.stride(1), sc=0)
        else:
            c_n = C.stride(2) == 1
            kw = dict(c_dt=inp.c_dt, c_nmajor=c_n, ldc=C.stride(1) if c_n else C.stride(2),
                      sc=C.stride(0))
    return oracle.Problem(inp.M, inp.N, inp.K, L, inp.a_dt, inp.b_dt, a_kmajor=a_k,
                          b_kmajor=b_k, lda=lda, ldb=ldb, sa=sa, sb=sb,
                          alpha=inp.alpha if alpha is None else alpha,
                          beta=inp.beta if beta is None else beta,
                          act=inp.act if act is None else act,
                          cu_seqlens=inp.cu_seqlens, **kw)


def run_all(inp, **kw):
    p = problem_of(inp, **kw)
    C = W.codes_of(inp.C) if (inp.C is not None and kw.get("c", True)) else None
    return p.all(W.codes_of(inp.A), W.codes_of(inp.B), C)


def small_inputs(M, N, K, L, dt, a_mmaj, b_nmaj, with_c, seed, act="none", alpha=1.0, beta=1.0,
                 c_nmaj=True):
    gen = W.uniform
    A = W.make_a(gen, L, M, K, a_mmaj, seed, dt)
    B = W.make_b(gen, L, N, K, b_nmaj, seed + 1, dt)
    C = None
    if with_c:
        C = gen(seed + 2, (L, M, N), "f32") if c_nmaj else gen(seed + 2, (L, N, M), "f32").permute(0, 2, 1)
    return W.Inputs("t", M, N, K, L, dt, dt, A, B, C=C, c_dt="f32" if with_c else "none",
                    d_dt="f32", alpha=alpha, beta=beta, act=act)


@pytest.mark.parametrize("dt", DT16 + ["e4m3"])
@pytest.mark.parametrize("a_mmaj,b_nmaj", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("L", [1, 3])
def test_brute_force_vs_numpy_einsum(dt, a_mmaj, b_nmaj, L):
    M, N, K = 13, 11, 17
    inp = small_inputs(M, N, K, L, dt, a_mmaj, b_nmaj, True, 100 + L, alpha=0.75, beta=-1.25,
                       c_nmaj=not a_mmaj)
    pre, post = run_all(inp)
    ref = 0.75 * np.einsum("lmk,lnk->lmn", f64(inp.A), f64(inp.B)) - 1.25 * f64(inp.C)
    np.testing.assert_allclose(pre, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(pre, post)  # act none


@pytest.mark.parametrize("dt", DT16)
def test_identity_exact(dt):
    K = 24
    eye = torch.eye(K, dtype=torch.float64).to(W.TORCH_DT[dt]).reshape(1, K, K)
    B = W.uniform(7, (1, 9, K), dt)
    inp = W.Inputs("id", K, 9, K, 1, dt, dt, eye, B)
    pre, _ = run_all(inp)
    # D[m][n] = B[n][m] exactly
    assert np.array_equal(pre[0], f64(B[0]).T)


def test_permutation_exact():
    K = 16
    perm = np.random.Generator(np.random.PCG64(3)).permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    A = torch.from_numpy(P).to(torch.bfloat16).reshape(1, K, K)
    B = W.uniform(8, (1, 5, K), "bf16")
    inp = W.Inputs("perm", K, 5, K, 1, "bf16", "bf16", A, B)
    pre, _ = run_all(inp)
    assert np.array_equal(pre[0], f64(B[0]).T[perm])


def test_rank1_closed_form():
    M, N, K = 10, 7, 33
    u = np.array([2.0 ** (i % 5 - 2) * (-1) ** i for i in range(M)])
    v = np.array([(i % 4) - 1.5 for i in range(N)])
    A = torch.from_numpy(np.repeat(u[:, None], K, 1)).to(torch.float16).reshape(1, M, K)
    B = torch.from_numpy(np.repeat(v[:, None], K, 1)).to(torch.float16).reshape(1, N, K)
    inp = W.Inputs("r1", M, N, K, 1, "f16", "f16", A, B)
    pre, _ = run_all(inp)
    assert np.array_equal(pre[0], K * np.outer(u, v))


@pytest.mark.parametrize("dt", ["f16", "bf16", "e4m3", "e5m2"])
def test_small_integer_exact(dt):
    r = np.random.Generator(np.random.PCG64(11))
    M, N, K = 8, 6, 40
    a = r.integers(-3, 4, size=(1, M, K)).astype(np.float64)
    b = r.integers(-3, 4, size=(1, N, K)).astype(np.float64)
    inp = W.Inputs("int", M, N, K, 1, dt, dt, W.to_dtype(a, dt), W.to_dtype(b, dt))
    pre, _ = run_all(inp)
    exact = np.einsum("lmk,lnk->lmn", a, b)  # integers: every step exact
    assert np.array_equal(pre, exact)


def test_linearity_power_of_two():
    inp = small_inputs(9, 12, 20, 1, "bf16", False, False, False, 21)
    pre1, _ = run_all(inp)
    inp2 = W.Inputs("x2", inp.M, inp.N, inp.K, 1, "bf16", "bf16",
                    (inp.A.to(torch.float64) * 2).to(torch.bfloat16), inp.B)
    pre2, _ = run_all(inp2)
    assert np.array_equal(pre2, 2 * pre1)


def test_k_zero_gives_beta_c():
    C = W.uniform(5, (1, 4, 5), "f32")
    A = torch.zeros((1, 4, 0), dtype=torch.bfloat16)
    B = torch.zeros((1, 5, 0), dtype=torch.bfloat16)
    inp = W.Inputs("k0", 4, 5, 0, 1, "bf16", "bf16", A, B, C=C, c_dt="f32", beta=0.5)
    p = problem_of(inp)
    pre, _ = p.all(np.zeros(1, np.uint16), np.zeros(1, np.uint16), W.codes_of(C))
    assert np.array_equal(pre, 0.5 * f64(C))


# ---------------------------------------------------------------------------------------
# epilogue
# ---------------------------------------------------------------------------------------

def test_b_zero_gives_beta_c_exactly():
    inp = small_inputs(7, 9, 12, 2, "f16", False, False, True, 31, beta=0.25)
    inp.B = torch.zeros_like(inp.B)
    pre, _ = run_all(inp)
    assert np.array_equal(pre, 0.25 * f64(inp.C))


def test_alpha_scales_and_beta_zero_still_reads_c():
    inp = small_inputs(6, 5, 8, 1, "bf16", False, False, True, 41)
    base, _ = run_all(inp, alpha=1.0, beta=0.0)
    scaled, _ = run_all(inp, alpha=-4.0, beta=0.0)
    assert np.array_equal(scaled, -4.0 * base)
    # beta = 0 with a NaN in C: NaN propagates (C is read and multiplied)
    Cn = inp.C.clone()
    Cn[0, 2, 3] = float("nan")
    inp.C = Cn
    pre, _ = run_all(inp, beta=0.0)
    assert math.isnan(pre[0, 2, 3]) and np.isfinite(np.delete(pre.ravel(), 2 * 5 + 3)).all()


@pytest.mark.parametrize("act", ["relu", "relu_sq", "gelu_tanh", "silu"])
def test_activation_applied_to_unrounded_pre(act):
    inp = small_inputs(11, 10, 9, 1, "bf16", False, False, True, 51, act=act, alpha=1.5, beta=0.5)
    pre, post = run_all(inp)
    ref = {"relu": lambda x: np.maximum(x, 0.0),
           "relu_sq": lambda x: np.maximum(x, 0.0) ** 2,
           "gelu_tanh": lambda x: torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy(),
           "silu": lambda x: x * scipy.special.expit(x)}[act](pre)
    np.testing.assert_allclose(post, ref, rtol=1e-13, atol=1e-15)


def test_activation_closed_forms():
    a = oracle.act
    xs = np.linspace(-7, 7, 57)
    for x in xs:
        assert a("relu", x) == max(x, 0.0)
        assert a("relu_sq", x) == max(x, 0.0) ** 2
        # x - act(-x) identity: act(x) - act(-x) = x for gelu_tanh and silu
        assert abs(a("gelu_tanh", x) - a("gelu_tanh", -x) - x) < 1e-14 * (1 + abs(x))
        assert abs(a("silu", x) - a("silu", -x) - x) < 1e-14 * (1 + abs(x))
        # GELU-tanh stays within 1e-3 of the exact (erf) GELU
        exact = 0.5 * x * (1 + math.erf(x / math.sqrt(2)))
        assert abs(a("gelu_tanh", x) - exact) < 1e-3
    assert a("gelu_tanh", 0.0) == 0.0 and a("silu", 0.0) == 0.0
    assert a("gelu_tanh", 40.0) == 40.0 and a("silu", 40.0) == pytest.approx(40.0, abs=1e-15)
    assert abs(a("gelu_tanh", -40.0)) < 1e-300 and abs(a("silu", -40.0)) < 1e-15
    # slope at the origin is 1/2 for both
    h = 1e-7
    assert a("gelu_tanh", h) / h == pytest.approx(0.5, rel=1e-6)
    assert a("silu", h) / h == pytest.approx(0.5, rel=1e-6)
    # scipy reference for SiLU and torch's float64 tanh-GELU
    for x in (-3.3, -0.2, 0.7, 2.9):
        assert a("silu", x) == pytest.approx(x * scipy.special.expit(x), rel=1e-15)
        g = torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh").item()
        assert a("gelu_tanh", x) == pytest.approx(g, rel=1e-14)


# ---------------------------------------------------------------------------------------
# varlen-M
# ---------------------------------------------------------------------------------------

def test_varlen_equal_groups_equals_batched():
    G, Mg, N, K = 3, 5, 7, 9
    A3 = W.uniform(61, (G, Mg, K), "bf16")
    B = W.uniform(62, (G, N, K), "bf16")
    batched = W.Inputs("b", Mg, N, K, G, "bf16", "bf16", A3, B)
    pb, _ = run_all(batched)
    cu = np.arange(G + 1, dtype=np.int32) * Mg
    var = W.Inputs("v", G * Mg, N, K, G, "bf16", "bf16", A3.reshape(G * Mg, K), B, cu_seqlens=cu)
    pv, _ = run_all(var)
    assert np.array_equal(pv, pb.reshape(G * Mg, N))


def test_varlen_one_group_equals_plain():
    M, N, K = 12, 6, 10
    A = W.uniform(71, (M, K), "f16")
    B = W.uniform(72, (1, N, K), "f16")
    var = W.Inputs("v", M, N, K, 1, "f16", "f16", A, B, cu_seqlens=np.array([0, M], np.int32))
    plain = W.Inputs("p", M, N, K, 1, "f16", "f16", A.reshape(1, M, K), B)
    pv, _ = run_all(var)
    pp, _ = run_all(plain)
    assert np.array_equal(pv, pp[0])


def test_varlen_empty_groups_and_per_group_b():
    sizes = [0, 4, 0, 3, 1, 0]
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G, M, N, K = len(sizes), int(cu[-1]), 5, 6
    A = W.uniform(81, (M, K), "bf16")
    B = W.uniform(82, (G, N, K), "bf16")
    C = W.uniform(83, (M, N), "f32")
    var = W.Inputs("v", M, N, K, G, "bf16", "bf16", A, B, C=C, c_dt="f32", beta=2.0,
                   act="relu", cu_seqlens=cu)
    pre, post = run_all(var)
    for g in range(G):
        r0, r1 = cu[g], cu[g + 1]
        ref = f64(A[r0:r1]) @ f64(B[g]).T + 2.0 * f64(C[r0:r1])
        assert np.allclose(pre[r0:r1], ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(post, np.maximum(pre, 0))


def test_points_and_rows_agree_with_all():
    inp = small_inputs(9, 8, 7, 2, "f16", True, False, True, 91, act="silu", beta=0.5)
    p = problem_of(inp)
    A, B, C = W.codes_of(inp.A), W.codes_of(inp.B), W.codes_of(inp.C)
    pre, post = p.all(A, B, C)
    pts = np.array([[1, 3, 4], [0, 0, 0], [1, 8, 7]])
    pp, qq = p.points(A, B, C, pts)
    assert np.array_equal(pp, pre[pts[:, 0], pts[:, 1], pts[:, 2]])
    assert np.array_equal(qq, post[pts[:, 0], pts[:, 1], pts[:, 2]])
    rr, _ = p.rows(A, B, C, np.array([[1, 2], [0, 5]]))
    assert np.array_equal(rr, np.stack([pre[1, 2], pre[0, 5]]))
