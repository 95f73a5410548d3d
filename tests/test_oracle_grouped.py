"""Pins for the oracle's variable-length-K grouped GEMM and its gathered-A modes.

Varlen-K (group l sums k over [cu_k[l], cu_k[l+1]) of an A (M, total_k) and a B
(N, total_k); outputs (l, m, n)) and gathered A (the A row of each global output row, or
the A column of each global k, read through an index array) are checked against numpy's
fp64 einsum on slices and fancy-indexed copies of the decoded operands (brute force on
tiny shapes, every major mode), against closed forms (all-ones operands give K_l exactly,
rank-1 operands K_l u_m v_n), against the partition of K (with small integers the group
results sum exactly to the GEMM over all of K), and against special cases (empty groups
give beta * C or zero; an identity gather equals no gather).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def f64(t):
    return t.to(torch.float64).numpy()


def a2(M, K, m_major, seed, dt, gen=W.uniform):
    """Logical (M, K) operand: storage [M][K] (K-major) or [K][M] (M-major)."""
    if m_major:
        return gen(seed, (K, M), dt).t()
    return gen(seed, (M, K), dt)


def lead(t, kmajor):
    return t.stride(0) if kmajor else t.stride(1)


def vk_problem(M, N, A, B, cu_k, dt, C=None, c_nmajor=True, alpha=1.0, beta=1.0, act="none",
               a_idx=None, a_rows=None):
    a_k, b_k = A.stride(1) == 1, B.stride(1) == 1
    L = len(cu_k) - 1
    kw = {}
    if C is not None:
        kw = dict(c_dt="f32", c_nmajor=c_nmajor, ldc=C.stride(1) if c_nmajor else C.stride(2),
                  sc=C.stride(0))
    return oracle.Problem(M, N, int(B.shape[1]), L, dt, dt, a_kmajor=a_k, b_kmajor=b_k,
                          lda=lead(A, a_k), ldb=lead(B, b_k), alpha=alpha, beta=beta, act=act,
                          cu_seqlens_k=cu_k, a_idx=a_idx, a_rows=a_rows, **kw)


def codes(t):
    return None if t is None else W.codes_of(t)


@pytest.mark.parametrize("dt", ["f16", "bf16", "e5m2"])
@pytest.mark.parametrize("a_mmaj,b_nmaj", [(False, False), (True, False), (False, True), (True, True)])
def test_varlen_k_brute_force_vs_numpy(dt, a_mmaj, b_nmaj):
    M, N = 9, 7
    cu_k = np.array([0, 5, 5, 17, 18, 30], dtype=np.int32)  # an empty group and a 1-wide one
    K = int(cu_k[-1])
    L = len(cu_k) - 1
    A = a2(M, K, a_mmaj, 300, dt)
    B = a2(N, K, b_nmaj, 301, dt)
    C = W.uniform(302, (L, M, N), "f32")
    p = vk_problem(M, N, A, B, cu_k, dt, C=C, alpha=0.5, beta=-2.0)
    pre, post = p.all(codes(A), codes(B), codes(C))
    a, b, c = f64(A), f64(B), f64(C)
    for g in range(L):
        lo, hi = cu_k[g], cu_k[g + 1]
        ref = 0.5 * np.einsum("mk,nk->mn", a[:, lo:hi], b[:, lo:hi]) - 2.0 * c[g]
        np.testing.assert_allclose(pre[g], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(pre, post)
    # the empty group is beta * C alone
    assert np.array_equal(pre[1], -2.0 * c[1])


def test_varlen_k_epilogue_relu_vs_numpy():
    M, N = 6, 10
    cu_k = np.array([0, 8, 24], dtype=np.int32)
    A = a2(M, 24, False, 310, "bf16")
    B = a2(N, 24, True, 311, "bf16")
    p = vk_problem(M, N, A, B, cu_k, "bf16", act="relu")
    pre, post = p.all(codes(A), codes(B), None)
    a, b = f64(A), f64(B)
    for g in range(2):
        ref = np.einsum("mk,nk->mn", a[:, cu_k[g]:cu_k[g + 1]], b[:, cu_k[g]:cu_k[g + 1]])
        np.testing.assert_allclose(pre[g], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(post[g], np.maximum(ref, 0.0), rtol=1e-12, atol=1e-12)


def test_varlen_k_all_ones_gives_group_length():
    M, N = 5, 4
    cu_k = np.array([0, 3, 3, 64, 100], dtype=np.int32)
    A = torch.ones((M, 100), dtype=torch.float16)
    B = torch.ones((100, N), dtype=torch.float16).t()  # N-major
    p = vk_problem(M, N, A, B, cu_k, "f16")
    pre, _ = p.all(codes(A), codes(B), None)
    for g in range(4):
        assert (pre[g] == float(cu_k[g + 1] - cu_k[g])).all()


def test_varlen_k_rank1_closed_form():
    M, N = 6, 5
    cu_k = np.array([0, 7, 40], dtype=np.int32)
    u = np.array([2.0 ** (i % 4 - 1) * (-1) ** i for i in range(M)])
    v = np.array([(i % 3) - 0.5 for i in range(N)])
    A = torch.from_numpy(np.repeat(u[:, None], 40, 1)).to(torch.bfloat16)
    B = torch.from_numpy(np.repeat(v[:, None], 40, 1)).to(torch.bfloat16)
    p = vk_problem(M, N, A, B, cu_k, "bf16")
    pre, _ = p.all(codes(A), codes(B), None)
    for g in range(2):
        assert np.array_equal(pre[g], (cu_k[g + 1] - cu_k[g]) * np.outer(u, v))


def test_varlen_k_partition_sums_to_full_k_exactly():
    """Small integers: every product and partial sum is exact, so the groups' results add up
    to the dot product over all of K, written out here as a numpy integer matmul."""
    M, N = 8, 6
    cu_k = np.array([0, 4, 11, 11, 32, 45], dtype=np.int32)
    r = np.random.Generator(np.random.PCG64(7))
    ai = r.integers(-3, 4, size=(M, 45))
    bi = r.integers(-3, 4, size=(N, 45))
    A = torch.from_numpy(ai.astype(np.float64)).to(torch.float16)
    B = torch.from_numpy(bi.astype(np.float64)).to(torch.float16)
    p = vk_problem(M, N, A, B, cu_k, "f16")
    pre, _ = p.all(codes(A), codes(B), None)
    assert np.array_equal(pre.sum(axis=0), (ai @ bi.T).astype(np.float64))


def test_varlen_k_empty_groups_without_c_are_zero():
    cu_k = np.array([0, 0, 0], dtype=np.int32)
    A = W.uniform(320, (4, 8), "bf16")
    B = W.uniform(321, (3, 8), "bf16")
    p = vk_problem(4, 3, A, B, cu_k, "bf16", act="gelu_tanh")
    pre, post = p.all(codes(A), codes(B), None)
    assert (pre == 0).all() and (post == 0).all()


@pytest.mark.parametrize("a_mmaj", [False, True])
def test_gather_rows_varlen_m_vs_numpy(a_mmaj):
    """Varlen-M with gathered A: output row r reads A row a_idx[r] (a_idx may repeat rows)."""
    rows_a, K, N = 23, 19, 6
    cu = np.array([0, 4, 4, 13], dtype=np.int32)
    G = len(cu) - 1
    a_idx = np.random.Generator(np.random.PCG64(11)).integers(0, rows_a, size=int(cu[-1])).astype(np.int32)
    A = a2(rows_a, K, a_mmaj, 330, "bf16")
    B = W.uniform(331, (G, N, K), "bf16")
    a_k = A.stride(1) == 1
    p = oracle.Problem(int(cu[-1]), N, K, G, "bf16", "bf16", a_kmajor=a_k, b_kmajor=True,
                       lda=lead(A, a_k), ldb=K, sb=N * K, cu_seqlens=cu, a_idx=a_idx, a_rows=rows_a)
    pre, _ = p.all(codes(A), codes(B), None)
    a, b = f64(A), f64(B)
    for g in range(G):
        rows = slice(cu[g], cu[g + 1])
        ref = np.einsum("mk,nk->mn", a[a_idx[rows]], b[g])
        np.testing.assert_allclose(pre[rows], ref, rtol=1e-12, atol=1e-12)


def test_gather_identity_equals_plain_varlen_m():
    K, N = 16, 5
    cu = np.array([0, 3, 10], dtype=np.int32)
    A = W.uniform(340, (10, K), "f16")
    B = W.uniform(341, (2, N, K), "f16")
    kw = dict(a_kmajor=True, b_kmajor=True, lda=K, ldb=K, sb=N * K, cu_seqlens=cu)
    plain = oracle.Problem(10, N, K, 2, "f16", "f16", **kw).all(codes(A), codes(B), None)[0]
    ident = oracle.Problem(10, N, K, 2, "f16", "f16", a_idx=np.arange(10, dtype=np.int32), a_rows=10,
                           **kw).all(codes(A), codes(B), None)[0]
    assert np.array_equal(plain, ident)


@pytest.mark.parametrize("b_nmaj", [False, True])
def test_gather_columns_varlen_k_vs_numpy(b_nmaj):
    """Varlen-K with gathered A: global k reads A column a_idx[k]; B is not gathered."""
    M, N, cols_a = 7, 5, 40
    cu_k = np.array([0, 9, 9, 21], dtype=np.int32)
    a_idx = np.random.Generator(np.random.PCG64(12)).permutation(cols_a)[:21].astype(np.int32)
    A = a2(M, cols_a, True, 350, "bf16")  # M-major: each k is one contiguous row of storage
    B = a2(N, 21, b_nmaj, 351, "bf16")
    p = vk_problem(M, N, A, B, cu_k, "bf16", a_idx=a_idx, a_rows=cols_a)
    pre, _ = p.all(codes(A), codes(B), None)
    a, b = f64(A), f64(B)
    for g in range(3):
        lo, hi = cu_k[g], cu_k[g + 1]
        ref = np.einsum("mk,nk->mn", a[:, a_idx[lo:hi]], b[:, lo:hi])
        np.testing.assert_allclose(pre[g], ref, rtol=1e-12, atol=1e-12)


def test_varlen_k_sampled_points_and_rows_agree_with_all():
    M, N = 10, 9
    cu_k = np.array([0, 6, 20, 33], dtype=np.int32)
    A = a2(M, 33, True, 360, "bf16")
    B = a2(N, 33, False, 361, "bf16")
    C = W.uniform(362, (3, M, N), "f32")
    p = vk_problem(M, N, A, B, cu_k, "bf16", C=C, beta=0.25, act="silu")
    pre, post = p.all(codes(A), codes(B), codes(C))
    pts = np.array([[0, 0, 0], [1, 9, 8], [2, 4, 3], [2, 0, 8]])
    pp, qq = p.points(codes(A), codes(B), codes(C), pts)
    for i, (l, m, n) in enumerate(pts):
        assert pp[i] == pre[l, m, n] and qq[i] == post[l, m, n]
    rp, rq = p.rows(codes(A), codes(B), codes(C), np.array([[1, 3], [2, 9]]))
    assert np.array_equal(rp[0], pre[1, 3]) and np.array_equal(rq[1], post[2, 9])


# ---------------------------------------------------------------------------------------
# gathered indices outside A, and the cu_seqlens preconditions
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("a_mmaj", [False, True])
def test_gather_rows_out_of_range_read_zero_vs_padded_numpy(a_mmaj):
    """An index outside [0, rows of A) reads a zero row: numpy gathers from A with an
    explicit zero row appended, the out-of-range indices sent to it."""
    rows_a, K, N = 11, 24, 5
    cu = np.array([0, 6, 6, 14], dtype=np.int32)
    G, M = len(cu) - 1, int(cu[-1])
    a_idx = np.random.Generator(np.random.PCG64(21)).integers(0, rows_a, size=M).astype(np.int32)
    a_idx[[0, 5, 7, 13]] = [-1, rows_a, 1 << 30, -(1 << 31)]
    A = a2(rows_a, K, a_mmaj, 370, "bf16")
    B = W.uniform(371, (G, N, K), "bf16")
    C = W.uniform(372, (M, N), "f32")
    a_k = A.stride(1) == 1
    p = oracle.Problem(M, N, K, G, "bf16", "bf16", a_kmajor=a_k, b_kmajor=True, lda=lead(A, a_k),
                       ldb=K, sb=N * K, c_dt="f32", ldc=N, alpha=2.0, beta=0.5, act="relu",
                       cu_seqlens=cu, a_idx=a_idx, a_rows=rows_a)
    pre, post = p.all(codes(A), codes(B), codes(C))
    a_pad = np.concatenate([f64(A), np.zeros((1, K))])
    idx = np.where((a_idx < 0) | (a_idx >= rows_a), rows_a, a_idx)
    b, c = f64(B), f64(C)
    for g in range(G):
        rows = slice(cu[g], cu[g + 1])
        ref = 2.0 * np.einsum("mk,nk->mn", a_pad[idx[rows]], b[g]) + 0.5 * c[rows]
        np.testing.assert_allclose(pre[rows], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(post[rows], np.maximum(ref, 0.0), rtol=1e-12, atol=1e-12)
    for r in (0, 5, 7, 13):  # those rows hold beta * C alone
        assert np.array_equal(pre[r], 0.5 * c[r])


def test_gather_columns_out_of_range_read_zero_vs_padded_numpy():
    M, N, cols_a = 6, 7, 30
    cu_k = np.array([0, 10, 10, 25], dtype=np.int32)
    a_idx = np.random.Generator(np.random.PCG64(22)).integers(0, cols_a, size=25).astype(np.int32)
    a_idx[[0, 9, 12, 24]] = [-5, cols_a, 1 << 29, cols_a + 1]
    A = a2(M, cols_a, True, 380, "bf16")
    B = a2(N, 25, False, 381, "bf16")
    p = vk_problem(M, N, A, B, cu_k, "bf16", a_idx=a_idx, a_rows=cols_a)
    pre, _ = p.all(codes(A), codes(B), None)
    a_pad = np.concatenate([f64(A), np.zeros((M, 1))], axis=1)
    idx = np.where((a_idx < 0) | (a_idx >= cols_a), cols_a, a_idx)
    b = f64(B)
    for g in range(3):
        lo, hi = cu_k[g], cu_k[g + 1]
        ref = np.einsum("mk,nk->mn", a_pad[:, idx[lo:hi]], b[:, lo:hi])
        np.testing.assert_allclose(pre[g], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cu", [[1, 4, 9], [0, 5, 4, 9], [0, 4, 8], [0, 4, 10], [0, -1, 9]])
def test_bad_cu_seqlens_m_is_rejected(cu):
    """cu_seqlens must start at 0, never decrease and end at M = 9."""
    cu = np.array(cu, dtype=np.int32)
    G = len(cu) - 1
    A = W.uniform(390, (9, 8), "bf16")
    B = W.uniform(391, (G, 3, 8), "bf16")
    p = oracle.Problem(9, 3, 8, G, "bf16", "bf16", lda=8, ldb=8, sb=24, cu_seqlens=cu)
    with pytest.raises(ValueError, match="cu_seqlens"):
        p.all(codes(A), codes(B), None)
    with pytest.raises(ValueError, match="cu_seqlens"):
        p.points(codes(A), codes(B), None, np.array([[0, 0, 0]]))


@pytest.mark.parametrize("cu_k", [[2, 5, 8], [0, 6, 5], [0, 4, 9]])
def test_bad_cu_seqlens_k_is_rejected(cu_k):
    """cu_seqlens_k must start at 0, never decrease and end at most at K = 8."""
    A = a2(3, 8, False, 392, "bf16")
    B = a2(4, 8, False, 393, "bf16")
    p = vk_problem(3, 4, A, B, np.array(cu_k, dtype=np.int32), "bf16")
    with pytest.raises(ValueError, match="cu_seqlens_k"):
        p.all(codes(A), codes(B), None)


def test_points_outside_the_output_are_rejected():
    A = W.uniform(394, (1, 5, 8), "bf16")
    B = W.uniform(395, (1, 4, 8), "bf16")
    p = oracle.Problem(5, 4, 8, 1, "bf16", "bf16")
    for bad in ([0, 5, 0], [0, 0, 4], [1, 0, 0], [0, -1, 0]):
        with pytest.raises(ValueError, match="outside"):
            p.points(codes(A), codes(B), None, np.array([bad]))
    with pytest.raises(ValueError, match="outside"):
        p.rows(codes(A), codes(B), None, np.array([[0, 5]]))
