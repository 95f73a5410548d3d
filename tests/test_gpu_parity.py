"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Small cases span several tiles and ragged tails in M, N and K and cover every dtype, major
mode, output type, activation, alpha/beta form, batch and varlen layout. Small-integer
cases must match exactly. The five workloads run at full size with sampled outputs.
The persistent schedule (device tile log) and the device FastDivmod are checked bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (check_close, gather, oracle_codes, out_like, problem_of, run_hip,
                    sample_points, tile_cover_points, tile_rows, to_dev, tol_for)

pytestmark = pytest.mark.gpu


def announce(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


def small(M, N, K, L, a_dt, b_dt=None, a_mmaj=False, b_nmaj=False, c_dt="none", d_dt="bf16",
          post_dt="none", act="none", alpha=1.0, beta=1.0, seed=0, gen=W.uniform, c_mmaj=False):
    b_dt = b_dt or a_dt
    A = W.make_a(gen, L, M, K, a_mmaj, 500 + seed, a_dt)
    B = W.make_b(gen, L, N, K, b_nmaj, 600 + seed, b_dt)
    C = None
    if c_dt != "none":
        C = gen(700 + seed, (L, N, M), c_dt).permute(0, 2, 1) if c_mmaj else gen(700 + seed, (L, M, N), c_dt)
    return W.Inputs(f"small_{a_dt}", M, N, K, L, a_dt, b_dt, A, B, C=C, c_dt=c_dt, d_dt=d_dt,
                    post_dt=post_dt, alpha=alpha, beta=beta, act=act)


def compare_full(inp, tile=None, d_major_m=False, **kw):
    announce(f"{inp.name} M={inp.M} N={inp.N} K={inp.K} L={inp.L} tile={tile} mmaj_out={d_major_m}")
    d, p, _ = run_hip(inp, d_major_m=d_major_m, tile=tile, **kw)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    if d is not None:
        check_close(d, pre, tol, rms, "D")
    if p is not None:
        check_close(p, post, tol, rms, "PostAct")
    return d, p, pre, post


# ---------------------------------------------------------------------------------------
# small shapes: every dtype / major / tile, ragged tails
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("a_mmaj,b_nmaj", [(False, False), (True, False), (False, True), (True, True)])
def test_small_16bit_majors(tile, dt, a_mmaj, b_nmaj):
    inp = small(296, 392, 200, 1, dt, a_mmaj=a_mmaj, b_nmaj=b_nmaj, d_dt=dt, seed=1)
    compare_full(inp, tile=tile)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e5m2", "e4m3")])
def test_small_fp8(tile, fa, fb):
    inp = small(264, 200, 336, 1, fa, fb, d_dt="bf16", seed=2, alpha=0.5)
    compare_full(inp, tile=tile)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("act", ["none", "relu", "relu_sq", "gelu_tanh", "silu"])
def test_small_epilogue_acts(tile, act):
    inp = small(136, 520, 96, 1, "bf16", c_dt="bf16", d_dt="bf16", post_dt="bf16", act=act,
                alpha=1.5, beta=0.5, seed=3, gen=lambda s, sh, dt: W.normal(s, sh, dt, 0.5))
    compare_full(inp, tile=tile)


@pytest.mark.parametrize("c_dt,d_dt,post_dt", [("f32", "f32", "none"), ("f16", "none", "f16"),
                                               ("none", "f32", "bf16"), ("bf16", "f16", "f32")])
def test_small_output_types(c_dt, d_dt, post_dt):
    act = "gelu_tanh" if post_dt != "none" else "none"
    inp = small(200, 264, 64, 1, "f16", c_dt=c_dt, d_dt=d_dt, post_dt=post_dt, act=act,
                alpha=-0.75, beta=2.0, seed=4)
    compare_full(inp)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_small_batched_strided(tile):
    inp = small(160, 136, 72, 3, "bf16", a_mmaj=True, c_dt="f32", d_dt="bf16", beta=-1.0, seed=5)
    compare_full(inp, tile=tile)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_small_m_major_outputs(tile):
    # C, D, PostAct all M-contiguous (computed as the transposed problem)
    inp = small(264, 136, 80, 2, "f16", b_nmaj=True, c_dt="f16", d_dt="f16", post_dt="bf16",
                act="relu", beta=0.25, seed=6, c_mmaj=True)
    compare_full(inp, tile=tile, d_major_m=True)


def test_k_zero_and_empty():
    inp = small(130, 136, 0, 2, "bf16", c_dt="f32", d_dt="f32", beta=0.5, seed=7)
    inp.A = torch.zeros((2, 130, 0), dtype=torch.bfloat16)
    inp.B = torch.zeros((2, 136, 0), dtype=torch.bfloat16)
    d, _, _ = run_hip(inp)
    assert np.array_equal(d, 0.5 * inp.C.double().numpy())
    # M = 0: nothing to do, no launch
    e = small(0, 64, 64, 1, "bf16", seed=8)
    d, _, _ = run_hip(e)
    assert d.shape == (1, 0, 64)


def test_alpha_beta_device_pointers():
    inp = small(256, 256, 128, 1, "bf16", c_dt="bf16", d_dt="f32", alpha=99.0, beta=99.0, seed=9)
    a = torch.tensor([0.25], dtype=torch.float32, device="cuda")
    b = torch.tensor([-2.0], dtype=torch.float32, device="cuda")
    d, _, _ = run_hip(inp, alpha_dev=a, beta_dev=b)
    pre, _ = problem_of(inp, alpha=0.25, beta=-2.0).all(*oracle_codes(inp))
    check_close(d, pre, 1e-5, 1e-5, "D")


@pytest.mark.parametrize("dt", ["f16", "bf16", "e4m3", "e5m2"])
@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_small_integers_exact(dt, tile):
    """Entries in {-3..3}: products and fp32 sums are exact, so f32 D equals the oracle."""
    r = np.random.Generator(np.random.PCG64(11))
    M, N, K = 200, 264, 512
    a = r.integers(-3, 4, size=(1, M, K)).astype(np.float64)
    b = r.integers(-3, 4, size=(1, N, K)).astype(np.float64)
    c = r.integers(-8, 9, size=(1, M, N)).astype(np.float64)
    inp = W.Inputs("ints", M, N, K, 1, dt, dt, W.to_dtype(a, dt), W.to_dtype(b, dt),
                   C=W.to_dtype(c, "f32"), c_dt="f32", d_dt="f32", beta=2.0)
    d, _, _ = run_hip(inp, tile=tile)
    exact = np.einsum("lmk,lnk->lmn", a, b) + 2.0 * c
    assert np.array_equal(d, exact)
    pre, _ = problem_of(inp).all(*oracle_codes(inp))
    assert np.array_equal(d, pre)


def test_identity_exact():
    K = 256
    eye = torch.eye(K, dtype=torch.float64).to(torch.bfloat16).reshape(1, K, K)
    B = W.uniform(12, (1, 384, K), "bf16")
    inp = W.Inputs("id", K, 384, K, 1, "bf16", "bf16", eye, B, d_dt="bf16")
    d, _, _ = run_hip(inp)
    assert np.array_equal(d[0], B[0].double().numpy().T)


# ---------------------------------------------------------------------------------------
# fp8 outputs (D / PostAct in e4m3 or e5m2: round to nearest even, saturating)
# ---------------------------------------------------------------------------------------

def check_fp8(got, want, dt, what):
    """got: decoded GPU fp8 outputs; want: the oracle's fp64 values. Each output must be the
    oracle's own encoding of its value, or - where that value lies within fp32 rounding of
    the midpoint between two fp8 neighbours - the other neighbour."""
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    enc = oracle.decode_array(dt, oracle.encode_array(dt, want))
    same = (got == enc) | (np.isnan(got) & np.isnan(enc))
    near_tie = np.abs(want - (got + enc) / 2) <= 1e-4 * np.abs(want) + 1e-7
    ok = same | near_tie
    assert ok.all(), (f"{what}: {(~ok).sum()} outputs off, first at {np.argmax(~ok)}: "
                      f"got {got[np.argmax(~ok)]} want {want[np.argmax(~ok)]} ({enc[np.argmax(~ok)]})")
    assert same.mean() > 0.99, f"{what}: only {same.mean():.4f} exact"


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_small_fp8_outputs(tile):
    inp = small(296, 400, 136, 2, "bf16", c_dt="bf16", d_dt="e4m3", post_dt="e5m2", act="gelu_tanh",
                alpha=3.0, beta=0.5, seed=60, gen=lambda s, sh, dt: W.normal(s, sh, dt, 0.5))
    announce(f"fp8 outputs tile={tile}")
    d, p, _ = run_hip(inp, tile=tile)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    check_fp8(d, pre, "e4m3", "D")
    check_fp8(p, post, "e5m2", "PostAct")


def test_fp8_outputs_exact_saturating_and_nan():
    r = np.random.Generator(np.random.PCG64(61))
    M, N, K = 136, 272, 32
    a = r.integers(-3, 4, size=(1, M, K)).astype(np.float64)
    b = r.integers(-3, 4, size=(1, N, K)).astype(np.float64)
    c = r.integers(-8, 9, size=(1, M, N)).astype(np.float64)
    c[0, 5, 7] = np.nan
    c[0, 9, 11] = np.inf
    c[0, 10, 12] = -np.inf
    for d_dt, p_dt in (("e4m3", "e5m2"), ("e5m2", "e4m3")):
        inp = W.Inputs("fp8out", M, N, K, 1, "bf16", "bf16", W.to_dtype(a, "bf16"), W.to_dtype(b, "bf16"),
                       C=W.to_dtype(c, "f32"), c_dt="f32", d_dt=d_dt, post_dt=p_dt, act="relu",
                       alpha=8.0, beta=1.0)  # |8 acc| up to 2304: past e4m3's 448
        d, p, _ = run_hip(inp)
        pre, post = problem_of(inp).all(*oracle_codes(inp))
        for got, want, dt in ((d, pre, d_dt), (p, post, p_dt)):
            enc = oracle.decode_array(dt, oracle.encode_array(dt, want.ravel())).reshape(want.shape)
            assert np.array_equal(np.isnan(got), np.isnan(enc))
            assert np.array_equal(got[~np.isnan(got)], enc[~np.isnan(enc)]), dt
        assert np.isnan(d[0, 5, 7]) and d[0, 9, 11] == (448.0 if d_dt == "e4m3" else 57344.0)


# ---------------------------------------------------------------------------------------
# activation backward (dact): D = (alpha A x B) * act'(C), PostAct = act(C)
# ---------------------------------------------------------------------------------------

def small_dact(M, N, K, L, act, c_dt="bf16", d_dt="bf16", post_dt="bf16", alpha=1.0, seed=50):
    inp = small(M, N, K, L, "bf16", c_dt=c_dt, d_dt=d_dt, post_dt=post_dt, act=act, alpha=alpha,
                seed=seed, gen=lambda s, sh, dt: W.normal(s, sh, dt, 0.5))
    inp.C = W.normal(700 + seed, (L, M, N), c_dt, 1.5) if c_dt != "none" else None
    inp.dact = True
    return inp


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("act", ["none", "relu", "relu_sq", "gelu_tanh", "silu"])
def test_small_dact(tile, act):
    compare_full(small_dact(296, 392, 136, 1, act, alpha=0.75), tile=tile)


@pytest.mark.parametrize("c_dt,d_dt,post_dt", [("f32", "f16", "f32"), ("f16", "f16", "none"),
                                               ("bf16", "f32", "bf16")])
def test_small_dact_types_and_batches(c_dt, d_dt, post_dt):
    compare_full(small_dact(200, 264, 72, 2, "gelu_tanh", c_dt=c_dt, d_dt=d_dt, post_dt=post_dt, seed=51))


def test_dact_small_integers_exact():
    r = np.random.Generator(np.random.PCG64(52))
    M, N, K = 136, 200, 96
    a = r.integers(-3, 4, size=(1, M, K)).astype(np.float64)
    b = r.integers(-3, 4, size=(1, N, K)).astype(np.float64)
    c = r.integers(-6, 7, size=(1, M, N)).astype(np.float64) / 2.0
    for act in ("none", "relu", "relu_sq"):
        inp = W.Inputs("dact_ints", M, N, K, 1, "bf16", "bf16", W.to_dtype(a, "bf16"), W.to_dtype(b, "bf16"),
                       C=W.to_dtype(c, "bf16"), c_dt="bf16", d_dt="f32", post_dt="f32", act=act, dact=True)
        d, p, _ = run_hip(inp)
        pre, post = problem_of(inp).all(*oracle_codes(inp))
        assert np.array_equal(d, pre) and np.array_equal(p, post), act


def test_dact_varlen_and_device_alpha():
    inp = varlen_small([0, 300, 129, 0, 255], K=72, act="gelu_tanh", seed=53)
    inp.C = W.normal(1053, (inp.M, inp.N), "bf16", 1.5)
    inp.c_dt = "bf16"
    inp.beta = 1.0
    inp.dact = True
    compare_full(inp)
    a = torch.tensor([-0.5], dtype=torch.float32, device="cuda")
    d, p, _ = run_hip(inp, alpha_dev=a)
    pre, post = problem_of(inp, alpha=-0.5).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    check_close(p, post, tol, rms, "PostAct")


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_small_dact_fp8(tile):
    # fp8 operands through the activation-backward kernels, dense and varlen-M (the 256x256
    # tiles take the 8-wave 16x16x128 loop, with a partly empty last M-block)
    M, N, K = 296, 392, 256
    A, sa = W.quantize_fp8(54, (1, M, K), "e4m3")
    B, sb = W.quantize_fp8(55, (1, N, K), "e5m2")
    inp = W.Inputs("dact_fp8", M, N, K, 1, "e4m3", "e5m2", A, B, C=W.normal(1054, (1, M, N), "bf16", 1.5),
                   c_dt="bf16", d_dt="bf16", post_dt="bf16", act="gelu_tanh", alpha=sa * sb, dact=True)
    compare_full(inp, tile=tile)
    sizes = np.array([0, 300, 129, 0, 255])
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, G = int(cu[-1]), len(sizes)
    A, sa = W.quantize_fp8(56, (M, K), "e5m2")
    B, sb = W.quantize_fp8(57, (G, N, K), "e4m3")
    inp = W.Inputs("dact_fp8_varlen", M, N, K, G, "e5m2", "e4m3", A, B, C=W.normal(1056, (M, N), "bf16", 1.5),
                   c_dt="bf16", d_dt="bf16", post_dt="bf16", act="silu", alpha=sa * sb, dact=True,
                   cu_seqlens=cu)
    compare_full(inp, tile=tile)


def test_workload_dact_4096():
    full_size(W.dact_4096())


# ---------------------------------------------------------------------------------------
# varlen-M
# ---------------------------------------------------------------------------------------

def varlen_small(sizes, N=264, K=136, seed=13, act="silu", c=True, a_mmaj=False, dt="bf16"):
    sizes = np.asarray(sizes)
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G, M = len(sizes), int(cu[-1])
    if a_mmaj:
        A = W.normal(800 + seed, (K, M), dt, 0.5).t()
    else:
        A = W.normal(800 + seed, (M, K), dt, 0.5)
    B = W.normal(900 + seed, (G, N, K), dt, 0.5)
    C = W.normal(1000 + seed, (M, N), "f32") if c else None
    return W.Inputs("varlen_small", M, N, K, G, dt, dt, A, B, C=C, c_dt="f32" if c else "none",
                    d_dt="bf16", post_dt="bf16", act=act, beta=0.5, cu_seqlens=cu)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
@pytest.mark.parametrize("sizes", [[0, 300, 0, 1, 129, 0], [256, 256, 256], [5], [0, 0, 77],
                                   [384, 0, 513, 128, 1, 255]])
def test_varlen_small(tile, sizes):
    compare_full(varlen_small(sizes), tile=tile)


def test_varlen_m_major_a_and_fp8():
    compare_full(varlen_small([136, 0, 264, 16], a_mmaj=True, dt="f16"))
    sizes = np.array([64, 0, 200, 128])
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M, N, K, G = int(cu[-1]), 136, 256, 4
    A, sa = W.quantize_fp8(31, (M, K), "e4m3")
    B, sb = W.quantize_fp8(32, (G, N, K), "e5m2")
    inp = W.Inputs("varlen_fp8", M, N, K, G, "e4m3", "e5m2", A, B, d_dt="bf16", alpha=sa * sb,
                   cu_seqlens=cu)
    compare_full(inp)


def test_varlen_all_groups_empty():
    inp = varlen_small([0, 0, 0])
    d, p, _ = run_hip(inp)
    assert d.shape == (0, 264)


# ---------------------------------------------------------------------------------------
# split tail: a partial last round of 256x256 tiles runs as 128x128 quarters in a second
# launch; the results must match the oracle and, bit for bit, the unsplit schedule (each
# output's k-order and epilogue arithmetic are the same in both kernels)
# ---------------------------------------------------------------------------------------

def _check_split(inp):
    d, p, plan = run_hip(inp)
    T, P = plan.grid()[4:6]
    if T >= 0:  # dense: the plan knows T
        assert T > P and 0 < T % P <= P // 2, (T, P)
    pre, post = problem_of(inp).all(*oracle_codes(inp))
    tol, rms = tol_for(inp)
    check_close(d, pre, tol, rms, "D")
    check_close(p, post, tol, rms, "PostAct")
    d0, p0, _ = run_hip(inp, tail_split=-1)
    assert np.array_equal(d, d0)
    assert np.array_equal(p, p0)


def test_split_tail_dense():
    # T = P + P/16 tiles; the last P/16 (the last M-block row, 100 rows, so the lower
    # quarters lie wholly outside the output) form the tail
    P = torch.cuda.get_device_properties(0).multi_processor_count
    if P % 16:
        pytest.skip(f"{P} CUs: shape below assumes a multiple of 16")
    tm = P // 16 + 1
    inp = small(256 * (tm - 1) + 100, 4024, 72, 1, "bf16", c_dt="f32", d_dt="bf16", post_dt="bf16",
                act="gelu_tanh", alpha=0.5, beta=0.75, seed=40, gen=lambda s, sh, dt: W.normal(s, sh, dt, 0.5))
    announce(f"split tail dense M={inp.M} N={inp.N} K={inp.K}")
    _check_split(inp)


def test_split_tail_varlen():
    # groups of 256-row blocks summing to (P + P/16) / 2 blocks with N = 392 (two N-blocks):
    # T = P + P/16 map tiles; the last group ends 156 rows short of a block
    P = torch.cuda.get_device_properties(0).multi_processor_count
    if P % 32:
        pytest.skip(f"{P} CUs: shape below assumes a multiple of 32")
    blocks = [30, 0, 17, 1, 40, 16]
    blocks.append((P + P // 16) // 2 - sum(blocks))
    assert blocks[-1] > 0
    sizes = [256 * b - (156 if i % 2 == 0 and b else 0) for i, b in enumerate(blocks)]
    sizes[-1] = 256 * blocks[-1] - 156
    inp = varlen_small(sizes, N=392, K=64, seed=41, act="relu_sq")
    announce(f"split tail varlen sizes={sizes}")
    _check_split(inp)


# ---------------------------------------------------------------------------------------
# persistent schedule and FastDivmod, bit for bit
# ---------------------------------------------------------------------------------------

def device_schedule(inp, P, max_iters, **tuning):
    log = torch.full((P * max_iters * 4,), -1, dtype=torch.int32, device="cuda")
    run_hip(inp, tile_log=log, max_iters=max_iters, **tuning)
    return log.view(P, max_iters, 4).cpu().numpy()


@pytest.mark.parametrize("M,N,L,G,xcd,tile,along_n", [(2560, 2176, 2, 8, 0, (256, 256), False),
                                                      (2560, 2176, 1, 4, 1, (128, 128), False),
                                                      (1280, 4224, 3, 16, 0, (128, 128), False),
                                                      (5000 - 8, 512, 1, 1, 0, (256, 256), False),
                                                      (1280, 4224, 2, 8, 1, (256, 256), True),
                                                      (2560, 2176 - 64, 1, 4, 0, (128, 128), True)])
def test_tile_schedule_dense(M, N, L, G, xcd, tile, along_n):
    inp = small(M, N, 16, L, "bf16", d_dt="bf16", seed=14)
    tm, tn = -(-M // tile[0]), -(-N // tile[1])
    T = tm * tn * L
    plan_args = dict(tile=tile, group_m=G, xcd_remap=1 if xcd else -1, raster_order=2 if along_n else 1)
    _, _, plan = run_hip(inp, **plan_args)
    _, _, Gp, xr, Tp, P = plan.grid()
    assert (Gp, Tp, xr) == (G, T, 1 if xcd else 0)
    max_iters = -(-T // P) + 1
    log = device_schedule(inp, P, max_iters, **plan_args)
    want = oracle.tile_schedule(P, T, lambda t: oracle.tile_dense(t, tm, tn, G, along_n), bool(xcd))
    for b in range(P):
        seq = want[b]
        got = log[b]
        assert [tuple(x[:3]) for x in got[:len(seq)]] == [tuple(s) for s in seq], b
        assert (got[len(seq):] == -1).all()
        assert [x[3] for x in got[:len(seq)]] == [oracle.wg_tile(b, i, P, bool(xcd)) for i in range(len(seq))]


def test_raster_along_n_results():
    # same outputs bit for bit as the M raster (only the tile order changes), and the oracle
    inp = small(1000, 1304, 136, 2, "bf16", c_dt="bf16", d_dt="bf16", post_dt="bf16", act="silu",
                beta=0.5, seed=44, gen=lambda s, sh, dt: W.normal(s, sh, dt, 0.5))
    d_n, p_n, _, _ = compare_full(inp, raster_order=2, group_m=4)
    d_m, p_m, _ = run_hip(inp, raster_order=1, group_m=4)
    assert np.array_equal(d_n, d_m) and np.array_equal(p_n, p_m)


def test_autotune_caches_the_tuned_choice():
    from gemm_epilogue_persistent_amd import configs, gemm, tuned_config
    inp = small(1100, 1200, 64, 1, "bf16", d_dt="bf16", seed=46)
    d_ref, _, _ = run_hip(inp)
    A, B = to_dev(inp.A), to_dev(inp.B)
    D = out_like(inp, "bf16")
    cands = configs()[::7]
    first = tuned_config(A, B, D=D, candidates=cands, steps=2, warmup=1)
    assert first in cands
    assert tuned_config(A, B, D=D, candidates=[]) == first  # cached: not timed again
    D.fill_(float("nan"))
    gemm(A, B, D, autotune=True)
    torch.cuda.synchronize()
    assert np.array_equal(D.double().cpu().numpy(), d_ref)


def test_tune_picks_a_config_with_identical_results():
    from gemm_epilogue_persistent_amd import configs, tune
    inp = small(1100, 1200, 64, 1, "f16", d_dt="f16", seed=45)
    d_ref, _, _ = run_hip(inp)
    A, B = to_dev(inp.A), to_dev(inp.B)
    D = out_like(inp, "f16")
    cands = configs()[::5]
    best, timed = tune(A, B, D=D, candidates=cands, steps=2, warmup=1)
    assert best in cands and len(timed) == len(cands)
    assert all(ms > 0 for ms, _ in timed)
    d_best, _, _ = run_hip(inp, **best)
    assert np.array_equal(d_best, d_ref)


@pytest.mark.parametrize("tile", [(128, 128), (256, 256)])
def test_tile_schedule_varlen(tile):
    inp = varlen_small([0, 300, 0, 1, 129, 0, 700, 256], N=520, K=16)
    cu = inp.cu_seqlens
    tn = -(-inp.N // tile[1])
    T = oracle.tile_count_varlen(cu, tile[0], tile[1], inp.N)
    _, _, plan = run_hip(inp, tile=tile, group_m=2)
    P = plan.grid()[5]
    max_iters = -(-T // P) + 1
    log = device_schedule(inp, P, max_iters, tile=tile, group_m=2)
    want = oracle.tile_schedule(P, T, lambda t: oracle.tile_varlen(t, cu, tile[0], tn, 2), True)
    for b in range(P):
        seq = want[b]
        assert [tuple(x[:3]) for x in log[b][:len(seq)]] == [tuple(s) for s in seq], b
        assert (log[b][len(seq):] == -1).all()


# dynamic schedule (gemm_run_dynamic): results equal the static schedule's bit for bit;
# every tile is taken exactly once, each workgroup starts on its static first tile and takes
# the rest, in increasing order, from its own queue; the counters are zero afterwards

def _dynamic_log_check(log, T, P, xcd, tile_fn):
    xq = bool(xcd) and P % 8 == 0
    Q = P // 8 if xq else P
    seen = []
    for b in range(P):
        ts = [int(x[3]) for x in log[b] if x[3] != -1]
        for x in log[b]:
            if x[3] != -1:
                assert tuple(int(v) for v in x[:3]) == tuple(tile_fn(int(x[3]))), (b, x)
        if ts:
            assert ts[0] == oracle.wg_tile(b, 0, P, xq), b
            assert ts == sorted(ts) and len(set(ts)) == len(ts), b
            qx = b % 8 if xq else 0
            assert all(qx * Q <= t % P < (qx + 1) * Q for t in ts), b
        seen += ts
    assert sorted(seen) == list(range(T))


@pytest.mark.parametrize("xcd", [1, 0])
def test_dynamic_schedule_dense(xcd):
    inp = small(8192 - 40, 4096 + 200, 24, 1, "bf16", d_dt="bf16", seed=42)
    announce(f"dynamic dense xcd={xcd} M={inp.M} N={inp.N}")
    tune = dict(xcd_remap=1 if xcd else -1, raster_order=1)
    d_static, _, plan = run_hip(inp, **tune)
    _, _, G, _, T, P = plan.grid()
    tm, tn = -(-inp.M // 256), -(-inp.N // 256)
    ctr = torch.zeros(8, dtype=torch.int32, device="cuda")
    log = torch.full((P * T * 4,), -1, dtype=torch.int32, device="cuda")
    d_dyn, _, _ = run_hip(inp, tile_log=log, max_iters=T, tile_counters=ctr, **tune)
    assert (ctr.cpu() == 0).all()
    assert np.array_equal(d_dyn, d_static)
    _dynamic_log_check(log.view(P, T, 4).cpu().numpy(), T, P, xcd, lambda t: oracle.tile_dense(t, tm, tn, G))
    # without a log (the split tail applies), three calls in a row on the same counters
    for _ in range(3):
        d_dyn, _, _ = run_hip(inp, tile_counters=ctr, **tune)
        assert np.array_equal(d_dyn, d_static)
    assert (ctr.cpu() == 0).all()
    # the static result against the oracle at sampled points
    pts = sample_points(inp, 2000, 3)
    pre, _ = problem_of(inp).points(*oracle_codes(inp), pts)
    tol, rms = tol_for(inp)
    check_close(gather(d_static, pts, False), pre, tol, rms, "D sampled")


def test_dynamic_schedule_varlen():
    inp = varlen_small([5000, 0, 3000, 129, 700, 9000, 1, 2048], N=1000, K=16, seed=43)
    announce(f"dynamic varlen M={inp.M} N={inp.N}")
    cu = inp.cu_seqlens
    tn = -(-inp.N // 256)
    T = oracle.tile_count_varlen(cu, 256, 256, inp.N)
    d_static, p_static, plan = run_hip(inp)
    P = plan.grid()[5]
    assert T > P
    ctr = torch.zeros(8, dtype=torch.int32, device="cuda")
    log = torch.full((P * T * 4,), -1, dtype=torch.int32, device="cuda")
    d_dyn, p_dyn, _ = run_hip(inp, tile_log=log, max_iters=T, tile_counters=ctr)
    assert (ctr.cpu() == 0).all()
    assert np.array_equal(d_dyn, d_static) and np.array_equal(p_dyn, p_static)
    G = plan.grid()[2]
    _dynamic_log_check(log.view(P, T, 4).cpu().numpy(), T, P, 1,
                       lambda t: oracle.tile_varlen(t, cu, 256, tn, G))
    for _ in range(2):
        d_dyn, p_dyn, _ = run_hip(inp, tile_counters=ctr)
        assert np.array_equal(d_dyn, d_static) and np.array_equal(p_dyn, p_static)
    assert (ctr.cpu() == 0).all()
    pts = sample_points(inp, 2000, 4)
    pre, post = problem_of(inp).points(*oracle_codes(inp), pts)
    tol, rms = tol_for(inp)
    check_close(gather(d_static, pts, True), pre, tol, rms, "D sampled")
    check_close(gather(p_static, pts, True), post, tol, rms, "PostAct sampled")


def test_fastdivmod_device_exhaustive_below_2_16():
    from gemm_epilogue_persistent_amd import fastdivmod_check
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    fastdivmod_check(1, 1 << 16, 1 << 16, bad)
    # the largest divisors with every dividend in [0, 2^31)
    fastdivmod_check((1 << 31) - 16, (1 << 31) - 1, 1 << 31, bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0


# ---------------------------------------------------------------------------------------
# the five workloads at full size (sampled outputs) and the guards that isolate the GEMM
# ---------------------------------------------------------------------------------------

def full_size(inp, seed=0, every_tile_row=False, **kw):
    """Full-size run checked on a deterministic sample that touches every output tile (one
    point per wave sub-tile of each tile, plus the output's corners) and on whole rows: one
    per M-block with every_tile_row, else two."""
    announce(f"{inp.name} full size")
    d, p, plan = run_hip(inp, **kw)
    TM, TN = plan.grid()[:2]
    prob = problem_of(inp)
    codes = oracle_codes(inp)
    pts = np.concatenate([tile_cover_points(inp, TM, TN, seed), sample_points(inp, 0, seed)])
    pre, post = prob.points(*codes, pts)
    tol, rms = tol_for(inp)
    if d is not None:
        check_close(gather(d, pts, inp.varlen), pre, tol, rms, "D sampled")
    if p is not None:
        check_close(gather(p, pts, inp.varlen), post, tol, rms, "PostAct sampled")
    rr = tile_rows(inp, TM, seed + 1)
    if not every_tile_row:
        rr = rr[np.random.Generator(np.random.PCG64(seed + 2)).choice(len(rr), size=min(2, len(rr)), replace=False)]
    rpre, rpost = prob.rows(*codes, rr)
    for i, (l, m) in enumerate(rr):
        if d is not None:
            check_close(d[m] if inp.varlen else d[l, m], rpre[i], tol, rms, "D row")
        if p is not None:
            check_close(p[m] if inp.varlen else p[l, m], rpost[i], tol, rms, "PostAct row")
    # every output element was written
    for x in (d, p):
        if x is not None:
            assert np.isfinite(x).all()
    return d, p


def test_workload_plain_256_full():
    compare_full(W.plain_256())


def test_workload_act_4096():
    full_size(W.act_4096())


def test_workload_act_4096_gemm_only_guard():
    # beta = 0 and no activation: the GEMM term alone must match
    full_size(W.act_4096(beta=0.0, act="none"))


def test_workload_square_8192_f16():
    full_size(W.square_8192("f16"), every_tile_row=True)


def test_workload_square_8192_bf16():
    full_size(W.square_8192("bf16"), every_tile_row=True)


def test_workload_batched_2048():
    full_size(W.batched_2048())


def test_workload_fp8_8192():
    full_size(W.fp8_8192(), every_tile_row=True)


def test_workload_varlen_moe():
    full_size(W.varlen_moe(), every_tile_row=True)


def test_workload_varlen_moe_unscaled_guard():
    # N(0,1) inputs: SiLU of O(64) values, far from the all-zero output
    full_size(W.varlen_moe(std=1.0))
