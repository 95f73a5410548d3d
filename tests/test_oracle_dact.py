"""Pins for the oracle's activation-backward epilogue (page 6, quack/gemm_dact_sm90.py).

act'(x) is checked against central differences of the oracle's own forward activations
(which test_oracle_gemm.py pins to torch / scipy routines), against closed-form values, and
against the identities that follow from act(x) - act(-x) = x for GELU-tanh and SiLU
(act'(x) + act'(-x) = 1). The GEMM with dact is checked on small integers, where dout is
exact: D = dout * act'(C) and PostAct = act(C) element by element from numpy, and with no
activation D = dout, PostAct = C exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

SMOOTH = ["gelu_tanh", "silu"]


@pytest.mark.parametrize("act", ["relu", "relu_sq", "gelu_tanh", "silu"])
def test_derivative_matches_central_difference(act):
    h = 1e-5
    for x in np.linspace(-7.0, 7.0, 281):
        if act in ("relu", "relu_sq") and abs(x) < 1e-3:
            continue  # kink at 0
        num = (oracle.act(act, x + h) - oracle.act(act, x - h)) / (2 * h)
        assert abs(oracle.dact(act, x) - num) <= 1e-7 * (1 + abs(num)), (act, x)


def test_closed_forms():
    assert oracle.dact("none", 3.5) == 1.0
    assert oracle.dact("relu", 2.0) == 1.0 and oracle.dact("relu", -2.0) == 0.0
    assert oracle.dact("relu", 0.0) == 0.0  # the derivative at the kink taken as 0
    assert oracle.dact("relu_sq", 3.0) == 6.0 and oracle.dact("relu_sq", -1.0) == 0.0
    assert oracle.dact("gelu_tanh", 0.0) == 0.5
    assert oracle.dact("silu", 0.0) == 0.5
    assert abs(oracle.dact("gelu_tanh", 12.0) - 1.0) < 1e-12
    assert abs(oracle.dact("gelu_tanh", -12.0)) < 1e-12
    assert abs(oracle.dact("silu", 40.0) - 1.0) < 1e-12
    assert abs(oracle.dact("silu", -40.0)) < 1e-12


@pytest.mark.parametrize("act", SMOOTH)
def test_odd_identity(act):
    # act(x) - act(-x) = x  =>  act'(x) + act'(-x) = 1
    for x in np.linspace(0.0, 9.0, 91):
        assert abs(oracle.dact(act, x) + oracle.dact(act, -x) - 1.0) < 1e-13, (act, x)


def _int_case(act, c_dt="bf16", seed=3):
    r = np.random.Generator(np.random.PCG64(seed))
    M, N, K, L = 24, 40, 32, 2
    a = r.integers(-3, 4, size=(L, M, K)).astype(np.float64)
    b = r.integers(-3, 4, size=(L, N, K)).astype(np.float64)
    c = r.integers(-6, 7, size=(L, M, N)).astype(np.float64) / 2.0  # exact in bf16 / f16
    inp = W.Inputs("dact_ints", M, N, K, L, "bf16", "bf16", W.to_dtype(a, "bf16"), W.to_dtype(b, "bf16"),
                   C=W.to_dtype(c, c_dt), c_dt=c_dt, d_dt="f32", post_dt="f32", act=act, alpha=0.5,
                   dact=True)
    dout = 0.5 * np.einsum("lmk,lnk->lmn", a, b)
    prob = oracle.problem_from(inp)
    codes = (W.codes_of(inp.A), W.codes_of(inp.B), W.codes_of(inp.C))
    return prob.all(*codes), dout, c


@pytest.mark.parametrize("act", ["none", "relu", "relu_sq", "gelu_tanh", "silu"])
def test_dact_gemm_small_integers(act):
    (d, post), dout, c = _int_case(act)
    fwd = np.vectorize(lambda x: oracle.act(act, x))
    der = np.vectorize(lambda x: oracle.dact(act, x))
    if act == "none":
        assert np.array_equal(d, dout) and np.array_equal(post, c)
    elif act == "relu":
        assert np.array_equal(d, np.where(c > 0, dout, 0.0))
        assert np.array_equal(post, np.maximum(c, 0.0))
    elif act == "relu_sq":
        assert np.array_equal(d, dout * 2.0 * np.maximum(c, 0.0))
        assert np.array_equal(post, np.maximum(c, 0.0) ** 2)
    else:
        assert np.allclose(d, dout * der(c), rtol=1e-15, atol=0)
        assert np.allclose(post, fwd(c), rtol=1e-15, atol=0)


def test_dact_ignores_beta_and_postact_ignores_the_product():
    r = np.random.Generator(np.random.PCG64(5))
    M, N, K = 16, 24, 8
    c = r.normal(size=(1, M, N))
    mk = lambda a: W.Inputs("d", M, N, K, 1, "bf16", "bf16", W.to_dtype(a, "bf16"),
                            W.to_dtype(r.normal(size=(1, N, K)), "bf16"), C=W.to_dtype(c, "f32"),
                            c_dt="f32", d_dt="f32", post_dt="f32", act="gelu_tanh", dact=True)
    inp = mk(r.normal(size=(1, M, K)))
    codes = (W.codes_of(inp.A), W.codes_of(inp.B), W.codes_of(inp.C))
    d1, p1 = oracle.problem_from(inp).all(*codes)
    d2, p2 = oracle.problem_from(inp, beta=3.0).all(*codes)
    assert np.array_equal(d1, d2) and np.array_equal(p1, p2)
    # a zero product: D = 0, PostAct unchanged (it depends on C alone)
    zero = W.codes_of(W.to_dtype(np.zeros((1, M, K)), "bf16"))
    d3, p3 = oracle.problem_from(inp).all(zero, codes[1], codes[2])
    assert (d3 == 0).all() and np.array_equal(p3, p1)
