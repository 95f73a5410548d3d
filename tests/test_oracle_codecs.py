"""Pins for the oracle's exact decoders and round-to-nearest-even encoders.

Each check compares against something other than the oracle's own code: numpy's IEEE half
type, the bit-level definition of bfloat16 (top half of a binary32), torch's float8 casts,
the OCP 8-bit float specification's published constants, and exact rational rounding
(Python's fractions) for the double -> bf16 / fp16 encoders.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def test_decode_f16_every_code():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode_array("f16", codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, oracle.decode("f16", 0x8000)) == -1.0


def test_decode_bf16_every_code():
    codes = np.arange(65536, dtype=np.uint32)
    ours = oracle.decode_array("bf16", codes)
    ref = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("dt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decode_fp8_every_code_vs_torch(dt, tdt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_array(dt, codes)
    ref = torch.from_numpy(codes).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_ocp_constants():
    """Published values of the OCP 8-bit formats (OCP 8-bit Floating Point Specification)."""
    d = oracle.decode
    # E4M3 ("fn"): bias 7, max normal 448 = S.1111.110, NaN = S.1111.111, no infinities
    assert d("e4m3", 0x7E) == 448.0
    assert d("e4m3", 0xFE) == -448.0
    assert math.isnan(d("e4m3", 0x7F)) and math.isnan(d("e4m3", 0xFF))
    assert d("e4m3", 0x78) == 256.0  # S.1111.000 is a number, not inf
    assert d("e4m3", 0x08) == 2.0 ** -6  # min normal
    assert d("e4m3", 0x01) == 2.0 ** -9  # min subnormal
    assert d("e4m3", 0x07) == 7 * 2.0 ** -9  # max subnormal
    # E5M2: bias 15, IEEE-like
    assert d("e5m2", 0x7B) == 57344.0
    assert d("e5m2", 0x7C) == math.inf and d("e5m2", 0xFC) == -math.inf
    assert all(math.isnan(d("e5m2", c)) for c in (0x7D, 0x7E, 0x7F))
    assert d("e5m2", 0x04) == 2.0 ** -14
    assert d("e5m2", 0x01) == 2.0 ** -16


def _rne_fraction(x: float, mbits: int, emin: int, emax: int):
    """Exact round-to-nearest-even of double x to a binary format, via rationals."""
    if x == 0:
        return 0.0
    fx = Fraction(x)
    a = abs(fx)
    e = emin
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - mbits)
    q = a / ulp
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    maxfin = (2 - Fraction(2) ** (-mbits)) * Fraction(2) ** emax
    if r > maxfin:
        return math.copysign(math.inf, x)
    return math.copysign(float(r), x)


def _sample_doubles(n, seed, lo_exp, hi_exp):
    r = np.random.Generator(np.random.PCG64(seed))
    mant = r.uniform(1.0, 2.0, size=n)
    ex = r.integers(lo_exp, hi_exp, size=n)
    sign = r.choice([-1.0, 1.0], size=n)
    return sign * np.ldexp(mant, ex)


def test_encode_f16_vs_numpy_and_ties():
    xs = _sample_doubles(20000, 5, -27, 17)
    ours = oracle.encode_array("f16", xs)
    ref = xs.astype(np.float16).view(np.uint16)  # numpy rounds double -> half directly
    assert np.array_equal(ours, ref)
    # every midpoint between consecutive positive finite halves rounds to the even code
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0  # exact in double
    got = oracle.encode_array("f16", mid)
    want = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # overflow threshold: 65520 = 65504 + half ulp rounds to inf (even), just below stays
    assert oracle.encode("f16", 65520.0) == 0x7C00
    assert oracle.encode("f16", np.nextafter(65520.0, 0)) == 0x7BFF
    assert oracle.encode("f16", -1e9) == 0xFC00


def test_encode_bf16_exact_rounding():
    xs = _sample_doubles(3000, 6, -140, 129)
    got = oracle.encode_array("bf16", xs)
    for x, c in zip(xs, got):
        ref = _rne_fraction(float(x), 7, -126, 127)
        val = oracle.decode("bf16", int(c))
        assert val == ref, (x, val, ref)
    # ties between consecutive bf16 values round to even
    codes = np.arange(0x0001, 0x7F7F, 97, dtype=np.uint32)
    lo = oracle.decode_array("bf16", codes)
    hi = oracle.decode_array("bf16", codes + 1)
    got = oracle.encode_array("bf16", (lo + hi) / 2.0)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got.astype(np.uint32), want)


def test_encode_bf16_matches_torch_on_float32_inputs():
    # for values that are already binary32, torch's float -> bfloat16 cast is one RNE step
    xs = _sample_doubles(20000, 7, -130, 128).astype(np.float32).astype(np.float64)
    ours = oracle.encode_array("bf16", xs)
    ref = torch.from_numpy(xs).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_f16_subnormal_exact():
    xs = _sample_doubles(3000, 8, -26, -13)
    got = oracle.encode_array("f16", xs)
    for x, c in zip(xs, got):
        assert oracle.decode("f16", int(c)) == _rne_fraction(float(x), 10, -14, 15)


def test_encode_f32_vs_numpy():
    xs = _sample_doubles(20000, 9, -160, 128)
    ours = oracle.encode_array("f32", xs)
    assert np.array_equal(ours, xs.astype(np.float32).view(np.uint32))


def test_encode_special_values():
    for dt, inf, qnan_mask in (("f16", 0x7C00, 0x7C00), ("bf16", 0x7F80, 0x7F80)):
        assert oracle.encode(dt, math.inf) == inf
        assert oracle.encode(dt, -math.inf) == inf | (0x8000)
        c = oracle.encode(dt, math.nan)
        assert (c & qnan_mask) == qnan_mask and (c & ~(qnan_mask | 0x8000)) != 0
        assert oracle.encode(dt, -0.0) == 0x8000
        assert oracle.encode(dt, 0.0) == 0


# ---------------------------------------------------------------------------------------
# fp8 encoders (round to nearest even, saturating to the largest finite value)
# ---------------------------------------------------------------------------------------

FP8_MAXCODE = {"e4m3": 0x7E, "e5m2": 0x7B}


def _finite_codes(dt):
    return [c for c in range(256) if math.isfinite(oracle.decode(dt, c))]


@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_fp8_encode_round_trips_every_finite_code(dt):
    for c in _finite_codes(dt):
        assert oracle.encode(dt, oracle.decode(dt, c)) == c, hex(c)


@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_fp8_encode_ties_to_even_at_every_midpoint(dt):
    pos = sorted((oracle.decode(dt, c), c) for c in _finite_codes(dt) if c < 0x80)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (Fraction(v0) + Fraction(v1)) / 2
        m = float(mid)
        assert Fraction(m) == mid  # exact in double
        even = c0 if c0 % 2 == 0 else c1
        assert oracle.encode(dt, m) == even, (v0, v1)
        assert oracle.encode(dt, -m) == even | 0x80
        step = (v1 - v0) * 1e-6
        assert oracle.encode(dt, m - step) == c0 and oracle.encode(dt, m + step) == c1


@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_fp8_encode_saturates_and_keeps_nan(dt):
    top = FP8_MAXCODE[dt]
    fmax = oracle.decode(dt, top)
    assert fmax == (448.0 if dt == "e4m3" else 57344.0)
    for x in (fmax * 1.0001, fmax * 4, 1e30, math.inf):
        assert oracle.encode(dt, x) == top and oracle.encode(dt, -x) == top | 0x80
    assert math.isnan(oracle.decode(dt, oracle.encode(dt, math.nan)))
    assert oracle.encode(dt, 0.0) == 0x00 and oracle.encode(dt, -0.0) == 0x80
    # below half the smallest subnormal: zero; just above: the smallest subnormal
    tiny = oracle.decode(dt, 0x01)
    assert oracle.encode(dt, tiny * 0.49) == 0x00 and oracle.encode(dt, tiny * 0.51) == 0x01


@pytest.mark.parametrize("dt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_encode_matches_torch_in_range(dt, tdt):
    r = np.random.Generator(np.random.PCG64(17))
    fmax = oracle.decode(dt, FP8_MAXCODE[dt])
    x = (r.standard_normal(20000) * np.exp(r.uniform(-12, np.log(fmax), 20000))).astype(np.float32)
    x = x[np.abs(x) <= fmax].astype(np.float64)
    ours = oracle.encode_array(dt, x)
    ref = torch.from_numpy(x).to(torch.float32).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
