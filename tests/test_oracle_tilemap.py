"""Pins for the oracle's tile map (plain division) and the pages' FastDivmod.

Tile map: hand-derived fixtures from the page's swizzle layout (tests/golden), bijection
onto all tiles for many shapes, special cases (tm < G, tm % G == 0, tn == 1, L > 1, empty
varlen groups), and the XCD remap being a permutation of the workgroup ids.
FastDivmod: hand-derived constants (tests/golden), an exhaustive sweep of every divisor and
dividend below 2^16 against quotient/remainder tracked by counting, an edge sweep of every
divisor below 2^20 and random pairs over the full 31-bit domain against C's '/' and '%'.
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append([int(x) for x in line.split()])
    return out


def test_golden_dense_raster():
    rows = _rows("tilemap_dense.txt")
    assert len(rows) == 30 + 6 + 12
    for tm, tn, G, t, m, n in rows:
        assert oracle.raster(t, tm, tn, G) == (m, n)
        # with L = 2 the second batch repeats the map, offset by tm*tn
        assert oracle.tile_dense(t + tm * tn, tm, tn, G) == (m, n, 1)


def test_golden_dense_raster_along_n():
    rows = _rows("tilemap_dense_n.txt")
    assert len(rows) == 16
    for tm, tn, G, t, m, n in rows:
        assert oracle.tile_dense(t, tm, tn, G, along_n=True) == (m, n, 0)
        assert oracle.tile_dense(t + tm * tn, tm, tn, G, along_n=True) == (m, n, 1)


def test_raster_along_n_bijection_and_g1():
    r = np.random.Generator(np.random.PCG64(21))
    for _ in range(60):
        tm, tn, L = int(r.integers(1, 12)), int(r.integers(1, 40)), int(r.integers(1, 4))
        G = int(2 ** r.integers(0, 5))
        T = tm * tn * L
        seen = {oracle.tile_dense(t, tm, tn, G, along_n=True) for t in range(T)}
        assert seen == {(m, n, l) for m in range(tm) for n in range(tn) for l in range(L)}
        assert len(seen) == T
    # G == 1 along N: groups of one N-block each, M fastest inside, i.e. M runs fastest
    assert [oracle.tile_dense(t, 3, 4, 1, along_n=True)[:2] for t in range(12)] == \
        [(t % 3, t // 3) for t in range(12)]


def test_golden_varlen():
    cu = [0, 0, 300, 300, 428]
    for t, m, n, g in _rows("tilemap_varlen.txt"):
        assert oracle.tile_varlen(t, cu, 128, 2, 2) == (m, n, g)
    assert oracle.tile_count_varlen(cu, 128, 64, 128) == 8


@pytest.mark.parametrize("seed", range(4))
def test_dense_bijection(seed):
    r = np.random.Generator(np.random.PCG64(seed))
    for _ in range(60):
        tm, tn, L = int(r.integers(1, 40)), int(r.integers(1, 12)), int(r.integers(1, 4))
        G = int(2 ** r.integers(0, 5))
        T = tm * tn * L
        seen = {oracle.tile_dense(t, tm, tn, G) for t in range(T)}
        assert len(seen) == T
        assert seen == {(m, n, l) for m in range(tm) for n in range(tn) for l in range(L)}


def test_special_cases():
    # tm < G: all tail, M fastest
    assert [oracle.raster(t, 3, 4, 8) for t in range(12)] == [(t % 3, t // 3) for t in range(12)]
    # tm % G == 0: no tail
    assert [oracle.raster(t, 16, 1, 8) for t in range(16)] == [(t, 0) for t in range(16)]
    # tn == 1 with a tail
    assert [oracle.raster(t, 10, 1, 8)[0] for t in range(10)] == list(range(10))
    # G == 1 is plain row-major over (m, n) with n fastest
    assert [oracle.raster(t, 3, 4, 1) for t in range(12)] == [(t // 4, t % 4) for t in range(12)]


def test_varlen_bijection_with_empty_groups():
    r = np.random.Generator(np.random.PCG64(9))
    for _ in range(40):
        G = int(r.integers(1, 9))
        sizes = r.integers(0, 700, size=G)
        sizes[r.random(G) < 0.3] = 0  # empty groups anywhere
        cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        TM, tn, Gsz = 128, int(r.integers(1, 5)), int(2 ** r.integers(0, 4))
        T = oracle.tile_count_varlen(cu, TM, 1, tn)
        got = {oracle.tile_varlen(t, cu, TM, tn, Gsz) for t in range(T)}
        want = {(m, n, g) for g in range(G) for m in range(-(-int(sizes[g]) // TM))
                for n in range(tn)}
        assert got == want and len(want) == T


@pytest.mark.parametrize("P", [1, 7, 8, 16, 256, 255])
def test_wg_remap_is_permutation(P):
    first = [oracle.wg_tile(b, 0, P, True) for b in range(P)]
    assert sorted(first) == list(range(P))
    if P % 8 == 0:
        # the 8 XCDs (b % 8) each own one contiguous block of P/8 tile ids
        for x in range(8):
            blk = sorted(oracle.wg_tile(b, 0, P, True) for b in range(x, P, 8))
            assert blk == list(range(x * (P // 8), (x + 1) * (P // 8)))
    else:
        assert first == list(range(P))
    assert [oracle.wg_tile(b, 2, P, False) for b in range(P)] == [b + 2 * P for b in range(P)]


def test_schedule_covers_each_tile_once():
    tm, tn, L, G = 9, 5, 2, 4
    T = tm * tn * L
    for P in (1, 8, 13, 64):
        sched = oracle.tile_schedule(P, T, lambda t: oracle.tile_dense(t, tm, tn, G), True)
        flat = [x for s in sched for x in s]
        assert len(flat) == T and len(set(flat)) == T


# ---------------------------------------------------------------------------------------
# FastDivmod
# ---------------------------------------------------------------------------------------

def test_fastdivmod_golden_constants():
    for d, mult, shift in _rows("fastdivmod_constants.txt"):
        assert oracle.fdm_create(d) == (mult, shift)


def test_fastdivmod_small_examples():
    assert oracle.fdm_divmod(100, 7) == (14, 2)
    assert oracle.fdm_divmod(17, 8) == (2, 1)
    assert oracle.fdm_divmod(12345, 1) == (12345, 0)
    assert oracle.fdm_divmod(2 ** 31 - 1, 2 ** 31 - 1) == (1, 0)
    assert oracle.fdm_divmod(2 ** 31 - 2, 2 ** 31 - 1) == (0, 2 ** 31 - 2)


def test_fastdivmod_exhaustive_below_2_16():
    # every divisor 1..2^16 and every dividend 0..2^16-1 (2^32 pairs)
    assert oracle.fdm_exhaustive(1, 1 << 16, 1 << 16) == 0


def test_fastdivmod_edges_below_2_20():
    assert oracle.fdm_edges(1, 1 << 20) == 0
    assert oracle.fdm_edges((1 << 31) - 4096, (1 << 31) - 1) == 0


def test_fastdivmod_random_full_domain():
    assert oracle.fdm_random(20_000_000, 1234) == 0


def test_fastdivmod_check_catches_a_planted_error():
    """The sweep is able to fail: a multiplier off by one breaks some quotient."""
    mult, shift = oracle.fdm_create(7)
    bad = 0
    for n in range(1 << 20):
        q = ((n * (mult - 1)) >> 32) >> shift
        bad += q != n // 7
    assert bad > 0
