"""Helpers shared by the parity tests: oracle problems from workload inputs, device copies
that keep each operand's memory layout, the HIP call through the binding, and the
tolerance checks (per element |gpu - oracle| <= tol * (|oracle| + 1), tol = 2e-2 for
16-bit inputs and 6e-2 for fp8 inputs, plus a normalised-RMS guard)."""
import numpy as np
import torch

import oracle
import workloads as W

TOL_16 = 2e-2
TOL_FP8 = 6e-2
RMS_16 = 1e-2
RMS_FP8 = 3e-2


def tol_for(inp):
    return (TOL_FP8, RMS_FP8) if inp.a_dt in ("e4m3", "e5m2") else (TOL_16, RMS_16)


def problem_of(inp, act=None, alpha=None, beta=None):
    return oracle.problem_from(inp, act=act, alpha=alpha, beta=beta)


def oracle_codes(inp):
    C = W.codes_of(inp.C) if inp.C is not None else None
    return W.codes_of(inp.A), W.codes_of(inp.B), C


to_dev = W.to_dev
out_like = W.out_like


def run_hip(inp, d_major_m=False, tile=None, alpha_dev=None, beta_dev=None, tile_log=None,
            max_iters=0, tile_counters=None, **tuning):
    """Run the HIP path on the GPU; returns (D, PostAct) as CPU float64 arrays (or None)."""
    from gemm_epilogue_persistent_amd import Plan
    A, B = to_dev(inp.A), to_dev(inp.B)
    C = to_dev(inp.C)
    D = out_like(inp, inp.d_dt, d_major_m) if inp.d_dt != "none" else None
    P = out_like(inp, inp.post_dt, d_major_m) if inp.post_dt != "none" else None
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda") if inp.varlen else None
    cuk = torch.from_numpy(inp.cu_seqlens_k).to("cuda") if inp.cu_seqlens_k is not None else None
    idx = torch.from_numpy(inp.a_idx).to("cuda") if inp.a_idx is not None else None
    if tile is not None:
        tuning["tile"] = tile
    if inp.dact:
        tuning["dact"] = True
    plan = Plan(A, B, C, D, P, inp.alpha, inp.beta, inp.act, cu, cuk, idx, **tuning)
    plan.run(A, B, C, D, P, alpha_dev, beta_dev, cu, tile_log=tile_log, max_iters=max_iters,
             tile_counters=tile_counters, cu_seqlens_k=cuk, a_idx=idx)
    torch.cuda.synchronize()
    d = None if D is None else D.double().cpu().numpy()
    p = None if P is None else P.double().cpu().numpy()
    return d, p, plan


def check_close(got, want, tol, rms_tol, what=""):
    """Per element |got - want| <= tol (|want| + 1), plus the normalised-RMS guard."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output (unwritten element?)"
    err = np.abs(got - want)
    bound = tol * (np.abs(want) + 1.0)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of bound, worst at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)}: got "
                           f"{got.flat[np.argmax(err - bound)]} want {want.flat[np.argmax(err - bound)]}")
    nrm = np.linalg.norm(want)
    if nrm > 0:
        rel = np.linalg.norm(got - want) / nrm
        assert rel <= rms_tol, f"{what}: normalised RMS error {rel:.3g} > {rms_tol}"
    return float(err.max()), float(np.linalg.norm(got - want) / max(nrm, 1e-300))


def sample_points(inp, n, seed):
    """Random (l, m, n) output coordinates plus the corners of the output."""
    r = np.random.Generator(np.random.PCG64(seed))
    L = 1 if inp.varlen else inp.L
    pts = np.stack([r.integers(0, L, n), r.integers(0, inp.M, n), r.integers(0, inp.N, n)], 1)
    corners = np.array([[l, m, c] for l in (0, L - 1) for m in (0, inp.M - 1) for c in (0, inp.N - 1)])
    return np.concatenate([pts, corners]).astype(np.int64)


def gather(arr, pts, varlen):
    if varlen:
        return arr[pts[:, 1], pts[:, 2]]
    return arr[pts[:, 0], pts[:, 1], pts[:, 2]]


def _m_blocks(inp, TM):
    """(l, first row, rows) of every M-block of the output: per batch, or per group (varlen)."""
    if inp.varlen:
        cu = inp.cu_seqlens
        return [(0, int(cu[g]) + b, min(TM, int(cu[g + 1]) - int(cu[g]) - b))
                for g in range(len(cu) - 1) for b in range(0, int(cu[g + 1]) - int(cu[g]), TM)]
    return [(l, b, min(TM, inp.M - b)) for l in range(inp.L) for b in range(0, inp.M, TM)]


def tile_cover_points(inp, TM, TN, seed, rows_split=2, cols_split=4):
    """Deterministic sample that touches every output tile: for each TM x TN tile, one point
    in each cell of a rows_split x cols_split grid over it (the wave sub-tiles of both the
    4-wave 2 x 2 and the 8-wave 2 x 4 layouts), drawn at a seeded position inside the cell
    and clipped to the output. Returns (l, m, n) triples (varlen: m is the global row)."""
    r = np.random.Generator(np.random.PCG64(seed))
    pts = []
    for l, m0, mr in _m_blocks(inp, TM):
        for n0 in range(0, inp.N, TN):
            nr = min(TN, inp.N - n0)
            for i in range(rows_split):
                for j in range(cols_split):
                    lo_m, lo_n = i * TM // rows_split, j * TN // cols_split
                    if lo_m >= mr or lo_n >= nr:
                        continue
                    hi_m = min(mr, (i + 1) * TM // rows_split)
                    hi_n = min(nr, (j + 1) * TN // cols_split)
                    pts.append((l, m0 + int(r.integers(lo_m, hi_m)), n0 + int(r.integers(lo_n, hi_n))))
    return np.array(pts, dtype=np.int64).reshape(-1, 3)


def tile_rows(inp, TM, seed):
    """One whole output row per M-block (a seeded row inside it): (l, m) pairs."""
    r = np.random.Generator(np.random.PCG64(seed))
    return np.array([(l, m0 + int(r.integers(0, mr))) for l, m0, mr in _m_blocks(inp, TM)],
                    dtype=np.int64).reshape(-1, 2)
