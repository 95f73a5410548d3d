"""GPU parity with an operand larger than 2^31 bytes: the kernels address every tile from a
64-bit base and clamp each buffer range to 2^31 - 1 bytes, so rows and k-tiles far past the
first 2 GiB of A must read the right elements. A is 40960 x 32768 bf16 (2.68 GB), K-major
or M-major; outputs are checked against the CPU oracle on sampled elements and on whole
rows near the end of A.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from parity import check_close, oracle_codes, problem_of, run_hip, sample_points, gather

pytestmark = pytest.mark.gpu

M, N, K = 40960, 256, 32768


def big_operand(rows, cols, seed):
    """(rows, cols) bf16 U[-1, 1), filled in slabs of 2048 rows, each from its own seed."""
    out = torch.empty((rows, cols), dtype=torch.bfloat16)
    for r0 in range(0, rows, 2048):
        r1 = min(rows, r0 + 2048)
        out[r0:r1] = W.uniform(seed + r0 // 2048, (r1 - r0, cols), "bf16")
    return out


@pytest.mark.parametrize("a_mmaj", [False, True])
def test_operand_over_2gib(a_mmaj):
    print(f"[case] A {M}x{K} bf16 ({M * K * 2 / 2**30:.2f} GiB) m_major={a_mmaj}", flush=True)
    sys.stdout.flush()
    if a_mmaj:
        A = big_operand(K, M, 5000).t().unsqueeze(0)  # storage [K][M]
    else:
        A = big_operand(M, K, 6000).unsqueeze(0)
    B = W.uniform(7000, (1, N, K), "bf16")
    inp = W.Inputs("large_a", M, N, K, 1, "bf16", "bf16", A, B, d_dt="bf16", alpha=0.5)
    d, _, _ = run_hip(inp)
    prob = problem_of(inp)
    codes = oracle_codes(inp)
    pts = sample_points(inp, 1500, 3)
    pts[:500, 1] = np.linspace(M - 4096, M - 1, 500).astype(np.int64)  # rows past 2 GiB of A
    pre, _ = prob.points(*codes, pts)
    check_close(gather(d, pts, False), pre, 2e-2, 1e-2, "D sampled")
    rows = np.array([[0, M - 1], [0, M - 257], [0, 33000], [0, 1]], dtype=np.int64)
    rpre, _ = prob.rows(*codes, rows)
    for i, (_, m) in enumerate(rows):
        check_close(d[0, m], rpre[i], 2e-2, 1e-2, "D row")
    assert np.isfinite(d).all()
    del A, inp
    torch.cuda.empty_cache()
