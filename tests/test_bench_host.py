"""Host-side logic of bench.py (no GPU): the algorithmic bytes and the roofline time.

Checked against hand-computed values: 8192^3 bf16 reads two 128 MiB operands and writes one
128 MiB output; its roofline time is FLOPs / 2.5 PFLOP/s (far above the ridge point). A
grouped problem's roofline time is the sum over its groups of max(FLOPs / peak, bytes / HBM
peak): a group of 128 rows against a 4096 x 4096 B is HBM-bound on B.
"""
import numpy as np
import pytest
import torch

import bench
import workloads as W


def dense(M, N, K, L=1, dt="bf16", d_dt="bf16"):
    A = torch.zeros((L, M, K), dtype=W.TORCH_DT[dt])
    B = torch.zeros((L, N, K), dtype=W.TORCH_DT[dt])
    return W.Inputs("t", M, N, K, L, dt, dt, A, B, d_dt=d_dt)


def test_dense_bytes_and_roof():
    inp = dense(8192, 8192, 8192)
    assert bench.algorithmic_bytes(inp) == 3 * 8192 * 8192 * 2
    assert bench.attainable_s(inp) == pytest.approx(2.0 * 8192 ** 3 / 2.5e15, rel=1e-12)


def test_hbm_bound_dense_roof():
    # M = 16: 2 * 16 * 4096 * 4096 FLOPs against ~33.8 MB -> HBM time dominates
    inp = dense(16, 4096, 4096)
    by = 16 * 4096 * 2 + 4096 * 4096 * 2 + 16 * 4096 * 2
    assert bench.algorithmic_bytes(inp) == by
    assert bench.attainable_s(inp) == pytest.approx(by / 8.0e12, rel=1e-12)


def test_varlen_roof_sums_groups():
    sizes = [128, 4096]
    cu = np.array([0, 128, 4224], dtype=np.int32)
    N = K = 4096
    A = torch.zeros((4224, K), dtype=torch.bfloat16)
    B = torch.zeros((2, N, K), dtype=torch.bfloat16)
    inp = W.Inputs("v", 4224, N, K, 2, "bf16", "bf16", A, B, post_dt="bf16", act="silu", cu_seqlens=cu)
    want = 0.0
    for m in sizes:
        fl = 2.0 * m * N * K
        by = m * K * 2 + N * K * 2 + m * N * 2
        want += max(fl / 2.5e15, by / 8.0e12)
    assert bench.attainable_s(inp) == pytest.approx(want, rel=1e-12)
    # the 128-row group is HBM-bound (its B read), the 4096-row one MFMA-bound
    assert (128 * K * 2 + N * K * 2 + 128 * N * 2) / 8.0e12 > 2.0 * 128 * N * K / 2.5e15
    assert bench.attainable_s(inp) > 2.0 * 4224 * N * K / 2.5e15


def test_cold_sets_copy_inputs_and_share_outputs():
    A, B, C, D = (torch.full((4, 4), float(i)) for i in range(4))
    sets = bench.cold_sets((A, B, C, D, None, None, None, None), 3)
    assert len(sets) == 3
    for s in sets[1:]:
        assert s[0] is not A and torch.equal(s[0], A) and s[0].data_ptr() != A.data_ptr()
        assert s[2] is not C and torch.equal(s[2], C)
        assert s[3] is D


def test_code_text_drops_comments_and_layout_only():
    # the traffic counters stay valid across comment and layout edits, not across code edits
    a = "int x = 1;  // one\n/* block\n comment */\nfloat y = x * 2;  \n\n"
    b = "// new header\nint   x = 1;\n\n  float y = x * 2; /* tail */\n"
    c = "int x = 2;\nfloat y = x * 2;\n"
    assert bench.code_text(a) == bench.code_text(b) == "int x = 1;\nfloat y = x * 2;"
    assert bench.code_text(c) != bench.code_text(a)
    # comment markers inside string and character literals are code
    s = 'const char* u = "a//b/*c*/"; char q = \'"\'; int z; // gone'
    assert bench.code_text(s) == 'const char* u = "a//b/*c*/"; char q = \'"\'; int z;'
    assert len(bench.source_hash()) == 16
