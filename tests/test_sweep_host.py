"""Host check of the GPU sweep's cases: every case the seeded sweep draws must be a problem
gemm_create accepts (no GPU work; CPU tensors with the same layouts), so that the sweep
covers the whole accepted range rather than failing on validation."""
import pytest

import workloads as W
from gemm_epilogue_persistent_amd import describe, gemm_create, _abi
from test_gpu_sweep import CASES, draw_case


def test_every_sweep_case_is_accepted():
    lib = _abi.load()
    seen_units = set()
    for i in range(CASES):
        inp, tile, m_major_out, desc = draw_case(i)
        D = W.out_like(inp, inp.d_dt, m_major_out, device="cpu") if inp.d_dt != "none" else None
        P = W.out_like(inp, inp.post_dt, m_major_out, device="cpu") if inp.post_dt != "none" else None
        kw = {} if tile is None else {"tile": tile}
        d = describe(inp.A, inp.B, inp.C, D, P, inp.alpha, inp.beta, inp.act, inp.varlen, **kw,
                     varlen_k=(len(inp.cu_seqlens_k) - 1) if inp.cu_seqlens_k is not None else 0,
                     gather=inp.a_idx is not None)
        h = gemm_create(d)  # raises with the library's message on rejection
        lib.gemm_destroy(h)
        contig = inp.M if m_major_out else inp.N
        seen_units.add(contig % 8)
    # some cases end a contiguous output extent half way through an 8-element group
    assert 4 in seen_units
