"""The benchmark's MFMA rate probe (measurement support, its own library) runs and reports
plausible counts."""
import pytest
import torch

from gemm_epilogue_persistent_amd.measure import probe_mfma

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "e4m3", "bf16_16x16", "e4m3_16x16"])
def test_probe_reports_cycles(dtype):
    blocks = 8
    out = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    probe_mfma(dtype, 200, 7, blocks, out)
    torch.cuda.synchronize()
    h = out.view(blocks, 2).cpu()
    assert (h[:, 0] > 0).all() and (h[:, 1] > 0).all()
    # 200 iterations of at least 512 MFMA cycles per wave (16 32x32 or 32 16x16 MFMAs)
    assert (h[:, 0] >= 200 * 16 * 32).all()
    mhz = h[:, 0].double() / (h[:, 1].double() / 100.0)
    assert (mhz > 100).all() and (mhz < 5000).all()


def test_probe_rejects_bad_arguments():
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        probe_mfma("f16", 10, 1, 1, out)
    with pytest.raises(ValueError):
        probe_mfma("bf16", 0, 1, 1, out)
