"""The bf16 MFMA calibration loop (the measured roofline denominator) runs
through the C ABI and leaves finite values."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_window_attention_amd")


def test_calib_mfma_runs():
    sink = torch.full((64,), float("nan"), dtype=torch.float32, device="cuda")
    flops = S.calib_mfma(sink, 64, 50)
    torch.cuda.synchronize()
    assert flops == 64 * 8 * 50 * 4 * 32768
    assert torch.isfinite(sink).all()
