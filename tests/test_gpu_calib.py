"""The matrix-rate calibration call (measurement only) runs in every mode."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_calib_modes_run(gpu):
    qk = gpu
    out = torch.empty(256 * 512, dtype=torch.float32, device="cuda:0")
    for mode in range(8):
        qk.qk_calib_matrix_rate(mode, 2, out)
    torch.cuda.synchronize()
    with pytest.raises(qk.QKError):
        qk.qk_calib_matrix_rate(8, 2, out)
