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


@pytest.mark.parametrize("d,nq_keep,e4m3,t_past", [
    (128, 32, False, 32768), (128, 32, True, 32768), (128, 32, False, 1000),
    (64, 40, False, 5000), (256, 32, False, 3000), (128, 1, False, 16384), (128, 32, False, 0),
])
def test_read_calibration_runs(gpu, d, nq_keep, e4m3, t_past):
    """The bare read of the scoring pass's keys (measurement only) runs for
    every ring and head dim, and leaves its sink alone."""
    qk = gpu
    bcp = max(nq_keep, 64)
    shape = qk.Shape(b=2, nq=8, nkv=2, d=d, bcp=bcp, t_past=t_past, kv_cap=t_past + bcp,
                     nq_keep=nq_keep, bsa=max(1, t_past // 4), scale=0.0, dtype=qk.QK_BF16)
    g = torch.Generator(device="cuda:0").manual_seed(7)
    k = torch.randn(2, 2, t_past + bcp, d, device="cuda:0", generator=g).to(torch.bfloat16)
    if e4m3:
        k = k.view(torch.uint8)[..., :d].contiguous()
    sink = torch.full((4,), 0x0BADF00D, dtype=torch.int32, device="cuda:0")
    qk.qk_calib_read_rate(shape, k, qk.QK_KEYS_E4M3 if e4m3 else qk.QK_KEYS_DTYPE, sink)
    torch.cuda.synchronize()
    assert (sink == 0x0BADF00D).all()
