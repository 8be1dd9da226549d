"""Device peak probes (measurement support): a streaming copy really copies,
and the measured rates fall between zero and the datasheet figures with room
for clock and board variation."""
import pytest
import torch

import decode_token_rmsnorm_amd as wm

pytestmark = pytest.mark.gpu


def test_peak_stream_copies_and_reports_plausible_rates():
    n = 64 << 20  # 256 MiB of int32
    src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    copy = wm.peak_stream(src, dst, iters=3)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    read = wm.peak_stream(src, None, iters=3)
    print(f"copy {copy:.0f} GB/s, read {read:.0f} GB/s")
    assert 500.0 < copy < 9000.0
    assert 500.0 < read < 9000.0


def test_peak_mfma_reports_plausible_rate():
    tf = wm.peak_mfma_bf16(iters=3)
    print(f"bf16 MFMA loop {tf:.0f} TFLOP/s")
    assert 200.0 < tf < 2800.0
