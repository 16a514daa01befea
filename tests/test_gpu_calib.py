"""The MFMA-loop ceiling kernel (ja_calibrate_mfma) computes what it claims:
with A all 1/256 and each lane's eight B values a rotation of 0..7 / 1024,
every 32x32x16 product adds (32 / 256) * (sum of B) = 0.21875 to the sum of a
wavefront's accumulator, so a wavefront's four chains after `iters` rounds
sum to 0.875 * iters (exact in fp32 at these sizes)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_loop_sums():
    import torch

    from tensor_relational_join_amd import binding as B

    wgs, iters = 8, 64
    sink = torch.zeros(wgs * 256, dtype=torch.float32, device="cuda")
    flops = B.ja_calibrate_mfma(wgs, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert flops == wgs * 4 * iters * 4 * 32768
    per_wave = sink.cpu().numpy().reshape(wgs * 4, 64).astype(np.float64).sum(axis=1)
    assert np.allclose(per_wave, 0.875 * iters, rtol=0, atol=1e-6)


def test_streaming_copy_is_exact():
    """ja_calibrate_copy moves every byte: sizes that fill whole rounds of the
    grid and sizes that end mid-round, with the bytes around the destination
    left untouched."""
    import torch

    from tensor_relational_join_amd import binding as B

    stream = torch.cuda.current_stream().cuda_stream
    for n in (16, 4096 * 16, (1 << 24) + 48, 3 * (1 << 20) + 16 * 7):
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
        B.ja_calibrate_copy(src.data_ptr(), dst.data_ptr() + 128, n, stream)
        torch.cuda.synchronize()
        assert torch.equal(dst[128:128 + n], src)
        assert not dst[:128].any() and not dst[128 + n:].any()
