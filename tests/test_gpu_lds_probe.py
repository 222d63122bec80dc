"""The LDS read-pattern probe (bench-only probe library, the evidence for the GEMM's
LDS swizzle) reads the bytes it claims: every lane sum equals the host's sum of the
dword indices that lane's fragments cover, for each chunk placement."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pattern", ["contiguous", "rows_no_swizzle", "rows_earlier_key", "rows_gemm_key"])
def test_lds_probe_reads(pattern):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd.probe as probe
    blocks, iters = 3, 5
    out = probe.lds(pattern, iters, blocks)
    torch.cuda.synchronize()
    want = torch.tensor(probe.lds_expected(pattern, iters) * blocks, dtype=torch.int32)
    assert torch.equal(out.cpu(), want)
