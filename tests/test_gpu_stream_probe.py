"""The streaming probe (bench-only probe library, the achievable-bandwidth reference
for the quantizer) moves the bytes it claims: the high byte of every bf16 element, or
an exact copy, on a ragged element count (not a multiple of a block's pieces) and on
one past a block boundary."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [8, 8 * 1023 + 8, 8 * 4 * 256 * 3 + 8 * 5])
def test_stream_probe_bytes(n):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd.probe as probe
    g = torch.Generator().manual_seed(n)
    bits = torch.randint(0, 1 << 16, (n,), generator=g, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).cuda()
    hi = torch.full((n + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    probe.stream("bf16_to_byte", x, hi)
    cp = torch.zeros(n + 32, dtype=torch.bfloat16, device="cuda")
    probe.stream("copy", x, cp)
    torch.cuda.synchronize()
    want_hi = (bits.to(torch.int32) >> 8) & 0xFF
    assert torch.equal(hi[:n].cpu().to(torch.int32), want_hi)
    assert torch.all(hi[n:].cpu() == 0xAB)                      # nothing written past the end
    assert torch.equal(cp[:n].cpu().view(torch.int16), bits)
    assert torch.all(cp[n:].cpu().view(torch.int16) == 0)
