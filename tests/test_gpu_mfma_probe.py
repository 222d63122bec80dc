"""The MFMA rate probe (a measurement aid in the bench-only probe library, not a step
of the path) computes what it claims: every wave's accumulator total equals the
closed form iters * sum over chains c, lane halves h and positions t of (sum of
operand A over the half's 32 lanes) times (sum of operand B over them) -- exact, for
int8 (32x32x32) and bf16 (32x32x16) with small integer operands.  The operand
formulas are the kernel's."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd.probe as probe
    return probe


def _i8(lane, s, t, which):
    return ((lane * 7 + t * 13 + s * 29 + which * 71) % 255) - 127


def _bf16(lane, s, t, which):
    return ((lane * 3 + t * 5 + s * 7 + which * 11) % 15) - 7


def _wave_total(kind, iters):
    f, positions = (_i8, 16) if kind == "int8" else (_bf16, 8)
    total = 0
    for c in range(4):
        sa, sb = c & 1, c >> 1
        for h in range(2):
            for t in range(positions):
                a = sum(f(l + 32 * h, sa, t, 0) for l in range(32))
                b = sum(f(l + 32 * h, sb, t, 1) for l in range(32))
                total += a * b
    return iters * total


@pytest.mark.parametrize("kind", ["int8", "bf16"])
def test_probe_accumulates_the_closed_form(probe, kind):
    iters, blocks = 5, 3
    sink = probe.mfma_rate(kind, iters, blocks)
    torch.cuda.synchronize()
    per_lane = sink.cpu().numpy().astype(np.int64).reshape(blocks * 4, 64)
    want = _wave_total(kind, iters)
    assert want != 0
    assert np.all(per_lane.sum(axis=1) == want), (per_lane.sum(axis=1)[:4], want)
