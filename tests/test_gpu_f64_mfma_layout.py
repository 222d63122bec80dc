"""The lane layout of v_mfma_f64_4x4x4f64 that the quantizer's rotation relies on
(bench-only probe library): four independent 4x4x4 products per wave, one per group
b of lanes with equal bits 2-3, with B[k][j] in lane 16k + 4b + j, A[i][k] in lane
16k + 4b + i and D[i][j] in lane 16i + 4b + j.  With A one-hot at lane L (A[i0][k0] of
group b0) and B[lane] = lane + 1, D must be B[k0][j] = lane 16k0 + 4b0 + j, plus one, in
lane 16i0 + 4b0 + j for j = 0..3, and zero everywhere else."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_f64_4x4x4_lane_layout():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd.probe as probe
    d = probe.f64_mfma_layout()
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    want = np.zeros((64, 64))
    for L in range(64):
        k0, b0, i0 = L >> 4, (L >> 2) & 3, L & 3          # A[i0][k0] of group b0 sits in lane L
        for j in range(4):
            want[L, 16 * i0 + 4 * b0 + j] = 16 * k0 + 4 * b0 + j + 1
    assert np.array_equal(d, want), np.argwhere(d != want)[:8]
