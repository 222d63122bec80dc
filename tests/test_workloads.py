"""The seeded input generators (CPU): same seed, same tensors; the ``rows`` cut keeps
the full draw's first rows; the device-side draws have the stated dtypes, ranges
and code sets (run here on the CPU device)."""
import numpy as np
import torch

import workloads as W


def test_make_inputs_is_seeded_and_rows_cut_matches():
    wl = W.custom("linear", 70, 256, 24, 128, seed=31)
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    assert torch.equal(a.x, b.x) and torch.equal(a.w, b.w) and torch.equal(a.bias, b.bias)
    cut = W.make_inputs(wl, rows=17)
    assert torch.equal(cut.x, a.x[:17]) and torch.equal(cut.w, a.w)
    assert len(a.outliers) == wl.n_outliers


def test_device_draws_on_cpu():
    x = W.device_normal_bf16(64, 512, seed=1, device="cpu", outlier_frac=0.01, outlier_factor=50.0,
                             sigma=0.5)
    assert x.dtype == torch.bfloat16 and x.shape == (64, 512)
    assert torch.equal(x, W.device_normal_bf16(64, 512, seed=1, device="cpu", outlier_frac=0.01,
                                               outlier_factor=50.0, sigma=0.5))
    col_max = x.float().abs().amax(0)
    assert int((col_max > 10).sum()) >= 1          # the scaled columns stand out

    c = W.device_codes((4096,), seed=2, device="cpu")
    assert c.dtype == torch.int8 and int(c.min()) >= -127 and int(c.max()) <= 127

    e = W.device_e4m3_codes((1 << 14,), seed=3, device="cpu").numpy()
    assert e.dtype == np.uint8
    expo = (e >> 3) & 0xF
    assert expo.min() == 4 and expo.max() == 11       # every code finite, never 0x7F / 0xFF
    assert not np.any((e & 0x7F) == 0x7F)
    dec = torch.from_numpy(e).view(torch.float8_e4m3fn).float()
    assert torch.isfinite(dec).all() and float(dec.abs().min()) >= 2.0 ** -3

    s = W.device_scales(1000, seed=4, device="cpu", lo=1e-4, hi=1e-1)
    assert s.dtype == torch.float32 and float(s.min()) >= 1e-4 * (1 - 1e-6) and float(s.max()) <= 0.1 * (1 + 1e-6)
    b = W.device_bias_bf16(100, seed=5, device="cpu")
    assert b.dtype == torch.bfloat16 and float(b.float().abs().max()) < 0.1
