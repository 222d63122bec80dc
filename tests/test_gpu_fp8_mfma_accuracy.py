"""How accurately the gfx950 matrix instructions sum E4M3FN products -- the measurement
behind the FP8 GEMM's instruction choice.

The FP8 W8A8 scheme ("clef-flash-FP8" card, Quantization table) multiplies E4M3
activations by E4M3 weights and accumulates in fp32.  On fp8-shaped data (the fp8
workload's recipe: N(0, 1) activations with 1% outlier channels x20, N(0, 0.02)
weights, K = 4,096, both quantized by the oracle), the bench-only probe library
computes the contraction four ways -- the fp8 MFMA (32x32x16, chained), the scaled
f8f6f4 MFMA (32x32x64, chained), the fp8 MFMA with every partial sum added in fp32 by
the VALU, and exact widening to bf16 on the bf16 MFMA (the library's route) -- and
each is compared with the oracle's exact sums (``orc.gemm_fp8``), then through the
dequant epilogue with the bf16 output tolerance (max relative error 1e-2, the error
taken relative to max(|ref|, 1e-3 * rms(ref)); 99.9% within 2 bf16 ulps).

Asserted: the bf16 route sums to fp32 accuracy and passes the output tolerance; each
fp8 MFMA route's error and tolerance outcome is measured and printed, and the
library's choice (bf16 route) is asserted to be the one that passes -- if a route
through the fp8 instructions met the tolerance, this test fails, flagging that the
GEMM should move onto it.

A second, independent fp8-MFMA implementation is measured the same way: the vendor
library's fp8 GEMM (hipBLASLt through torch._scaled_mm, row-wise scales, bf16 output)
on the fp8 workload at its full size (16,384 x 4,096 x 12,288), with codes and scales
from the oracle's quantizer, on sampled rows against the oracle's epilogue.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import REL_TOL, ULP_FRAC, ULPS, bits_to_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd.probe as probe
    return probe


def _output_stats(y_bits, ref_bits):
    got, ref = bits_to_f64(y_bits), bits_to_f64(ref_bits)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), 1e-3 * rms)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    return float(rel.max()), float((err <= ULPS * ulp).mean())


def test_fp8_contraction_accuracy(probe, orc):
    M, K, N = 512, 4096, 512
    wl = W.custom("fp8", M, K, N, 0, bias=False, outlier_frac=0.01, outlier_factor=20.0, seed=4242)
    inp = W.make_inputs(wl)
    qx, s_tok = orc.quantize_fp8(W.bits(inp.x), 0)
    wq, s_ch = orc.quantize_fp8(W.bits(inp.w), 0)
    exact = orc.gemm_fp8(qx, wq)                      # fp64, exact
    y_ref = orc.fp8_gemm_dequant(qx, s_tok, wq, s_ch, None)
    rms = float(np.sqrt(np.mean(exact * exact)))
    dev = torch.device("cuda")
    a, b = torch.from_numpy(qx).to(dev), torch.from_numpy(wq).to(dev)
    scale = s_tok[:, None].astype(np.float64) * s_ch[None, :].astype(np.float64)
    results = {}
    for kind in probe.FP8_KINDS:
        c = probe.fp8_contraction(kind, a, b)
        torch.cuda.synchronize()
        c = c.cpu().numpy().astype(np.float64)
        err = np.abs(c - exact)
        y = orc.bf16_from_f64(c * scale)
        max_rel, within = _output_stats(y, y_ref)
        passes = max_rel <= REL_TOL and within >= ULP_FRAC
        results[kind] = (float(err.max() / rms), float(err.mean() / rms), max_rel, within, passes)
        say(f"  {kind}: |err|/rms max {err.max() / rms:.3e} mean {err.mean() / rms:.3e}; output max rel "
            f"{max_rel:.3e}, within 2 ulp {within:.6f} -> {'passes' if passes else 'fails'} the tolerance")
    # the library's route: fp32-accurate sums (a few fp32 roundings of the running sum)
    assert results["bf16_widened"][0] < 1e-5 and results["bf16_widened"][4]
    # the fp8 instructions: measured; none meets the output tolerance at this shape
    for kind in ("fp8_32x32x16", "f8f6f4_32x32x64", "fp8_32x32x16_fp32_adds"):
        assert not results[kind][4], f"{kind} meets the output tolerance: the fp8 GEMM should use it"


def test_vendor_fp8_gemm_accuracy(orc):
    wl = W.WORKLOADS["fp8_16384x4096x12288"]
    inp = W.make_inputs(wl)
    qx, s_tok = orc.quantize_fp8(W.bits(inp.x), 0)
    wq, s_ch = orc.quantize_fp8(W.bits(inp.w), 0)
    M, K = qx.shape
    N = wq.shape[0]
    dev = torch.device("cuda")
    a8 = torch.from_numpy(qx).to(dev).view(torch.float8_e4m3fn)
    b8 = torch.from_numpy(wq).to(dev).view(torch.float8_e4m3fn)
    sa = torch.from_numpy(s_tok).to(dev).view(M, 1).contiguous()
    sb = torch.from_numpy(s_ch).to(dev).view(1, N).contiguous()
    try:
        y = torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
    except Exception as e:   # no fp8 GEMM with row-wise scales in this torch build
        pytest.skip(f"torch._scaled_mm with row-wise scales unavailable: {e!r}"[:200])
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).choice(M, 30, replace=False)]))
    y_ref = orc.fp8_gemm_dequant(qx[rows], s_tok[rows], wq, s_ch, None)
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    max_rel, within = _output_stats(got, y_ref)
    passes = max_rel <= REL_TOL and within >= ULP_FRAC
    say(f"  vendor fp8 GEMM ({len(rows)} rows x {N}): output max rel {max_rel:.3e}, within 2 ulp "
        f"{within:.6f} -> {'passes' if passes else 'fails'} the tolerance")
    assert within > 0.99, "the vendor fp8 GEMM is far off: check the operand layout of this test"
    assert not passes, "the vendor fp8 GEMM meets the output tolerance: the fp8 MFMA route should be reconsidered"
