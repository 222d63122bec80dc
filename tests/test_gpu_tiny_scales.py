"""Rows and blocks whose scale is tiny (down to subnormal), on every kernel that forms codes.

The kernels form fl32(y / s) from the reciprocal of s with one correction step;
that is exact only while the residual of the step stays out of the subnormal
range, so a row whose scale is below 2^-90 is multiplied, values and scale, by
2^64 first (an exact change that leaves the quotient unchanged).  These cases put
row scales on both sides of that threshold and down to the smallest subnormals,
and require the codes and scales to equal the oracle's (IEEE division) bit for
bit: the int8 and E4M3FN quantizers (row-major and packed, rotation on and off),
the single-launch short path's workspace codes, and the quantizer of the gate/up
SwiGLU output for the next linear.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


def _unpack(flat, rows, K):
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    return flat[((r // 32) * (K // 64) + k // 64) * 2048 + (r % 32) * 64 + k % 64]


# Row magnitudes 2^e: with N(0, 1) values amax is ~3.5 * 2^e, so the int8 scale is
# ~2^(e - 5) (the fp8 one ~2^(e - 7)) -- rows below, near and above the 2^-90
# threshold, rows of bf16 subnormals (e <= -127), a row with one nonzero element,
# and a zero row.
EXPONENTS = [-150, -140, -133, -127, -120, -110, -100, -95, -90, -87, -86, -85, -84, -83, -80, -60, 0]


def _tiny_rows(K, seed):
    g = torch.Generator().manual_seed(seed)
    rows = [torch.randn(K, generator=g) * 2.0 ** e for e in EXPONENTS]
    one = torch.zeros(K)
    one[K // 3] = -3.0 * 2.0 ** -118
    rows += [one, torch.zeros(K)]
    # rows as bf16: the subnormal and underflowing ones keep what bf16 can hold
    return torch.stack(rows).to(torch.bfloat16)


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@pytest.mark.parametrize("rot", [0, 128])
def test_quantizer_on_tiny_rows(lib, orc, fp8, rot):
    K = 512
    x = _tiny_rows(K, seed=7 + rot + fp8)
    M = x.shape[0]
    say(f"tiny-scale rows, quantizer fp8={fp8} rot={rot} M={M} K={K}")
    xs = W.bits(x)
    q_ref, s_ref = (orc.quantize_fp8 if fp8 else orc.quantize_i8)(xs, rot)
    say(f"  oracle scales from {float(np.min(s_ref[s_ref > 0])):.3e} to {float(np.max(s_ref)):.3e}")
    quant = lib.w8a8_quantize_act_fp8 if fp8 else lib.w8a8_quantize_act
    quant_p = lib.w8a8_quantize_act_fp8_packed if fp8 else lib.w8a8_quantize_act_packed
    q, s = quant(x.cuda(), rot)
    qp, sp = quant_p(x.cuda(), rot)
    torch.cuda.synchronize()
    qn = q.cpu().numpy().view(np.uint8)
    ref = q_ref.view(np.uint8)
    assert np.array_equal(qn, ref), f"codes: {np.count_nonzero(qn != ref)} differ"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales"
    assert np.array_equal(_unpack(qp.cpu().numpy().view(np.uint8), M, K), ref), "packed codes"
    assert np.array_equal(sp.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "packed scales"


@pytest.mark.parametrize("rot", [0, 128])
def test_short_path_on_tiny_rows(lib, orc, rot):
    K, N = 256, 128
    x = _tiny_rows(K, seed=11 + rot)
    M = x.shape[0]
    say(f"tiny-scale rows, single-launch short path rot={rot} M={M} K={K} N={N}")
    wl = W.custom("linear", M, K, N, rot, bias=False, seed=5)
    w = W.make_inputs(wl).w
    dev = torch.device("cuda")
    wq, s_ch = lib.w8a8_quantize_act(w.to(dev), rot)
    wp = lib.w8a8_pack_weight(wq)
    ws = torch.full((lib.workspace_bytes(M, K),), 0x5A, dtype=torch.uint8, device=dev)
    lib.w8a8_linear_packed(x.to(dev), wp, N, s_ch, None, rot_block=rot, workspace=ws)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quantize_i8(W.bits(x), rot)
    flat = ws.cpu().numpy()
    got = _unpack(flat, M, K).view(np.int8)
    assert np.array_equal(got, q_ref), f"workspace codes: {np.count_nonzero(got != q_ref)} differ"
    off = (lib.packed_bytes(M, K) + 255) // 256 * 256
    assert np.array_equal(flat[off:off + 4 * M].view(np.uint32), s_ref.view(np.uint32)), "scales"


@pytest.mark.parametrize("shift", [38, 44, 50, 56])
def test_swiglu_output_quantizer_on_tiny_values(lib, orc, shift):
    """Per-channel weight scales times 2^-shift make the SwiGLU output ~2^(-2 shift), so
    the row scales of its per-token quantization run from ~2^-80 down into the
    subnormal range: on every row whose SwiGLU output equals the oracle's bit for bit
    (the quantizer's input is then the same), codes and scales equal the oracle's
    composition bit for bit; at least half the rows are such rows."""
    M, K, N, rot_out = 70, 256, 384, 128
    say(f"tiny SwiGLU output, quantized for the next linear, scales x 2^-{shift}")
    wl = W.custom("gateup", M, K, N, 0, bias=False, seed=shift)
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), 0)
    s_ch = (s_ch.astype(np.float64) * 2.0 ** -shift).astype(np.float32)
    wp = lib.w8a8_pack_weight(torch.from_numpy(wq).to(dev))
    ws = torch.empty(lib.swiglu_quant_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    q, s = lib.w8a8_gateup_swiglu_quant_packed(inp.x.to(dev), wp, N, torch.from_numpy(s_ch).to(dev), None,
                                               rot_in=0, rot_out=rot_out, workspace=ws)
    torch.cuda.synchronize()
    h_gpu = bf16_bits(lib.swiglu_quant_h(ws, M, N, K))
    x_bits = W.bits(inp.x)
    h_ref = orc.gateup_swiglu(x_bits, wq, s_ch, None, 0)
    q_ref, s_ref = orc.gateup_swiglu_quant(x_bits, wq, s_ch, None, 0, rot_out)
    say(f"  row scales from {float(np.min(s_ref[s_ref > 0])):.3e} to {float(np.max(s_ref)):.3e}")
    eq = np.all(h_gpu == h_ref, axis=1)
    say(f"  {int(eq.sum())} of {M} rows with the oracle's SwiGLU output bit for bit")
    assert eq.sum() >= M // 2
    got = _unpack(q.cpu().numpy(), M, N).view(np.int8)
    assert np.array_equal(got[eq], q_ref[eq]), f"codes: {np.count_nonzero(got[eq] != q_ref[eq])} differ"
    assert np.array_equal(s.cpu().numpy()[eq].view(np.uint32), s_ref[eq].view(np.uint32)), "scales"
