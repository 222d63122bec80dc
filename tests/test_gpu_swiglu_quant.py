"""GPU parity of the gate/up SwiGLU whose output is quantized for the next linear.

The fused path has two steps (oracle reading R7): the gate/up GEMM's epilogue
quantizes each 128-column block of the SwiGLU output h on its own scale, then
a pass rescales the blocks to the row scale.  Checked here:

* step 1 alone on the oracle's activation codes: h (written on request) against
  the oracle's SwiGLU epilogue within the bf16 tolerance, and the block codes
  and block amax against the oracle's block quantizer applied to the GPU's own
  h -- the same decision in the same precision, so bit for bit; the kernel
  gives the same codes whether or not it also writes h;
* step 2 alone on the GPU's block codes: codes and scales bit for bit against
  the oracle's rescaling;
* the whole entry point against the composition of the stages (bit for bit),
  and against the oracle's whole chain through the error bound
  |q s - y| <= s + |y_gpu - y_oracle| (y the rotated oracle h; s/2 per rounding
  step plus the difference of the two h), with the row scales within the bf16
  tolerance;
* the gate/up workload (2,270 x 5,120 x 2 x 17,408) at full size with the
  rotation of the down projection (block 128), in the launch configuration
  the benchmark times, on sampled rows recomputed by the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, compare_bf16, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


def _unpack(flat: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Packed layout -> row-major [rows, K] (blocks of 32 rows x 64 bytes, block
    (r // 32, k // 64) at byte ((r // 32) * (K // 64) + k // 64) * 2048)."""
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    return flat[((r // 32) * (K // 64) + k // 64) * 2048 + (r % 32) * 64 + k % 64]


def _setup(lib, orc, wl):
    """Weight codes/scales from the oracle, packed on the GPU; x on the GPU."""
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), wl.rot_block)
    wq_d = torch.from_numpy(wq).to(dev)
    wp = lib.w8a8_pack_weight(wq_d)
    bias_bits = None if inp.bias is None else W.bits(inp.bias)
    bias = None if inp.bias is None else inp.bias.to(dev)
    return inp, wq, s_ch, wp, torch.from_numpy(s_ch).to(dev), bias, bias_bits


# (M, K, N, rot_in, rot_out, bias): ragged M over 256-row tiles, several 128-column
# tiles, a last block of 64 columns (no rotation), a single block per row.
SHAPES = [
    (300, 256, 384, 0, 128, True),
    (530, 512, 256, 128, 0, False),
    (64, 256, 320, 0, 0, True),
    (257, 384, 128, 0, 128, True),
    (1, 128, 1024, 0, 128, False),
    (777, 256, 640, 0, 128, True),
]


def _random_shapes(n, seed):
    """Seeded (M, K, N, rot_in, rot_out, bias) within the entry point's rules: N a multiple
    of 128 with the output rotation, of 64 without; K a multiple of 128."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        rot_out = int(rng.integers(0, 2)) * 128
        N = int(rng.integers(1, 13)) * (128 if rot_out else 64)
        out.append((int(rng.integers(1, 900)), int(rng.integers(1, 7)) * 128, N, int(rng.integers(0, 2)) * 128,
                    rot_out, bool(rng.integers(0, 2))))
    return out


SHAPES += _random_shapes(8, seed=17)


@pytest.mark.parametrize("M,K,N,rot_in,rot_out,has_bias", SHAPES,
                         ids=[f"{m}x{k}x{n}_ri{a}_ro{b}" for m, k, n, a, b, _ in SHAPES])
def test_stages_against_the_oracle(lib, orc, M, K, N, rot_in, rot_out, has_bias):
    say(f"swiglu-quant stages M={M} K={K} N={N} rot_in={rot_in} rot_out={rot_out} bias={has_bias}")
    wl = W.custom("gateup", M, K, N, rot_in, bias=has_bias, seed=M + K + N)
    inp, wq, s_ch, wp, s_ch_d, bias, bias_bits = _setup(lib, orc, wl)
    dev = torch.device("cuda")
    qx, sx = orc.quantize_i8(W.bits(inp.x), rot_in)
    qx_p = lib.w8a8_pack_weight(torch.from_numpy(qx).to(dev))
    sx_d = torch.from_numpy(sx).to(dev)

    codes, amax, h = lib.w8a8_gemm_swiglu_blockquant_packed(qx_p, sx_d, wp, s_ch_d, K, bias=bias,
                                                             rot_out=rot_out, want_h=True)
    codes2, amax2, _ = lib.w8a8_gemm_swiglu_blockquant_packed(qx_p, sx_d, wp, s_ch_d, K, bias=bias,
                                                               rot_out=rot_out, want_h=False)
    torch.cuda.synchronize()
    # (padding rows of the packed buffers are never written: compare the M rows)
    assert np.array_equal(_unpack(codes.cpu().numpy(), M, N), _unpack(codes2.cpu().numpy(), M, N))
    assert torch.equal(amax, amax2)

    h_ref = orc.gemm_swiglu(qx, sx, wq, s_ch, bias_bits)
    h_gpu = bf16_bits(h)
    compare_bf16(h_gpu, h_ref, "SwiGLU output h")
    qb_ref, amax_ref = orc.block_quantize(h_gpu, rot_out)
    qb_gpu = _unpack(codes.cpu().numpy(), M, N)
    assert np.array_equal(qb_gpu, qb_ref), f"block codes: {np.count_nonzero(qb_gpu != qb_ref)} differ"
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), amax_ref.view(np.uint32)), "block amax"

    s = lib.w8a8_requantize_blocks_packed(codes, amax, M, N)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.requantize_blocks(qb_ref, amax_ref)
    q_gpu = _unpack(codes.cpu().numpy(), M, N)
    assert np.array_equal(q_gpu, q_ref), f"rescaled codes: {np.count_nonzero(q_gpu != q_ref)} differ"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "row scales"

    # whole entry point == the stages (GPU quantizer of x, bit-exact with the oracle's)
    x = inp.x.to(dev)
    q_w, s_w = lib.w8a8_gateup_swiglu_quant_packed(x, wp, N, s_ch_d, bias, rot_in=rot_in, rot_out=rot_out)
    torch.cuda.synchronize()
    assert np.array_equal(_unpack(q_w.cpu().numpy(), M, N), q_gpu), "whole path codes vs stages"
    assert torch.equal(s_w, s), "whole path scales vs stages"

    # against the oracle's whole chain: bound on the dequantized values
    q_o, s_o = orc.gateup_swiglu_quant(W.bits(inp.x), wq, s_ch, bias_bits, rot_in, rot_out)
    y_ref = orc.rotate(h_ref, rot_out).astype(np.float64)
    y_gpu = orc.rotate(h_gpu, rot_out).astype(np.float64)
    sg = s.cpu().numpy().astype(np.float64)
    err = np.abs(q_gpu.astype(np.float64) * sg[:, None] - y_ref)
    # (1e-4: the fp32 quotient and product in each rounding step, <= 127 * 2^-23 of a step)
    assert np.all(err <= sg[:, None] * (1 + 1e-4) + np.abs(y_gpu - y_ref)), "dequantized error bound"
    rel_s = np.abs(sg - s_o) / np.maximum(s_o, 1e-30)
    assert rel_s.max() <= 1e-2
    say(f"  vs oracle chain: codes equal {np.mean(q_gpu == q_o):.6f}, max |dq| "
        f"{np.abs(q_gpu.astype(np.int16) - q_o).max()}, scales equal {np.mean(sg == s_o):.4f}")


def test_zero_and_repeated_calls(lib, orc):
    """Zero activations give zero codes and scales; a second call with fewer rows
    into the same buffers touches only its rows."""
    M, K, N = 200, 256, 256
    wl = W.custom("gateup", M, K, N, 0, bias=False, seed=99)
    inp, wq, s_ch, wp, s_ch_d, bias, _ = _setup(lib, orc, wl)
    dev = torch.device("cuda")
    x = inp.x.to(dev).clone()
    x[7] = 0
    q, s = lib.w8a8_gateup_swiglu_quant_packed(x, wp, N, s_ch_d, None, rot_in=0, rot_out=128)
    torch.cuda.synchronize()
    qa = _unpack(q.cpu().numpy(), M, N)
    assert s[7].item() == 0 and not qa[7].any()
    q_o, s_o = orc.gateup_swiglu_quant(W.bits(x.cpu()), wq, s_ch, None, 0, 128)
    assert s_o[7] == 0
    before, s_before = q.clone(), s.clone()
    q2, s2 = lib.w8a8_gateup_swiglu_quant_packed(x[:33].contiguous(), wp, N, s_ch_d, None, rot_in=0,
                                                 rot_out=128, q_out=q, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(q2, before), "rows are independent of the batch they come in"
    assert torch.equal(s2, s_before)


def test_gateup_full_size_with_down_rotation(lib, orc):
    wl = W.WORKLOADS["gateup_2270x5120x2x17408"]
    M, K, N = wl.M, wl.K, wl.N
    say(f"swiglu-quant full size M={M} K={K} N={N} rot_out=128")
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    # the benchmark's configuration: weight quantized on the GPU and packed once
    wq_d, s_ch_d = lib.w8a8_quantize_act(inp.w.to(dev), 0)
    wp = lib.w8a8_pack_weight(wq_d)
    x = inp.x.to(dev)
    ws = torch.empty(lib.swiglu_quant_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    q, s = lib.w8a8_gateup_swiglu_quant_packed(x, wp, N, s_ch_d, None, rot_in=0, rot_out=128, workspace=ws)
    # stages with h, for the sampled-row check
    qx, sx = lib.w8a8_quantize_act_packed(x, 0)
    codes, amax, h = lib.w8a8_gemm_swiglu_blockquant_packed(qx, sx, wp, s_ch_d, K, rot_out=128, want_h=True)
    s_st = lib.w8a8_requantize_blocks_packed(codes, amax, M, N)
    torch.cuda.synchronize()
    q_all = q.cpu().numpy()
    assert np.array_equal(_unpack(q_all, M, N), _unpack(codes.cpu().numpy(), M, N)), "whole path vs stages"
    assert torch.equal(s, s_st)
    wq, s_chv = wq_d.cpu().numpy(), s_ch_d.cpu().numpy()
    del wq_d, wp
    wq_ref, s_ch_ref = orc.quantize_i8(W.bits(inp.w), 0)
    assert np.array_equal(wq, wq_ref) and np.array_equal(s_chv.view(np.uint32), s_ch_ref.view(np.uint32))

    rows = sample_rows(M, n=24, seed=wl.seed, tile=256)
    qx_ref, sx_ref = orc.quantize_i8(W.bits(inp.x)[rows], 0)
    h_ref = orc.gemm_swiglu(qx_ref, sx_ref, wq_ref, s_ch_ref, None)
    h_gpu = bf16_bits(h)[rows]
    compare_bf16(h_gpu, h_ref, f"h ({len(rows)} rows)")
    qb_ref, amax_ref = orc.block_quantize(h_gpu, 128)
    q_ref, s_ref = orc.requantize_blocks(qb_ref, amax_ref)
    assert np.array_equal(amax.cpu().numpy()[rows].view(np.uint32), amax_ref.view(np.uint32)), "block amax"
    q_gpu = _unpack(q_all, M, N)[rows]
    assert np.array_equal(q_gpu, q_ref), f"codes: {np.count_nonzero(q_gpu != q_ref)} differ"
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), s_ref.view(np.uint32)), "scales"
