"""The single-launch short-input path (quantizer inside the GEMM kernel), which the
whole-path entry points take for short batches (int8, M <= 512, K <= 1024, at most 256
tiles of 32 tokens x 64 weight rows): it must give the same bytes as the two-kernel path -- the packed
quantizer followed by the packed GEMM stage -- for the outputs, the workspace codes
and the scales, and match the oracle on every element.  Shapes cover ragged M and N,
the smallest K (one 32-byte step per wave), K with a partial group of 8 chunks, the
largest K, both weight layouts, rotation on and off, both epilogues, and grids of exactly
256 tiles."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, compare_bf16, compare_codes_i8, say

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


CASES = [
    ("linear", 1, 128, 8, 0, True), ("linear", 31, 384, 72, 128, False), ("linear", 33, 1024, 64, 0, True),
    ("linear", 298, 1024, 1024, 0, True), ("linear", 130, 1024, 200, 128, True), ("linear", 512, 896, 136, 128, False),
    ("gateup", 1, 128, 8, 128, True), ("gateup", 65, 640, 40, 0, True), ("gateup", 300, 1024, 96, 128, False),
    # exactly 256 tiles, the most the single launch takes (16 x 16 and 8 x 32)
    ("linear", 512, 1024, 1024, 0, True), ("gateup", 256, 1024, 1024, 128, True),
]


@pytest.mark.parametrize("kind,M,K,N,rot,packed_w", CASES,
                         ids=[f"{c[0]}_{c[1]}x{c[2]}x{c[3]}_r{c[4]}_{'pw' if c[5] else 'rw'}" for c in CASES])
def test_single_launch_matches_two_kernels_and_oracle(lib, orc, kind, M, K, N, rot, packed_w):
    wl = W.custom(kind, M, K, N, rot, bias=(M % 2 == 0), seed=M + K + N)
    say(f"short path {wl.name} packed_w={packed_w}")
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    x = inp.x.to(dev)
    bias = None if inp.bias is None else inp.bias.to(dev)
    wq, s_ch = lib.w8a8_quantize_act(inp.w.to(dev), rot)
    wp = lib.w8a8_pack_weight(wq)
    ws = torch.full((lib.workspace_bytes(M, K),), 0x5A, dtype=torch.uint8, device=dev)
    if kind == "linear":
        y = (lib.w8a8_linear_packed(x, wp, N, s_ch, bias, rot_block=rot, workspace=ws) if packed_w
             else lib.w8a8_linear(x, wq, s_ch, bias, rot_block=rot, workspace=ws))
    else:
        y = (lib.w8a8_gateup_swiglu_packed(x, wp, N, s_ch, bias, rot_block=rot, workspace=ws) if packed_w
             else lib.w8a8_gateup_swiglu(x, wq, s_ch, bias, rot_block=rot, workspace=ws))
    # the two-kernel path, stage by stage
    qp, s_tok = lib.w8a8_quantize_act_packed(x, rot)
    gemm = lib.w8a8_gemm_dequant_packed if kind == "linear" else lib.w8a8_gemm_swiglu_packed
    y2 = gemm(qp, s_tok, wp, s_ch, K, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "single launch and two kernels differ"
    flat = ws.cpu().numpy()
    off = (lib.packed_bytes(M, K) + 255) // 256 * 256
    assert np.array_equal(_unpack(flat, M, K).view(np.int8), _unpack(qp.cpu().numpy(), M, K)), "workspace codes"
    assert np.array_equal(flat[off:off + 4 * M].view(np.uint32), s_tok.cpu().numpy().view(np.uint32)), "scales"
    # and the oracle
    x_bits = W.bits(inp.x)
    q_ref, s_ref = orc.quantize_i8(x_bits, rot)
    compare_codes_i8(_unpack(flat, M, K).view(np.int8), q_ref, "codes")
    wq_ref, s_ch_ref = orc.quantize_i8(W.bits(inp.w), rot)
    bias_bits = None if inp.bias is None else W.bits(inp.bias)
    ref = (orc.gemm_dequant if kind == "linear" else orc.gemm_swiglu)(q_ref, s_ref, wq_ref, s_ch_ref, bias_bits)
    compare_bf16(bf16_bits(y), ref, "outputs")
