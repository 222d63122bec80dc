"""GPU parity of the gate/up SwiGLU whose output is quantized for the next linear.

The down projection's input is the per-token int8 quantization (optionally after
the block-128 rotation) of the bf16 SwiGLU output h ("CLEF Calibrated INT8 ConvRot"
card, notes under the latency table; "Loading CLEF INT8", fuse_mlp): the oracle is
``orc.gateup_swiglu_quant`` = ``orc.quantize_i8(orc.gateup_swiglu(x), rot_out)``.
``w8a8_gateup_swiglu_quant_packed`` runs the quantizer of x, the gate/up GEMM with
the SwiGLU epilogue (h into its workspace) and the quantizer of h.  Checked here:

* h (read back from the workspace) against the oracle's SwiGLU epilogue within the
  bf16 tolerance;
* on the rows where the kernel's h equals the oracle's bit for bit -- the quantizer's
  input is then the same, so the integer decision is taken on the same values in the
  same precision -- codes and scales against the oracle's composition bit for bit;
* the codes against the oracle's whole composition with the flip budget
  (``compare_codes_i8``: at most one step, in at most 1e-4 of the elements) on the
  rows whose scale equals the oracle's.  A row's scale can differ only where the
  fp32 epilogue rounded an element of h the other way from the fp64 oracle (within
  the bf16 tolerance) inside the block that sets the row's rotated amax; such rows
  are counted and each is tied to such an element of h;
* small hand-picked and seeded random shapes, a zero row, repeated calls into the
  same buffers, and the gate/up workload (2,270 x 5,120 x 2 x 17,408) at full size
  with the down projection's rotation, in the launch configuration the benchmark
  times, on sampled rows recomputed by the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, compare_bf16, compare_codes_i8, sample_rows, say

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


def _check_against_oracle(orc, q_gpu, s_gpu, h_gpu, h_ref, x_bits, wq, s_ch, bias_bits, rot_in, rot_out,
                          what):
    """q_gpu int8 [m, N], s_gpu fp32 [m], h_gpu / h_ref bf16 bits [m, N] for the same rows."""
    compare_bf16(h_gpu, h_ref, f"{what}: SwiGLU output h")
    # the oracle's whole composition
    q_o, s_o = orc.gateup_swiglu_quant(x_bits, wq, s_ch, bias_bits, rot_in, rot_out)
    assert np.array_equal(orc.quantize_i8(h_ref, rot_out)[0], q_o)
    # rows whose h is the oracle's bit for bit: the same quantizer input, so bit-exact codes and scales
    eq = np.all(h_gpu == h_ref, axis=1)
    assert np.array_equal(s_gpu[eq].view(np.uint32), s_o[eq].view(np.uint32)), f"{what}: scales (rows with equal h)"
    assert np.array_equal(q_gpu[eq], q_o[eq]), \
        f"{what}: {np.count_nonzero(q_gpu[eq] != q_o[eq])} codes differ on rows with equal h"
    same = s_gpu.view(np.uint32) == s_o.view(np.uint32)
    if same.any():
        compare_codes_i8(q_gpu[same], q_o[same], f"{what}: codes vs the oracle chain ({int(same.sum())} rows)")
    for m in np.nonzero(~same)[0]:
        # the row's scale moved: an element of h in the row rounded the other way (one bf16 step)
        d = np.nonzero(h_gpu[m] != h_ref[m])[0]
        assert d.size > 0, f"{what}: row {m} scale differs with an identical h"
        step = np.abs(h_gpu[m, d].astype(np.int32) - h_ref[m, d].astype(np.int32))
        assert np.all(step == 1), f"{what}: row {m}: h differs by more than one bf16 step"
        assert abs(float(s_gpu[m]) - float(s_o[m])) <= 2.0 ** -7 * float(s_o[m]), f"{what}: row {m} scale"
    say(f"  {what}: {int(eq.sum())} of {len(eq)} rows with h equal to the oracle's (bit-exact codes); "
        f"{int((~same).sum())} with a scale moved by h's rounding; codes equal {np.mean(q_gpu == q_o):.6f}")


def _setup(lib, orc, wl):
    """Weight codes/scales from the oracle, packed on the GPU."""
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), wl.rot_block)
    wp = lib.w8a8_pack_weight(torch.from_numpy(wq).to(dev))
    bias_bits = None if inp.bias is None else W.bits(inp.bias)
    bias = None if inp.bias is None else inp.bias.to(dev)
    return inp, wq, s_ch, wp, torch.from_numpy(s_ch).to(dev), bias, bias_bits


# (M, K, N, rot_in, rot_out, bias): ragged M over the GEMM tiles and the packed
# 32-row blocks, several output blocks, a 64-column multiple without rotation, a
# single block per row.
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
def test_against_the_oracle(lib, orc, M, K, N, rot_in, rot_out, has_bias):
    say(f"swiglu-quant M={M} K={K} N={N} rot_in={rot_in} rot_out={rot_out} bias={has_bias}")
    wl = W.custom("gateup", M, K, N, rot_in, bias=has_bias, seed=M + K + N)
    inp, wq, s_ch, wp, s_ch_d, bias, bias_bits = _setup(lib, orc, wl)
    dev = torch.device("cuda")
    ws = torch.empty(lib.swiglu_quant_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    q, s = lib.w8a8_gateup_swiglu_quant_packed(inp.x.to(dev), wp, N, s_ch_d, bias, rot_in=rot_in,
                                               rot_out=rot_out, workspace=ws)
    torch.cuda.synchronize()
    q_gpu = _unpack(q.cpu().numpy(), M, N)
    h_gpu = bf16_bits(lib.swiglu_quant_h(ws, M, N, K))
    x_bits = W.bits(inp.x)
    h_ref = orc.gateup_swiglu(x_bits, wq, s_ch, bias_bits, rot_in)
    _check_against_oracle(orc, q_gpu, s.cpu().numpy(), h_gpu, h_ref, x_bits, wq, s_ch, bias_bits, rot_in, rot_out,
                          f"{M}x{K}x{N}")
    # the workspace's h is the fused gate/up path's output, byte for byte
    y = lib.w8a8_gateup_swiglu_packed(inp.x.to(dev), wp, N, s_ch_d, bias, rot_block=rot_in)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), h_gpu)


def test_zero_and_repeated_calls(lib, orc):
    """A zero activation row gives zero codes and a zero scale; a second call with fewer
    rows into the same buffers rewrites exactly its rows with the same bytes."""
    M, K, N = 200, 256, 256
    wl = W.custom("gateup", M, K, N, 0, bias=False, seed=99)
    inp, wq, s_ch, wp, s_ch_d, bias, _ = _setup(lib, orc, wl)
    dev = torch.device("cuda")
    x_h = inp.x.clone()
    x_h[7] = 0
    x = x_h.to(dev)
    q, s = lib.w8a8_gateup_swiglu_quant_packed(x, wp, N, s_ch_d, None, rot_in=0, rot_out=128)
    torch.cuda.synchronize()
    qa = _unpack(q.cpu().numpy(), M, N)
    assert s[7].item() == 0 and not qa[7].any()
    q_o, s_o = orc.gateup_swiglu_quant(W.bits(x_h), wq, s_ch, None, 0, 128)
    assert s_o[7] == 0
    before, s_before = q.clone(), s.clone()
    q2, s2 = lib.w8a8_gateup_swiglu_quant_packed(x[:33].contiguous(), wp, N, s_ch_d, None, rot_in=0,
                                                 rot_out=128, q_out=q, s_out=s[:33])
    torch.cuda.synchronize()
    assert torch.equal(q2, before), "rows are independent of the batch they come in"
    assert torch.equal(s, s_before)


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
    torch.cuda.synchronize()
    rows = sample_rows(M, n=24, seed=wl.seed, tile=256)
    q_gpu = _unpack(q.cpu().numpy(), M, N)[rows]
    s_gpu = s.cpu().numpy()[rows]
    h_gpu = bf16_bits(lib.swiglu_quant_h(ws, M, N, K))[rows]
    wq, s_chv = wq_d.cpu().numpy(), s_ch_d.cpu().numpy()
    del wq_d, wp, ws
    wq_ref, s_ch_ref = orc.quantize_i8(W.bits(inp.w), 0)
    assert np.array_equal(wq, wq_ref) and np.array_equal(s_chv.view(np.uint32), s_ch_ref.view(np.uint32))
    x_rows = np.ascontiguousarray(W.bits(inp.x)[rows])
    h_ref = orc.gateup_swiglu(x_rows, wq_ref, s_ch_ref, None, 0)
    _check_against_oracle(orc, q_gpu, s_gpu, h_gpu, h_ref, x_rows, wq_ref, s_ch_ref, None, 0, 128,
                          f"full size, {len(rows)} rows")


def test_codes_feed_the_down_projection(lib, orc):
    """The packed codes and scales are the down projection's A operand as they stand:
    w8a8_gemm_dequant_packed on them (K = N) against the oracle's chain (SwiGLU output
    quantized per token, then the down projection's GEMM and dequant), on the rows whose
    SwiGLU output equals the oracle's (the same codes, so the outputs within the bf16
    tolerance)."""
    M, K, N, N2 = 300, 256, 384, 264
    wl = W.custom("gateup", M, K, N, 0, bias=True, seed=123)
    inp, wq, s_ch, wp, s_ch_d, bias, bias_bits = _setup(lib, orc, wl)
    dev = torch.device("cuda")
    down = W.custom("linear", M, N, N2, 128, bias=True, seed=124)
    dinp = W.make_inputs(down)
    w2q, s2_ch = orc.quantize_i8(W.bits(dinp.w), 128)
    ws = torch.empty(lib.swiglu_quant_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    q, s = lib.w8a8_gateup_swiglu_quant_packed(inp.x.to(dev), wp, N, s_ch_d, bias, rot_in=0, rot_out=128,
                                               workspace=ws)
    y2 = lib.w8a8_gemm_dequant_packed(q, s, lib.w8a8_pack_weight(torch.from_numpy(w2q).to(dev)),
                                      torch.from_numpy(s2_ch).to(dev), N, bias=dinp.bias.to(dev))
    torch.cuda.synchronize()
    x_bits = W.bits(inp.x)
    h_ref = orc.gateup_swiglu(x_bits, wq, s_ch, bias_bits, 0)
    q_o, s_o = orc.gateup_swiglu_quant(x_bits, wq, s_ch, bias_bits, 0, 128)
    y2_ref = orc.gemm_dequant(q_o, s_o, w2q, s2_ch, W.bits(dinp.bias))
    eq = np.all(bf16_bits(lib.swiglu_quant_h(ws, M, N, K)) == h_ref, axis=1)
    say(f"  down projection on the SwiGLU output's codes: {int(eq.sum())} of {M} rows with equal h")
    assert eq.sum() >= M // 2
    compare_bf16(bf16_bits(y2)[eq], y2_ref[eq], "down projection outputs")
