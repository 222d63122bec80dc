"""GPU parity of the unfused gate/up path ("Loading CLEF INT8" page, fuse_mlp=False)
against the CPU oracle: the SwiGLU stage alone, and the chain quantize -> linear onto
the 2N packed rows (bf16 [M, 2N]) -> w8a8_swiglu of its halves, on every element of
small shapes and on sampled rows of the full gate/up workload."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, bits_to_f64, compare_bf16, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


@pytest.mark.parametrize("M,N,ld", [(1, 8, 8), (37, 96, 192), (300, 1024, 1024), (129, 4088, 8192)])
def test_swiglu_stage(lib, orc, M, N, ld):
    """ld == N: gate and up are separate dense tensors; ld >= 2N: they are the first two
    N-column blocks of one [M, ld] buffer (rows ld elements apart)."""
    say(f"swiglu M={M} N={N} ld={ld}")
    g = torch.Generator().manual_seed(M * 31 + N)
    if ld == N:
        gate = (torch.randn(M, N, generator=g, dtype=torch.float64) * 3).to(torch.bfloat16)
        up = (torch.randn(M, N, generator=g, dtype=torch.float64) * 3).to(torch.bfloat16)
        gate[0, :4] = torch.tensor([0.0, -0.0, 90.0, -90.0], dtype=torch.bfloat16)
        gd, ud = gate.cuda(), up.cuda()
    else:
        h = (torch.randn(M, ld, generator=g, dtype=torch.float64) * 3).to(torch.bfloat16)
        h[0, :4] = torch.tensor([0.0, -0.0, 90.0, -90.0], dtype=torch.bfloat16)
        gate, up = h[:, :N].contiguous(), h[:, N:2 * N].contiguous()
        hd = h.cuda()
        gd, ud = hd[:, :N], hd[:, N:2 * N]
    y = lib.w8a8_swiglu(gd, ud)
    torch.cuda.synchronize()
    ref = orc.swiglu_bf16(W.bits(gate), W.bits(up))
    compare_bf16(bf16_bits(y), ref, "swiglu")


def _check(lib, orc, wl, rows=None):
    """Stage by stage, each at the single-rounding tolerance: the projection onto the 2N
    packed rows against the oracle's, then the GPU's SwiGLU pass run on the oracle's
    projection against the oracle's SwiGLU of it.  End to end against the oracle's chain
    the bound is wider:
    where the two projections differ by an ulp (an fp32-vs-fp64 near-tie), the SwiGLU
    scales that relative change by |d ln silu(g) / d ln g| = |1 + g (1 - sigmoid(g))|,
    which grows like |g| for very negative gates, so the chain is held to the first-order
    propagation of the actual projection differences plus the two final roundings."""
    say(f"unfused gate/up {wl.name}: M={wl.M} K={wl.K} N={wl.N} rot={wl.rot_block}")
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    wq, s_ch = lib.w8a8_quantize_act(inp.w.to(dev), wl.rot_block)
    wp = lib.w8a8_pack_weight(wq)
    bias = None if inp.bias is None else inp.bias.to(dev)
    N = wl.N
    h = lib.w8a8_linear_packed(inp.x.to(dev), wp, 2 * N, s_ch, bias, rot_block=wl.rot_block)
    y = lib.w8a8_swiglu(h[:, :N], h[:, N:])
    torch.cuda.synchronize()
    rows = np.arange(wl.M) if rows is None else rows
    wq_ref, s_ch_ref = orc.quantize_i8(W.bits(inp.w), wl.rot_block)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    bias_bits = None if inp.bias is None else W.bits(inp.bias)
    x_rows = W.bits(inp.x)[rows]
    h_ref = orc.linear(x_rows, wq_ref, s_ch_ref, bias_bits, wl.rot_block)
    h_got = bf16_bits(h)[rows]
    compare_bf16(h_got, h_ref, f"{wl.name} projection onto 2N rows ({len(rows)} rows)")
    y_got = bf16_bits(y)[rows]
    # the SwiGLU stage on the oracle's projection (uploaded; same row stride as the GPU's)
    h_ref_d = torch.from_numpy(h_ref.view(np.int16)).view(torch.bfloat16).to(dev)
    y_stage = lib.w8a8_swiglu(h_ref_d[:, :N], h_ref_d[:, N:])
    torch.cuda.synchronize()
    compare_bf16(bf16_bits(y_stage), orc.swiglu_bf16(h_ref[:, :N], h_ref[:, N:]), f"{wl.name} swiglu stage")
    y_ref = orc.gateup_unfused(x_rows, wq_ref, s_ch_ref, bias_bits, wl.rot_block)
    # end to end: first-order propagation of the projection differences through
    # silu(g) * u, plus the final rounding of each side (at most 2 ulp apart)
    g_got, u_got = bits_to_f64(h_got[:, :N]), bits_to_f64(h_got[:, N:])
    g_ref, u_ref = bits_to_f64(h_ref[:, :N]), bits_to_f64(h_ref[:, N:])
    sig = 1.0 / (1.0 + np.exp(-g_ref))
    dsilu = sig * (1.0 + g_ref * (1.0 - sig))
    dg, du = np.abs(g_got - g_ref), np.abs(u_got - u_ref)
    got, ref = bits_to_f64(y_got), bits_to_f64(y_ref)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    bound = 1.1 * (np.abs(dsilu) * dg * (np.abs(u_ref) + du) + np.abs(g_ref * sig) * du) + 2 * ulp
    err = np.abs(got - ref)
    say(f"  chain end to end: {int(((dg > 0) | (du > 0)).sum())} outputs with a differing projection, "
        f"max err / bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)


SMALL = [W.custom("gateup", 130, 512, 136, 0, bias=False, seed=71),
         W.custom("gateup", 257, 384, 72, 128, bias=True, seed=72),
         W.custom("gateup", 1099, 256, 2040, 0, bias=True, seed=73)]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_unfused_small_every_element(lib, orc, wl):
    _check(lib, orc, wl)


def test_unfused_gateup_workload(lib, orc):
    wl = W.WORKLOADS["gateup_2270x5120x2x17408"]
    _check(lib, orc, wl, sample_rows(wl.M, n=24, seed=wl.seed))
