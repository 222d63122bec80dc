"""GPU parity of the whole paths (quantize + GEMM + epilogue) against the CPU oracle.

* Each of the five workloads at its full size, in the launch configuration the
  benchmark times (weight quantized on the GPU, packed once, whole path on the
  packed weight): the weight codes and scales are compared with the oracle's
  over the whole matrix, and a seeded sample of token rows (first/last rows,
  rows on tile boundaries) is recomputed by the oracle one by one: activation
  codes and scales (read back from the workspace, whose codes are in the
  packed layout) and every output column of those rows.  The row-major-weight
  entry point must give the same bytes.
* Smaller shapes compared on every element, through both weight layouts; they
  are chosen so that every tile configuration (128 x 128, 192 x 128 and
  256 x 256) runs with each epilogue, with ragged M and N edges.
* Properties that hold at any size: rows are byte-identical however the batch
  is split (row results must not depend on batching), repeated runs are
  byte-identical, and a non-default stream gives the same bytes.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import (bf16_bits, compare_bf16, compare_codes_fp8, compare_codes_i8, sample_rows, say,
                    tile_choice)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


def _gpu_path(lib, wl, x, wq, s_ch, bias, workspace=None, out=None):
    fn = {"linear": lib.w8a8_linear, "gateup": lib.w8a8_gateup_swiglu, "fp8": lib.w8a8_fp8_linear}[wl.kind]
    return fn(x, wq, s_ch, bias, rot_block=wl.rot_block, workspace=workspace, out=out)


def _gpu_path_packed(lib, wl, x, wp, s_ch, bias, workspace=None, out=None):
    fn = {"linear": lib.w8a8_linear_packed, "gateup": lib.w8a8_gateup_swiglu_packed,
          "fp8": lib.w8a8_fp8_linear_packed}[wl.kind]
    return fn(x, wp, wl.N, s_ch, bias, rot_block=wl.rot_block, workspace=workspace, out=out)


def _unpack(flat: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Packed layout -> row-major [rows, K]: blocks of 32 rows x 64 bytes, block
    (r // 32, k // 64) at byte ((r // 32) * (K // 64) + k // 64) * 2048, row r % 32
    of the block at byte 64 * (r % 32) within it."""
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    idx = ((r // 32) * (K // 64) + k // 64) * 2048 + (r % 32) * 64 + k % 64
    return flat[idx]


def _oracle_quant(orc, wl, a_bits):
    return orc.quantize_fp8(a_bits, wl.rot_block) if wl.kind == "fp8" else orc.quantize_i8(a_bits, wl.rot_block)


def _oracle_epilogue(orc, wl, q, s_tok, wq, s_ch, bias_bits):
    if wl.kind == "fp8":
        return orc.fp8_gemm_dequant(q, s_tok, wq, s_ch, bias_bits)
    if wl.kind == "gateup":
        return orc.gemm_swiglu(q, s_tok, wq, s_ch, bias_bits)
    return orc.gemm_dequant(q, s_tok, wq, s_ch, bias_bits)


def _check_workload(lib, orc, wl, rows=None):
    say(f"workload {wl.name}: M={wl.M} K={wl.K} N={wl.N} kind={wl.kind} rot={wl.rot_block}")
    inp = W.make_inputs(wl)
    fp8 = wl.kind == "fp8"
    quant = lib.w8a8_quantize_act_fp8 if fp8 else lib.w8a8_quantize_act
    compare_codes = compare_codes_fp8 if fp8 else compare_codes_i8
    dev = torch.device("cuda")
    x = inp.x.to(dev)
    bias = None if inp.bias is None else inp.bias.to(dev)
    wq, s_ch = quant(inp.w.to(dev), wl.rot_block)
    wp = lib.w8a8_pack_weight(wq)
    ws = torch.empty(lib.workspace_bytes(wl.M, wl.K), dtype=torch.uint8, device=dev)
    y = _gpu_path_packed(lib, wl, x, wp, s_ch, bias, workspace=ws)
    torch.cuda.synchronize()
    codes_flat = ws.cpu().numpy()
    y_rowmajor_w = _gpu_path(lib, wl, x, wq, s_ch, bias)
    assert torch.equal(y_rowmajor_w, y), "row-major and packed weights give different outputs"
    del y_rowmajor_w

    wq_ref, s_ch_ref = _oracle_quant(orc, wl, W.bits(inp.w))
    compare_codes(wq.cpu().numpy(), wq_ref, "weight codes")
    assert np.array_equal(s_ch.cpu().numpy().view(np.uint32), s_ch_ref.view(np.uint32)), "weight scales"

    rows = np.arange(wl.M) if rows is None else rows
    x_rows = W.bits(inp.x)[rows]
    q_ref, s_ref = _oracle_quant(orc, wl, x_rows)
    # workspace: packed codes (rows rounded up to 32), then the scales at the next 256-byte boundary
    off = ((wl.M + 31) // 32 * 32 * wl.K + 255) // 256 * 256
    assert lib.workspace_bytes(wl.M, wl.K) == off + (4 * wl.M + 255) // 256 * 256
    codes = _unpack(codes_flat, wl.M, wl.K)
    s_tok = codes_flat[off: off + 4 * wl.M].view(np.float32)
    compare_codes(codes[rows].view(np.uint8 if fp8 else np.int8), q_ref, "activation codes")
    assert np.array_equal(s_tok[rows].view(np.uint32), s_ref.view(np.uint32)), "activation scales"

    bias_bits = None if inp.bias is None else W.bits(inp.bias)
    y_ref = _oracle_epilogue(orc, wl, q_ref, s_ref, wq_ref, s_ch_ref, bias_bits)
    compare_bf16(bf16_bits(y)[rows], y_ref, f"{wl.name} outputs ({len(rows)} rows)")


@pytest.mark.parametrize("name", W.ORDER)
def test_workload_full_size(lib, orc, name):
    wl = W.WORKLOADS[name]
    # every element where the oracle's pass is cheap (the short and the default 1,502-token
    # workloads, ~25 G multiply-adds); sampled rows for the three largest
    rows = None if wl.M * wl.n_w * wl.K <= 2 ** 35 else sample_rows(wl.M, n=40 if wl.kind != "fp8" else 24,
                                                                   seed=wl.seed)
    _check_workload(lib, orc, wl, rows)


SMALL = [
    W.custom("linear", 1, 128, 8, 0, seed=1),
    W.custom("linear", 129, 256, 136, 128, seed=2),
    W.custom("linear", 300, 1024, 264, 128, outlier_frac=0.005, outlier_factor=50.0, seed=3),
    W.custom("linear", 64, 768, 40, 0, bias=False, x_kind="silu_product", sigma_w=0.01, seed=4),
    W.custom("gateup", 130, 512, 136, 0, bias=False, seed=5),
    W.custom("gateup", 257, 384, 72, 128, bias=True, seed=6),
    W.custom("fp8", 200, 512, 128, 0, bias=False, seed=7),
    W.custom("fp8", 131, 1024, 264, 128, bias=True, seed=8),
    # 192 x 128 tiles (ragged M and N)
    W.custom("linear", 1099, 256, 8184, 0, seed=21),
    W.custom("gateup", 1099, 384, 4088, 128, seed=22),
    W.custom("fp8", 1099, 256, 8184, 0, bias=True, seed=23),
    # 256 x 256 tiles (ragged M and N; the gate/up up-row panel starts off a 32-row boundary)
    W.custom("linear", 2047, 256, 8184, 128, seed=24),
    W.custom("gateup", 2047, 256, 4088, 0, bias=True, seed=25),
    W.custom("fp8", 2047, 384, 8184, 128, bias=False, seed=26),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_every_element(lib, orc, wl):
    _check_workload(lib, orc, wl)


@pytest.mark.parametrize("kind,rot", [("linear", 128), ("gateup", 0), ("fp8", 0)])
def test_batch_split_invariance_and_determinism(lib, kind, rot):
    wl = W.custom(kind, 600, 1024, 264, rot, seed=11)
    say(f"batch invariance {wl.name}")
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    quant = lib.w8a8_quantize_act_fp8 if kind == "fp8" else lib.w8a8_quantize_act
    wq, s_ch = quant(inp.w.to(dev), rot)
    x = inp.x.to(dev)
    bias = None if inp.bias is None else inp.bias.to(dev)
    whole = _gpu_path(lib, wl, x, wq, s_ch, bias)
    again = _gpu_path(lib, wl, x, wq, s_ch, bias)
    pieces, r = [], 0
    for n in (1, 7, 64, 129, 255, 144):
        pieces.append(_gpu_path(lib, wl, x[r:r + n].contiguous(), wq, s_ch, bias))
        r += n
    assert r == wl.M
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        other = _gpu_path(lib, wl, x, wq, s_ch, bias)
    torch.cuda.synchronize()
    b = bf16_bits(whole)
    assert np.array_equal(b, bf16_bits(again)), "repeat run differs"
    assert np.array_equal(b, bf16_bits(torch.cat(pieces))), "batch split changes row results"
    assert np.array_equal(b, bf16_bits(other)), "non-default stream differs"


@pytest.mark.parametrize("kind", ["linear", "fp8"])
def test_batch_split_across_tile_configurations(lib, kind):
    """2100 tokens run with 192 x 128 tiles, a 2048-token piece with 256 x 256
    tiles and a 52-token piece with 128 x 128 tiles: the rows must agree byte
    for byte (the k order of every output element is the same in all three)."""
    wl = W.custom(kind, 2100, 256, 8192, 0, seed=12)
    say(f"batch split across tile configurations {wl.name}")
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    quant = lib.w8a8_quantize_act_fp8 if kind == "fp8" else lib.w8a8_quantize_act
    wq, s_ch = quant(inp.w.to(dev), 0)
    wp = lib.w8a8_pack_weight(wq)
    x = inp.x.to(dev)
    bias = inp.bias.to(dev)
    whole = _gpu_path_packed(lib, wl, x, wp, s_ch, bias)
    a = _gpu_path_packed(lib, wl, x[:2048].contiguous(), wp, s_ch, bias)
    b = _gpu_path_packed(lib, wl, x[2048:].contiguous(), wp, s_ch, bias)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(whole), bf16_bits(torch.cat([a, b]))), "tile configuration changes rows"


@pytest.mark.parametrize("rows,K", [(1, 64), (31, 128), (32, 192), (100, 4096), (4097, 256)])
def test_pack_weight_layout(lib, rows, K):
    """w8a8_pack_weight writes the documented layout byte for byte, with zero padding rows."""
    say(f"pack rows={rows} K={K}")
    g = torch.Generator().manual_seed(rows * 7919 + K)
    w = torch.randint(-128, 128, (rows, K), generator=g, dtype=torch.int8)
    wp = lib.w8a8_pack_weight(w.to("cuda"))
    torch.cuda.synchronize()
    flat = wp.cpu().numpy()
    prow = (rows + 31) // 32 * 32
    assert flat.size == prow * K == lib.packed_bytes(rows, K)
    wn = w.numpy()
    assert np.array_equal(_unpack(flat, rows, K), wn)
    assert np.array_equal(lib.unpack_rows(wp, rows, K).cpu().numpy(), wn)
    if prow > rows:
        pad = _unpack(flat, prow, K)[rows:]
        assert not pad.any(), "padding rows must be zero"


def _random_shapes(n, seed, m_range=(1, 701), k_blocks=(1, 13), n_groups=(1, 126)):
    """Seeded shapes within the API's rules: M in m_range, N a multiple of 8, K a multiple of
    128 (defaults: M up to 700, N up to 1,000, K up to 1,536 -- mostly short-path sizes);
    kind, rotation and bias drawn too."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("linear", "gateup", "fp8")[i % 3]
        M = int(rng.integers(*m_range))
        N = int(rng.integers(*n_groups)) * 8
        K = int(rng.integers(*k_blocks)) * 128
        rot = int(rng.integers(0, 2)) * 128
        out.append(W.custom(kind, M, K, N, rot, bias=bool(rng.integers(0, 2)), seed=seed + i))
    return out


# 48 shapes around the short path's range, 12 with M up to 2,600 (two-kernel path, ragged
# tiles of every shape)
RANDOM = (_random_shapes(48, seed=2026) +
          _random_shapes(12, seed=4052, m_range=(700, 2601), k_blocks=(1, 9), n_groups=(1, 200)))


@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
def test_random_shapes_every_element(lib, orc, wl):
    """Seeded random shapes (ragged M, N and K, every path kind, with and without rotation),
    every element against the oracle through both weight layouts."""
    _check_workload(lib, orc, wl)


def _random_persistent_shapes(n, seed):
    """Seeded shapes on which the launcher picks the 256 x 256 tile (run by the persistent
    GEMM: several tiles per workgroup, ragged in M and N), K = 256 .. 512."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = ("linear", "gateup", "fp8")[len(out) % 3]
        M, N, K = int(rng.integers(2600, 4200)), int(rng.integers(500, 1100)) * 8, int(rng.integers(2, 5)) * 128
        rot, bias = int(rng.integers(0, 2)) * 128, bool(rng.integers(0, 2))
        if tile_choice(M, 2 * N if kind == "gateup" else N) == "256x256":
            out.append(W.custom(kind, M, K, N, rot, bias=bias, seed=seed + len(out)))
    return out


RANDOM_PERSISTENT = _random_persistent_shapes(6, seed=6078)


@pytest.mark.parametrize("wl", RANDOM_PERSISTENT, ids=[w.name for w in RANDOM_PERSISTENT])
def test_random_persistent_shapes_every_element(lib, orc, wl):
    """Seeded random shapes that run the persistent 256 x 256 GEMM (2-5 tiles per
    workgroup, ragged M and N, every path kind), every element against the oracle."""
    assert tile_choice(wl.M, wl.n_w) == "256x256"
    _check_workload(lib, orc, wl)


def test_concurrent_streams(lib):
    """Two unrelated whole-path calls running at the same time on two streams, each with
    its own workspace, give the bytes of the same calls run one after the other (the
    library keeps no mutable state between calls)."""
    dev = torch.device("cuda")
    cases = []
    for kind, M, K, N, rot, seed in (("linear", 1502, 1024, 1024, 128, 31), ("gateup", 700, 512, 640, 0, 32)):
        wl = W.custom(kind, M, K, N, rot, seed=seed)
        inp = W.make_inputs(wl)
        wq, s_ch = lib.w8a8_quantize_act(inp.w.to(dev), rot)
        cases.append((wl, inp.x.to(dev), lib.w8a8_pack_weight(wq), s_ch, inp.bias.to(dev)))
    torch.cuda.synchronize()
    seq = [_gpu_path_packed(lib, wl, x, wp, s_ch, b) for wl, x, wp, s_ch, b in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for _ in range(3):
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        res = [None, None]
        for i, ((wl, x, wp, s_ch, b), st) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(st):
                res[i] = _gpu_path_packed(lib, wl, x, wp, s_ch, b)
        torch.cuda.synchronize()
        outs.append(res)
    for res in outs:
        for got, ref in zip(res, seq):
            assert torch.equal(got, ref), "concurrent calls differ from sequential ones"
