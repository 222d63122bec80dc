"""GPU parity where byte offsets pass 2^31 and 2^32: inputs, codes and outputs of
several GiB, checked against the CPU oracle on sampled rows on both sides of each
boundary.

* The int8 whole path with the block-128 rotation on 131,137 x 16,384 bf16
  activations (4.3 GB in, 2.15 GB of packed codes in the workspace): the codes,
  the scales and every output column of the sampled rows.
* The quantizer stage entry points (row-major int8, rotated row-major E4M3FN,
  packed E4M3FN) on the same activations.
* GEMMs whose output passes 2^31 bytes, which the launcher runs one tile per
  workgroup, and outputs just under 2^31 bytes, which it runs persistent (its
  stores take 31-bit buffer offsets): dequant, SwiGLU, E4M3FN and exact int32,
  checked on the rows around the 2^31-byte mark and the last rows.

Inputs are drawn on the device (``workloads.device_*``); the oracle reads the
sampled rows of those same input tensors back to the CPU.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, compare_bf16, compare_codes_fp8, compare_codes_i8, say, tile_choice

pytestmark = pytest.mark.gpu

BIG_M, BIG_K = 131_137, 16_384   # M * K > 2^31 elements; the bf16 input > 2^32 bytes


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


@pytest.fixture(scope="module")
def big_x():
    assert BIG_M * BIG_K > 2 ** 31
    x = W.device_normal_bf16(BIG_M, BIG_K, seed=9100, device="cuda")
    yield x
    del x
    torch.cuda.empty_cache()


def _rows_around(M: int, row_bytes, seed: int, n_random: int = 6) -> np.ndarray:
    """First rows, last rows, the rows on each side of the 2^31- and 2^32-byte marks of
    buffers with ``row_bytes`` bytes per row (one figure or several), and a seeded sample."""
    fixed = {0, 1, M - 2, M - 1}
    for rb in np.atleast_1d(row_bytes).tolist():
        for mark in (2 ** 31, 2 ** 32):
            r = mark // rb
            fixed |= {r - 1, r, r + 1}
    fixed = {r for r in fixed if 0 <= r < M}
    rng = np.random.default_rng(seed)
    return np.array(sorted(fixed | set(rng.choice(M, n_random, replace=False).tolist())))


def _host_rows(t: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    return t[torch.as_tensor(rows, device=t.device)].cpu()


def _packed_rows(flat: torch.Tensor, rows: np.ndarray, K: int) -> np.ndarray:
    """Rows of a packed code buffer (blocks of 32 rows x 64 bytes; block (r // 32, k // 64)
    at byte ((r // 32) * (K // 64) + k // 64) * 2048, row r % 32 at byte 64 * (r % 32))."""
    out = []
    for r in rows.tolist():
        base = (r // 32) * 32 * K
        blk = flat[base: base + 32 * K].view(K // 64, 32, 64)
        out.append(blk[:, r % 32, :].reshape(K).cpu())
    return torch.stack(out).numpy()


def test_whole_path_past_4_gib_of_activations(lib, orc, big_x):
    M, K, N = BIG_M, BIG_K, 64
    rows = _rows_around(M, (2 * K, K), seed=9101)
    say(f"int8 whole path, rotation 128: M={M} K={K} N={N}; rows {rows.tolist()}")
    dev = big_x.device
    w = W.device_normal_bf16(N, K, seed=9102, device=dev, outlier_frac=0.0, sigma=0.02)
    bias = W.device_bias_bf16(N, seed=9103, device=dev)
    wq, s_ch = lib.w8a8_quantize_act(w, 128)
    wp = lib.w8a8_pack_weight(wq)
    ws = torch.empty(lib.workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    y = lib.w8a8_linear_packed(big_x, wp, N, s_ch, bias, rot_block=128, workspace=ws)
    torch.cuda.synchronize()

    wq_ref, s_ch_ref = orc.quantize_i8(W.bits(w.cpu()), 128)
    compare_codes_i8(wq.cpu().numpy(), wq_ref, "weight codes")
    assert np.array_equal(s_ch.cpu().numpy().view(np.uint32), s_ch_ref.view(np.uint32)), "weight scales"

    q_ref, s_ref = orc.quantize_i8(W.bits(_host_rows(big_x, rows)), 128)
    codes = _packed_rows(ws, rows, K).view(np.int8)
    compare_codes_i8(codes, q_ref, "activation codes (workspace)")
    off = ((M + 31) // 32 * 32 * K + 255) // 256 * 256
    assert off > 2 ** 31
    s_tok = ws[off: off + 4 * M].view(torch.float32)
    assert np.array_equal(_host_rows(s_tok, rows).numpy().view(np.uint32), s_ref.view(np.uint32)), \
        "activation scales (workspace)"
    y_ref = orc.gemm_dequant(q_ref, s_ref, wq_ref, s_ch_ref, W.bits(bias.cpu()))
    compare_bf16(bf16_bits(_host_rows(y, rows)), y_ref, f"outputs ({len(rows)} rows)")


@pytest.mark.parametrize("fmt,layout,rot", [("i8", "rowmajor", 0), ("fp8", "rowmajor", 128),
                                            ("fp8", "packed", 0)])
def test_quantizer_past_2_gib_of_codes(lib, orc, big_x, fmt, layout, rot):
    M, K = BIG_M, BIG_K
    rows = _rows_around(M, (2 * K, K), seed=9110 + rot + (fmt == "fp8"))
    say(f"quantizer {fmt} {layout} rotation {rot}: M={M} K={K}; rows {rows.tolist()}")
    fn = {("i8", "rowmajor"): lib.w8a8_quantize_act, ("fp8", "rowmajor"): lib.w8a8_quantize_act_fp8,
          ("fp8", "packed"): lib.w8a8_quantize_act_fp8_packed}[(fmt, layout)]
    q, s = fn(big_x, rot)
    torch.cuda.synchronize()
    ref_fn = orc.quantize_fp8 if fmt == "fp8" else orc.quantize_i8
    q_ref, s_ref = ref_fn(W.bits(_host_rows(big_x, rows)), rot)
    got = _packed_rows(q, rows, K) if layout == "packed" else _host_rows(q, rows).numpy()
    if fmt == "fp8":
        compare_codes_fp8(got.view(np.uint8), q_ref, "codes")
    else:
        compare_codes_i8(got.view(np.int8), q_ref, "codes")
    assert np.array_equal(_host_rows(s, rows).numpy().view(np.uint32), s_ref.view(np.uint32)), "scales"
    del q, s
    torch.cuda.empty_cache()


# (epilogue, M, N): outputs past 2^31 bytes (one tile per workgroup) and just under (persistent)
GEMM_CASES = [
    ("dequant", 65_601, 16_384),
    ("dequant", 65_504, 16_384),
    ("swiglu", 65_601, 16_384),
    ("fp8", 65_601, 16_384),
    ("fp8", 65_504, 16_384),
    ("i32", 32_801, 16_384),
    ("i32", 32_752, 16_384),
]


@pytest.mark.parametrize("epi,M,N", GEMM_CASES, ids=[f"{e}-{m}x{n}" for e, m, n in GEMM_CASES])
def test_gemm_output_around_2_gib(lib, orc, epi, M, N):
    K = 256
    elem = 4 if epi == "i32" else 2
    out_bytes = M * N * elem
    say(f"GEMM {epi}: M={M} N={N} K={K}, output {out_bytes} bytes "
        f"({'past' if out_bytes >= 2 ** 31 else 'under'} 2^31)")
    dev = torch.device("cuda")
    nw = 2 * N if epi == "swiglu" else N
    assert tile_choice(M, nw) == "256x256"   # persistent exactly when out_bytes < 2^31
    seed = 9200 + M % 97
    if epi == "fp8":
        q = W.device_e4m3_codes((M, K), seed, dev)
        w = W.device_e4m3_codes((nw, K), seed + 1, dev)
    else:
        q = W.device_codes((M, K), seed, dev)
        w = W.device_codes((nw, K), seed + 1, dev)
    q_pk, w_pk = lib.w8a8_pack_weight(q), lib.w8a8_pack_weight(w)
    s_tok = W.device_scales(M, seed + 2, dev)
    s_ch = W.device_scales(nw, seed + 3, dev)
    bias = W.device_bias_bf16(nw, seed + 4, dev)
    if epi == "i32":
        y = lib.w8a8_gemm_i32_packed(q_pk, w_pk, M, N, K)
    elif epi == "dequant":
        y = lib.w8a8_gemm_dequant_packed(q_pk, s_tok, w_pk, s_ch, K, bias)
    elif epi == "swiglu":
        y = lib.w8a8_gemm_swiglu_packed(q_pk, s_tok, w_pk, s_ch, K, bias)
    else:
        y = lib.w8a8_fp8_gemm_dequant_packed(q_pk, s_tok, w_pk, s_ch, K, bias)
    torch.cuda.synchronize()
    rows = _rows_around(M, N * elem, seed=seed)
    q_rows = _host_rows(q, rows).numpy()
    w_h = w.cpu().numpy()
    got = _host_rows(y, rows)
    if epi == "i32":
        ref = orc.gemm_i32(q_rows, w_h)
        assert np.array_equal(got.numpy(), ref), "int32 accumulators differ"
        return
    st, sc, b = _host_rows(s_tok, rows).numpy(), s_ch.cpu().numpy(), W.bits(bias.cpu())
    if epi == "dequant":
        ref = orc.gemm_dequant(q_rows, st, w_h, sc, b)
    elif epi == "swiglu":
        ref = orc.gemm_swiglu(q_rows, st, w_h, sc, b)
    else:
        ref = orc.fp8_gemm_dequant(q_rows, st, w_h, sc, b)
    compare_bf16(bf16_bits(got), ref, f"{epi} outputs ({len(rows)} rows)")
