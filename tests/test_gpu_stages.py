"""GPU parity of each stage against the CPU oracle, through the C ABI.

Stage 1 (quantizer): codes and scales bit-exact (flip budget 1e-4 of one step).
Stage 2 (integer GEMM, fed identical int8 codes): int32 bit-exact.
Stage 3 (epilogues, fed identical codes and scales): bf16 within the
tolerances in tests/parity.py.  Shapes span several 128-wide tiles with ragged
tails in M and N, the smallest legal shapes, and the largest K.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import (bf16_bits, compare_bf16, compare_codes_fp8, compare_codes_i8, sample_rows, say,
                    tile_choice as _tile_choice)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib  # raises if the HIP library is not built
    return lib


def _x_case(M, K, rot, seed, zero_rows=()):
    wl = W.custom("linear", M, K, 8, rot, outlier_frac=0.01, outlier_factor=30.0, seed=seed)
    x = W.make_inputs(wl).x.clone()
    for r in zero_rows:
        if r < M:
            x[r] = 0
    return x


QUANT_CASES = [
    (298, 1024, 0), (1, 32, 0), (7, 96, 0), (5, 5120, 0), (3, 17408, 0), (2, 131072, 0),
    (600, 4096, 0), (1502, 4096, 128), (129, 5120, 128),
    (300, 1024, 128), (64, 4096, 128), (9, 17408, 128), (2, 131072, 128), (5, 5120, 128),
]


@pytest.mark.parametrize("M,K,rot", QUANT_CASES)
def test_quantize_int8(lib, orc, M, K, rot):
    say(f"quantize int8 M={M} K={K} rot={rot}")
    x = _x_case(M, K, rot, seed=100 + M + K, zero_rows=(1,))
    q, s = lib.w8a8_quantize_act(x.cuda(), rot)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quantize_i8(W.bits(x), rot)
    compare_codes_i8(q.cpu().numpy(), q_ref, "codes")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("M,K,rot", [(298, 1024, 0), (3, 96, 0), (4, 17408, 0), (33, 4096, 128),
                                     (3, 17408, 128), (2, 131072, 0)])
def test_quantize_fp8(lib, orc, M, K, rot):
    say(f"quantize fp8 M={M} K={K} rot={rot}")
    x = _x_case(M, K, rot, seed=200 + M + K, zero_rows=(1,))
    q, s = lib.w8a8_quantize_act_fp8(x.cuda(), rot)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quantize_fp8(W.bits(x), rot)
    compare_codes_fp8(q.cpu().numpy(), q_ref, "fp8 codes")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"


def test_fp8_converter_on_every_bf16_value(lib, orc):
    """Row amax 448 gives s = 1 exactly, so the codes are the converter's RNE of every input."""
    vals = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    vals = vals[torch.isfinite(vals.float()) & (vals.float().abs() < 448)]
    n = (vals.numel() // 127) * 127
    body = vals[:n].reshape(-1, 127)
    x = torch.cat([body, torch.full((body.shape[0], 1), 448.0, dtype=torch.bfloat16)], dim=1)
    x = x.contiguous()  # K = 128
    say(f"fp8 converter sweep over {n} bf16 values")
    q, s = lib.w8a8_quantize_act_fp8(x.cuda(), 0)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quantize_fp8(W.bits(x), 0)
    assert np.all(s_ref == 1.0)
    got = q.cpu().numpy()
    assert np.array_equal(got, q_ref), f"{np.count_nonzero(got != q_ref)} codes differ (sign of zero included)"


GEMM_SHAPES = [(1, 8, 128), (130, 136, 256), (298, 1024, 1024), (257, 264, 384), (64, 8, 17408)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_exact(lib, orc, M, N, K):
    say(f"gemm_i32 M={M} N={N} K={K}")
    q = W.random_codes((M, K), seed=M + 3 * K)
    w = W.random_codes((N, K), seed=N + 5 * K)
    acc = lib.w8a8_gemm_i32(q.cuda(), w.cuda())
    torch.cuda.synchronize()
    ref = orc.gemm_i32(q.numpy(), w.numpy())
    assert np.array_equal(acc.cpu().numpy(), ref)


# One shape per tile the launcher picks, at the workloads' depths (K = 5,120 and
# 17,408: long K loops over the 4-stage ring), in both operand layouts; the last
# runs the persistent 256 x 256 form with two tiles per workgroup, ragged in M and N.
TILE_SHAPES = [(300, 264, 512, "128x128"), (1502, 4096, 5120, "192x128"), (2048, 8192, 17408, "256x256"),
               (4000, 8136, 1024, "256x256")]


@pytest.mark.parametrize("packed", [False, True], ids=["row-major", "packed"])
@pytest.mark.parametrize("M,N,K,tile", TILE_SHAPES, ids=[t[3] + ("-2-per-workgroup" if t[0] == 4000 else "")
                                                          for t in TILE_SHAPES])
def test_gemm_i32_exact_on_every_tile(lib, orc, M, N, K, tile, packed):
    """int32 accumulators bit for bit against the oracle's integer GEMM, on the tile
    shapes and K loops the workloads run (the dequant and SwiGLU epilogues read exactly
    these accumulators)."""
    assert _tile_choice(M, N) == tile
    say(f"gemm_i32 {'packed' if packed else 'row-major'} M={M} N={N} K={K} ({tile} tiles)")
    dev = torch.device("cuda")
    q_h, w_h = W.random_codes((M, K), seed=M + K), W.random_codes((N, K), seed=N + K + 1)
    q_h[1] = 127                          # extreme rows: |acc| up to 127^2 K
    w_h[2] = -127
    q_h[M - 1, ::2] = -127
    q, w = q_h.to(dev), w_h.to(dev)
    if packed:
        acc = lib.w8a8_gemm_i32_packed(lib.w8a8_pack_weight(q), lib.w8a8_pack_weight(w), M, N, K)
    else:
        acc = lib.w8a8_gemm_i32(q, w)
    torch.cuda.synchronize()
    rows = sample_rows(M, n=16, seed=K, tile=256 if tile == "256x256" else 128) if M > 300 else np.arange(M)
    got = acc.cpu().numpy()[rows]
    ref = orc.gemm_i32(np.ascontiguousarray(q_h.numpy()[rows]), w_h.numpy())
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"
    assert int(acc[1, 2]) == -16129 * K


def test_gemm_i32_extremes(lib, orc):
    K = 131072
    say(f"gemm_i32 extreme codes K={K}")
    q = torch.full((3, K), 127, dtype=torch.int8)
    q[1] = -127
    q[2, ::2] = -127
    w = torch.full((8, K), -127, dtype=torch.int8)
    w[1] = 127
    acc = lib.w8a8_gemm_i32(q.cuda(), w.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), orc.gemm_i32(q.numpy(), w.numpy()))
    assert int(acc[0, 0]) == -16129 * K


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_dequant_extremes(lib, orc, packed):
    """Largest K with extreme codes through the dequant epilogue: |acc| up to 127^2 * 2^17, so
    fl32(acc) itself rounds; N = 8, the smallest legal width (the epilogue's clamped column
    loads then stay inside the 8 scales), with a bias."""
    K, M, N = 131072, 3, 8
    say(f"gemm_dequant extreme codes K={K} packed={packed}")
    q = torch.full((M, K), 127, dtype=torch.int8)
    q[1] = -127
    q[2, ::2] = -127
    w = torch.full((N, K), -127, dtype=torch.int8)
    w[1] = 127
    w[2, 1::2] = 127
    w[3] = 0
    s_tok, s_ch, b = _scales_bias(M, N, 61, bias=True)
    if packed:
        y = lib.w8a8_gemm_dequant_packed(lib.w8a8_pack_weight(q.cuda()), s_tok.cuda(), lib.w8a8_pack_weight(w.cuda()),
                                         s_ch.cuda(), K, bias=b.cuda())
    else:
        y = lib.w8a8_gemm_dequant(q.cuda(), s_tok.cuda(), w.cuda(), s_ch.cuda(), b.cuda())
    torch.cuda.synchronize()
    ref = orc.gemm_dequant(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), W.bits(b))
    compare_bf16(bf16_bits(y), ref, "y")


def _scales_bias(M, Nw, seed, bias=True):
    s_tok = W.random_scales(M, seed=seed)
    s_ch = W.random_scales(Nw, seed=seed + 1, lo=1e-5, hi=1e-3)
    b = ((torch.randn(Nw, generator=torch.Generator().manual_seed(seed + 2)) * 0.01).to(torch.bfloat16)
         if bias else None)
    return s_tok, s_ch, b


@pytest.mark.parametrize("M,N,K,bias", [(1, 8, 128, True), (130, 136, 256, False),
                                        (298, 1024, 1024, True), (257, 264, 384, True)])
def test_gemm_dequant(lib, orc, M, N, K, bias):
    say(f"gemm_dequant M={M} N={N} K={K} bias={bias}")
    q = W.random_codes((M, K), seed=11 + M)
    w = W.random_codes((N, K), seed=13 + N)
    s_tok, s_ch, b = _scales_bias(M, N, 17, bias)
    y = lib.w8a8_gemm_dequant(q.cuda(), s_tok.cuda(), w.cuda(), s_ch.cuda(), None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = orc.gemm_dequant(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), None if b is None else W.bits(b))
    compare_bf16(bf16_bits(y), ref, "y")


@pytest.mark.parametrize("M,N,K,bias", [(1, 8, 128, False), (130, 72, 256, True),
                                        (298, 512, 1024, False), (200, 200, 384, True)])
def test_gemm_swiglu(lib, orc, M, N, K, bias):
    say(f"gemm_swiglu M={M} N={N} K={K} bias={bias}")
    q = W.random_codes((M, K), seed=21 + M)
    w = W.random_codes((2 * N, K), seed=23 + N)
    s_tok, s_ch, b = _scales_bias(M, 2 * N, 27, bias)
    y = lib.w8a8_gemm_swiglu(q.cuda(), s_tok.cuda(), w.cuda(), s_ch.cuda(), None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = orc.gemm_swiglu(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), None if b is None else W.bits(b))
    compare_bf16(bf16_bits(y), ref, "y")


def _fp8_codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    return torch.where((c & 0x7F) == 0x7F, c ^ 0x01, c)  # no NaN codes


@pytest.mark.parametrize("M,N,K,bias", [(1, 8, 128, True), (130, 136, 256, False),
                                        (298, 1024, 1024, True), (64, 16, 4096, False)])
def test_fp8_gemm_dequant(lib, orc, M, N, K, bias):
    say(f"fp8_gemm_dequant M={M} N={N} K={K} bias={bias}")
    q = _fp8_codes((M, K), 31 + M)
    w = _fp8_codes((N, K), 37 + N)
    s_tok, s_ch, b = _scales_bias(M, N, 41, bias)
    y = lib.w8a8_fp8_gemm_dequant(q.cuda(), s_tok.cuda(), w.cuda(), s_ch.cuda(), None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = orc.fp8_gemm_dequant(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), None if b is None else W.bits(b))
    compare_bf16(bf16_bits(y), ref, "y")


def test_zero_rows_and_empty_batch(lib, orc):
    say("zero rows / M == 0")
    x = torch.zeros((3, 256), dtype=torch.bfloat16)
    x[1, 5] = 2.0
    q, s = lib.w8a8_quantize_act(x.cuda(), 128)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quantize_i8(W.bits(x), 128)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)
    assert s_ref[0] == 0 and s_ref[2] == 0
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    wq = W.random_codes((8, 256), seed=1).cuda()
    y = lib.w8a8_linear(empty, wq, torch.ones(8, device="cuda"), None, 0)
    assert y.shape == (0, 8)


def test_errors_surface_as_exceptions(lib):
    say("error statuses")
    x = torch.zeros((4, 200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.W8A8Error) as e:
        lib.w8a8_quantize_act(x, 128)
    assert e.value.status == 2
    xb = torch.zeros((4 * 256 + 8,), dtype=torch.bfloat16, device="cuda")[1:1 + 4 * 256].view(4, 256)
    with pytest.raises(lib.W8A8Error) as e:
        lib.w8a8_quantize_act(xb, 0)
    assert e.value.status == 3


def _unpack(flat: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Packed layout (blocks of 32 rows x 64 bytes, block (r // 32, k // 64) at byte
    ((r // 32) * (K // 64) + k // 64) * 2048, row r % 32 at byte 64 * (r % 32) in
    it) -> row-major [rows, K]."""
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    return flat[((r // 32) * (K // 64) + k // 64) * 2048 + (r % 32) * 64 + k % 64]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("M,K,rot", [(1, 64, 0), (33, 192, 0), (298, 1024, 128), (7, 17408, 0),
                                     (65, 4096, 128), (2, 131072, 0)])
def test_quantize_packed(lib, orc, fp8, M, K, rot):
    """The packed-layout quantizer writes the oracle's codes at the packed addresses."""
    say(f"quantize packed fp8={fp8} M={M} K={K} rot={rot}")
    x = _x_case(M, K, rot, seed=300 + M + K, zero_rows=(1,))
    qp, s = (lib.w8a8_quantize_act_fp8_packed if fp8 else lib.w8a8_quantize_act_packed)(x.cuda(), rot)
    torch.cuda.synchronize()
    q_ref, s_ref = (orc.quantize_fp8 if fp8 else orc.quantize_i8)(W.bits(x), rot)
    got = _unpack(qp.cpu().numpy(), M, K)
    (compare_codes_fp8 if fp8 else compare_codes_i8)(got, q_ref, "packed codes")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("kind", ["dequant", "swiglu", "fp8"])
@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (130, 136, 256), (1099, 4088, 256), (2047, 4088, 384),
                                   (4000, 8136, 256)])
def test_gemm_stages_on_packed_operands(lib, orc, kind, M, N, K):
    """Packed activation codes x packed weight codes through the *_packed GEMM entry
    points, against the oracle (tile configurations 128, 192 and 256 all run).  The
    last shape runs the persistent 256 x 256 form with 2 tiles per workgroup (4 for
    SwiGLU: 1,024 tiles of 128 output columns), ragged in M and N, so every workgroup
    carries its operand ring, scales and bias from one tile into the next."""
    if (M, N) == (4000, 8136):
        assert _tile_choice(M, 2 * N if kind == "swiglu" else N) == "256x256"
    say(f"packed gemm {kind} M={M} N={N} K={K}")
    Nw = 2 * N if kind == "swiglu" else N
    if kind == "fp8":
        q, w = _fp8_codes((M, K), 51 + M), _fp8_codes((Nw, K), 53 + N)
    else:
        q, w = W.random_codes((M, K), seed=51 + M), W.random_codes((Nw, K), seed=53 + N)
    s_tok, s_ch, b = _scales_bias(M, Nw, 57, bias=True)
    qp, wp = lib.w8a8_pack_weight(q.cuda()), lib.w8a8_pack_weight(w.cuda())
    fn = {"dequant": lib.w8a8_gemm_dequant_packed, "swiglu": lib.w8a8_gemm_swiglu_packed,
          "fp8": lib.w8a8_fp8_gemm_dequant_packed}[kind]
    y = fn(qp, s_tok.cuda(), wp, s_ch.cuda(), K, bias=b.cuda())
    torch.cuda.synchronize()
    ref_fn = {"dequant": orc.gemm_dequant, "swiglu": orc.gemm_swiglu, "fp8": orc.fp8_gemm_dequant}[kind]
    ref = ref_fn(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), W.bits(b))
    compare_bf16(bf16_bits(y), ref, "y")


def _pow2(exps) -> torch.Tensor:
    return torch.tensor([2.0 ** int(e) for e in exps], dtype=torch.float32)


@pytest.mark.parametrize("M,N,K,case", [(300, 520, 128, "bias"), (1502, 4096, 128, "packed"),
                                        (2048, 8192, 128, "subnormal")])
def test_gemm_dequant_rounding_bit_exact(lib, orc, M, N, K, case):
    """With power-of-two scales every fp32 step of the dequant epilogue is exact
    (|acc| < 2^21 at K = 128, so fl32(acc), the scale product and the FMA lose
    nothing; with the bias, scales >= 1 and integer biases keep the sum below 2^24),
    so the kernel's bf16 must be the oracle's single rounding of the exact value,
    bit for bit: round-half-even ties (values with more than 8 significant bits) and,
    with products of 2^-130 .. 2^-137, bf16 subnormals and underflow to zero.  The
    shapes run the 128 x 128, 192 x 128 and 256 x 256 tiles."""
    say(f"gemm_dequant exact rounding M={M} N={N} K={K} {case}")
    q = W.random_codes((M, K), seed=71 + M)
    w = W.random_codes((N, K), seed=73 + N)
    r, c = np.arange(M), np.arange(N)
    b = None
    if case == "bias":
        s_tok, s_ch = _pow2(r % 3), _pow2(c % 2)
        g = torch.Generator().manual_seed(79)
        b = torch.randint(-256, 257, (N,), generator=g).to(torch.bfloat16)   # integers, exact in bf16
    elif case == "packed":
        s_tok, s_ch = _pow2(r % 3 - 1), _pow2(-(c % 4))
    else:
        s_tok, s_ch = _pow2(-62 - r % 4), _pow2(-68 - c % 5)
    if case == "packed":
        y = lib.w8a8_gemm_dequant_packed(lib.w8a8_pack_weight(q.cuda()), s_tok.cuda(),
                                         lib.w8a8_pack_weight(w.cuda()), s_ch.cuda(), K)
    else:
        y = lib.w8a8_gemm_dequant(q.cuda(), s_tok.cuda(), w.cuda(), s_ch.cuda(), None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = orc.gemm_dequant(q.numpy(), s_tok.numpy(), w.numpy(), s_ch.numpy(), None if b is None else W.bits(b))
    got = bf16_bits(y)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (f"{bad.size} of {got.size} outputs differ; first at {divmod(int(bad[0]), N)}: "
                           f"got {got.flat[bad[0]]:#06x}, oracle {ref.flat[bad[0]]:#06x}")
    if case == "subnormal":   # the case reaches what it is meant to
        mag = got & 0x7FFF
        assert ((mag > 0) & (mag < 0x0080)).sum() > 1000 and (mag >= 0x0080).sum() > 1000
