"""Pins of the oracle's contraction and epilogues.

The integer contraction has a plain definition (sum_k q[m,k] * w[n,k]), so it is
checked against numpy's int64 matmul and closed forms.  The epilogue (scales +
bias fused after the integer GEMM, "CLEF Calibrated INT8 ConvRot" card,
Benefits list) and the paired gate/up SwiGLU ("Loading CLEF INT8": gate/up
packed into one weight at load time, fuse_mlp) are checked against exact
rational arithmetic and scipy's logistic function; the whole int8 path is
checked against the unquantized fp64 product through an a-priori error bound.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import workloads as W


def _bf16_values():
    codes = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)
    return codes.view(torch.bfloat16).to(torch.float64).numpy()


BF16 = _bf16_values()


def _nearest_bf16_fraction(v: Fraction) -> int:
    """Nearest bf16 code to an exact rational (ties to even), by comparison with neighbours."""
    mag = abs(v)
    j = int(np.searchsorted(BF16, float(mag)))
    best, bestd = None, None
    for c in range(max(0, j - 2), min(len(BF16), j + 2)):
        d = abs(Fraction(float(BF16[c])) - mag)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x8000 if v < 0 else 0)


def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (7, 5, 192), (33, 17, 1024), (298, 64, 1024)])
def test_gemm_i32_matches_numpy(orc, M, N, K):
    q = W.random_codes((M, K), seed=M * 7 + K).numpy()
    w = W.random_codes((N, K), seed=N * 11 + K).numpy()
    ref = q.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(orc.gemm_i32(q, w), ref.astype(np.int32))


def test_gemm_i32_closed_forms(orc):
    K = 17408
    q = np.full((2, K), 127, dtype=np.int8)
    q[1] = -127
    w = np.full((3, K), -127, dtype=np.int8)
    w[1] = 127
    w[2] = 0
    w[2, 5] = 1                          # one-hot column picks q[:, 5]
    acc = orc.gemm_i32(q, w)
    assert acc[0, 0] == -16129 * K and acc[1, 0] == 16129 * K
    assert acc[0, 1] == 16129 * K and acc[1, 1] == -16129 * K
    assert acc[0, 2] == 127 and acc[1, 2] == -127
    big = 131072                         # largest K whose worst case still fits int32
    a = orc.gemm_i32(np.full((1, big), -127, np.int8), np.full((1, big), -127, np.int8))
    assert a[0, 0] == 16129 * big < 2 ** 31


def test_gemm_fp8_is_exact(orc):
    g = np.random.default_rng(41)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q = g.choice(codes, (9, 512)).astype(np.uint8)
    w = g.choice(codes, (6, 512)).astype(np.uint8)
    dq = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    dw = torch.from_numpy(w).view(torch.float8_e4m3fn).double().numpy()
    # products have <= 8 significant bits in [2^-18, 2^17]; their fp64 sums are exact
    assert np.array_equal(orc.gemm_fp8(q, w), dq @ dw.T)


def test_dequant_unit_scales_is_bf16_of_acc(orc):
    q = W.random_codes((5, 256), seed=42).numpy()
    w = W.random_codes((7, 256), seed=43).numpy()
    ones_m = np.ones(5, np.float32)
    ones_n = np.ones(7, np.float32)
    y = orc.gemm_dequant(q, ones_m, w, ones_n, None)
    acc = q.astype(np.int64) @ w.astype(np.int64).T
    want = np.array([[_nearest_bf16_fraction(Fraction(int(a))) for a in row] for row in acc], np.uint16)
    assert np.array_equal(y, want)


def test_dequant_exact_rational(orc):
    M, N, K = 6, 40, 320
    q = W.random_codes((M, K), seed=44).numpy()
    w = W.random_codes((N, K), seed=45).numpy()
    s_tok = W.random_scales(M, seed=46).numpy()
    s_ch = W.random_scales(N, seed=47, lo=1e-5, hi=1e-3).numpy()
    bias = W.bits((torch.randn(N, generator=torch.Generator().manual_seed(48)) * 0.01).to(torch.bfloat16))
    y = orc.gemm_dequant(q, s_tok, w, s_ch, bias)
    acc = q.astype(np.int64) @ w.astype(np.int64).T
    b = _bf16_to_f64(bias)
    for m in range(M):
        for n in range(N):
            v = Fraction(int(acc[m, n])) * Fraction(float(s_tok[m])) * Fraction(float(s_ch[n])) + Fraction(float(b[n]))
            assert int(y[m, n]) == _nearest_bf16_fraction(v), (m, n)
    # bias is added to every row: the NULL-bias result differs exactly by it before rounding
    y0 = orc.gemm_dequant(q, s_tok, w, s_ch, None)
    assert not np.array_equal(y0, y)


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_fp8_dequant_exact_rational(orc):
    """E4M3FN epilogue ("clef-flash-FP8" card, Quantization table: FP8 W8A8 with
    per-token and per-channel scales): y = bf16(sum_k dec(q) dec(w) * s_tok * s_ch + b)
    with one rounding, codes decoded by torch's float8_e4m3fn and the sum, products
    and bias taken as exact rationals."""
    M, N, K = 5, 24, 256
    g = np.random.default_rng(73)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q = g.choice(codes, (M, K)).astype(np.uint8)
    w = g.choice(codes, (N, K)).astype(np.uint8)
    q[1, :] = 0x38                                   # a row of 1.0: the sum is that of w's row
    s_tok = W.random_scales(M, seed=74, lo=1e-3, hi=1.0).numpy()
    s_ch = W.random_scales(N, seed=75, lo=1e-4, hi=1e-2).numpy()
    bias = W.bits((torch.randn(N, generator=torch.Generator().manual_seed(76)) * 0.05).to(torch.bfloat16))
    y = orc.fp8_gemm_dequant(q, s_tok, w, s_ch, bias)
    dq, dw = _e4m3_values(q), _e4m3_values(w)
    b = _bf16_to_f64(bias)
    for m in range(M):
        for n in range(N):
            dot = sum((Fraction(float(a)) * Fraction(float(c)) for a, c in zip(dq[m], dw[n])), Fraction(0))
            v = dot * Fraction(float(s_tok[m])) * Fraction(float(s_ch[n])) + Fraction(float(b[n]))
            assert int(y[m, n]) == _nearest_bf16_fraction(v), (m, n)
    # and without a bias the same rational minus b
    y0 = orc.fp8_gemm_dequant(q, s_tok, w, s_ch, None)
    dot = sum((Fraction(float(a)) * Fraction(float(c)) for a, c in zip(dq[2], dw[3])), Fraction(0))
    assert int(y0[2, 3]) == _nearest_bf16_fraction(dot * Fraction(float(s_tok[2])) * Fraction(float(s_ch[3])))


def test_fp8_linear_through_the_exact_epilogue(orc):
    """The whole fp8 path = the (pinned) E4M3FN quantizer's codes and scales through
    the exact-rational epilogue above, on a small rotated workload."""
    wl = W.custom("fp8", 4, 256, 16, 128, bias=True, seed=77)
    inp = W.make_inputs(wl)
    x, w, bias = W.bits(inp.x), W.bits(inp.w), W.bits(inp.bias)
    wq, s_ch = orc.quantize_fp8(w, 128)
    qx, s_tok = orc.quantize_fp8(x, 128)
    y = orc.fp8_linear(x, wq, s_ch, bias, 128)
    dq, dw = _e4m3_values(qx), _e4m3_values(wq)
    b = _bf16_to_f64(bias)
    for m in range(4):
        for n in range(16):
            dot = sum((Fraction(float(a)) * Fraction(float(c)) for a, c in zip(dq[m], dw[n])), Fraction(0))
            v = dot * Fraction(float(s_tok[m])) * Fraction(float(s_ch[n])) + Fraction(float(b[n]))
            assert int(y[m, n]) == _nearest_bf16_fraction(v), (m, n)


def test_swiglu_packing_and_values(orc):
    M, N, K = 5, 24, 256
    q = W.random_codes((M, K), seed=51).numpy()
    w = W.random_codes((2 * N, K), seed=52).numpy()
    w[3] = 0                              # gate row 3 is zero: silu(0) * u = 0
    s_tok = W.random_scales(M, seed=53).numpy()
    s_ch = W.random_scales(2 * N, seed=54, lo=1e-4, hi=1e-3).numpy()
    bias = W.bits((torch.randn(2 * N, generator=torch.Generator().manual_seed(55)) * 0.05).to(torch.bfloat16))
    bias[3] = 0
    y = orc.gemm_swiglu(q, s_tok, w, s_ch, bias)
    assert y.shape == (M, N)
    acc = q.astype(np.int64) @ w.astype(np.int64).T
    b = _bf16_to_f64(bias)
    vals = acc * s_tok[:, None].astype(np.float64) * s_ch[None, :].astype(np.float64) + b[None, :]
    g, u = vals[:, :N], vals[:, N:]
    ref = g * expit(g) * u                # gate = first half of the packed rows
    got = _bf16_to_f64(y)
    assert np.all((y[:, 3] & 0x7FFF) == 0)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9))
    swapped = u * expit(u) * g            # a transposed packing would give this
    assert not np.allclose(got, swapped, rtol=1e-2)


def test_silu_limits(orc):
    K = 64
    q = np.ones((1, K), dtype=np.int8)
    w = np.zeros((4, K), dtype=np.int8)
    w[0] = 100                            # gate 0: large positive; up 0 (row 2) = 1
    w[1] = -100                           # gate 1: large negative
    w[2] = 1
    w[3] = 1
    s_tok = np.ones(1, np.float32)
    s_ch = np.array([1.0, 1.0, 0.5, 0.5], np.float32)
    y = _bf16_to_f64(orc.gemm_swiglu(q, s_tok, w, s_ch, None))
    assert y[0, 0] == 6400.0 * 32.0        # silu(6400) = 6400 in fp64; times up = 32
    assert y[0, 1] == 0.0 and np.signbit(y[0, 1])   # silu(-6400) = -0 (underflow), times 32


def test_linear_is_quantize_then_gemm_dequant(orc):
    wl = W.custom("linear", 40, 512, 72, 128, seed=56)
    inp = W.make_inputs(wl)
    x, w, bias = W.bits(inp.x), W.bits(inp.w), W.bits(inp.bias)
    wq, s_ch = orc.quantize_i8(w, 128)
    q, s_tok = orc.quantize_i8(x, 128)
    assert np.array_equal(orc.linear(x, wq, s_ch, bias, 128), orc.gemm_dequant(q, s_tok, wq, s_ch, bias))
    wqf, s_chf = orc.quantize_fp8(w, 128)
    qf, s_tokf = orc.quantize_fp8(x, 128)
    assert np.array_equal(orc.fp8_linear(x, wqf, s_chf, bias, 128),
                          orc.fp8_gemm_dequant(qf, s_tokf, wqf, s_chf, bias))
    wg = W.bits(torch.cat([inp.w, inp.w.flip(0)]))
    wgq, s_g = orc.quantize_i8(wg, 128)
    assert np.array_equal(orc.gateup_swiglu(x, wgq, s_g, None, 128), orc.gemm_swiglu(q, s_tok, wgq, s_g, None))


def test_linear_error_bound_against_unquantized(orc):
    """|y_q - (x W^T + b)| <= s_tok/2 sum|W| + s_ch/2 sum|x| + K s_tok s_ch / 4 + bf16 half-ulp."""
    wl = W.WORKLOADS["short_298x1024x1024"]
    inp = W.make_inputs(wl)
    x, w, bias = W.bits(inp.x), W.bits(inp.w), W.bits(inp.bias)
    wq, s_ch = orc.quantize_i8(w)
    q, s_tok = orc.quantize_i8(x)
    y = _bf16_to_f64(orc.linear(x, wq, s_ch, bias))
    xf, wf, bf = inp.x.double().numpy(), inp.w.double().numpy(), inp.bias.double().numpy()
    exact = xf @ wf.T + bf
    bound = (s_tok[:, None] / 2 * np.abs(wf).sum(1)[None, :] * (1 + 2.0 ** -16)
             + s_ch[None, :] / 2 * np.abs(xf).sum(1)[:, None] * (1 + 2.0 ** -16)
             + wl.K * s_tok[:, None] * s_ch[None, :] / 4
             + np.abs(y) * 2.0 ** -8)
    assert np.all(np.abs(y - exact) <= bound)
    # and the error is a small fraction of the output scale (the method is usable)
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel < 0.05


# ---- unfused gate/up ("Loading CLEF INT8", fuse_mlp=False) ----------------------
def _bf16_bits_of(v):
    return W.bits(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16))


def test_swiglu_bf16_against_expit(orc):
    """silu(g) * u on bf16 inputs, one rounding: within half a bf16 ulp of an fp64
    evaluation through scipy's logistic function (an implementation independent of
    the oracle's), over a wide range of magnitudes and signs."""
    g_t = torch.randn(64, 96, generator=torch.Generator().manual_seed(61), dtype=torch.float64) * 4
    u_t = torch.randn(64, 96, generator=torch.Generator().manual_seed(62), dtype=torch.float64) * 3
    g_t[0, :8] = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 80.0, -80.0, 1000.0, -1000.0])
    g, u = W.bits(g_t.to(torch.bfloat16)), W.bits(u_t.to(torch.bfloat16))
    y = orc.swiglu_bf16(g, u)
    gv, uv = _bf16_to_f64(g), _bf16_to_f64(u)
    ref = gv * expit(gv) * uv
    got = _bf16_to_f64(y)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9))


def test_swiglu_bf16_identities(orc):
    """silu(g) - silu(-g) = g (with u = 1, up to the two output roundings); silu(0) = 0;
    silu(g) -> g for large g and -> -0 for large negative g; odd in u."""
    g = _bf16_bits_of(np.linspace(-12, 12, 97).reshape(1, -1))
    gn = _bf16_bits_of(-np.linspace(-12, 12, 97).reshape(1, -1))
    one = _bf16_bits_of(np.ones((1, 97)))
    y_pos, y_neg = _bf16_to_f64(orc.swiglu_bf16(g, one)), _bf16_to_f64(orc.swiglu_bf16(gn, one))
    gv = _bf16_to_f64(g)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(gv), 1e-38))) - 7)
    assert np.all(np.abs((y_pos - y_neg) - gv) <= ulp)
    assert _bf16_to_f64(orc.swiglu_bf16(_bf16_bits_of([[0.0]]), _bf16_bits_of([[5.0]])))[0, 0] == 0.0
    big = orc.swiglu_bf16(_bf16_bits_of([[64.0, -800.0]]), _bf16_bits_of([[3.0, 3.0]]))
    assert _bf16_to_f64(big)[0, 0] == 192.0
    assert _bf16_to_f64(big)[0, 1] == 0.0 and np.signbit(_bf16_to_f64(big)[0, 1])
    mu = orc.swiglu_bf16(g, _bf16_bits_of(-np.ones((1, 97))))
    assert np.array_equal(_bf16_to_f64(mu), -y_pos)


def test_gateup_unfused_is_linear_then_swiglu(orc):
    """The unfused path rounds gate and up to bf16 (the 2N-column linear) before the
    SwiGLU, so it equals swiglu_bf16 of the linear's halves -- and differs from the
    fused epilogue only by that intermediate rounding."""
    wl = W.custom("gateup", 33, 384, 40, 128, bias=True, seed=63)
    inp = W.make_inputs(wl)
    x, w, bias = W.bits(inp.x), W.bits(inp.w), W.bits(inp.bias)
    wq, s_ch = orc.quantize_i8(w, 128)
    h = orc.linear(x, wq, s_ch, bias, 128)
    assert h.shape == (33, 80)
    y = orc.gateup_unfused(x, wq, s_ch, bias, 128)
    assert np.array_equal(y, orc.swiglu_bf16(h[:, :40], h[:, 40:]))
    fused = _bf16_to_f64(orc.gateup_swiglu(x, wq, s_ch, bias, 128))
    unf = _bf16_to_f64(y)
    scale = np.sqrt(np.mean(fused ** 2))
    assert np.max(np.abs(unf - fused)) <= 0.03 * scale          # one extra bf16 rounding of g and u
    assert not np.array_equal(unf, fused)
