"""Pins of the oracle's per-row symmetric quantizers.

The pages fix the granularity (per token, dynamic, for activations; per output
channel, straight from the weights, for weights: clef-flash-FP8 card,
Quantization table and the note after recipe.yaml; per-token int8 activations
from the ConvRot quantizer on the INT8 ConvRot card).  The readings for the
rest (amax/127 and amax/448, IEEE fp32 division, round half to even, OCP
E4M3FN with saturation, zero rows) are stated in the oracle's header.  These
tests pin the oracle against exact rational arithmetic (Python fractions),
against torch's E4M3FN cast, and against the invariants any correct symmetric
quantizer has.
"""
from fractions import Fraction

import numpy as np
import torch

import workloads as W


def _rows(seed, M=16, K=512, outliers=True):
    wl = W.custom("linear", M, K, 8, 0, outlier_frac=0.02 if outliers else 0.0,
                  outlier_factor=30.0, seed=seed)
    return W.bits(W.make_inputs(wl).x), W.make_inputs(wl).x.float().numpy()


def _rne(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_scale_is_correctly_rounded_amax_over_127(orc):
    x, xf = _rows(31)
    q, s = orc.quantize_i8(x)
    for m in range(xf.shape[0]):
        amax = Fraction(float(np.max(np.abs(xf[m]))))
        exact = amax / 127
        err = abs(Fraction(float(s[m])) - exact)
        assert err <= Fraction(float(np.spacing(np.float32(s[m])))) / 2


def test_int8_codes_match_exact_rational_rounding(orc):
    """q == RNE(y / s) with y / s exact, except where y / s sits within fp32 rounding of a tie."""
    x, xf = _rows(32, M=32, K=1024)
    q, s = orc.quantize_i8(x)
    near_ties = 0
    for m in range(xf.shape[0]):
        sm = Fraction(float(s[m]))
        for k in range(xf.shape[1]):
            t = Fraction(float(xf[m, k])) / sm
            want = max(-127, min(127, _rne(t)))
            if int(q[m, k]) != want:
                frac = t - (t.numerator // t.denominator)
                assert abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 16), (m, k, float(t))
                near_ties += 1
    assert near_ties <= 2


def test_int8_invariants(orc):
    x, xf = _rows(33, M=64, K=768)
    q, s = orc.quantize_i8(x)
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert np.all((np.sign(q) == np.sign(xf)) | (q == 0))
    for m in range(xf.shape[0]):
        order = np.argsort(xf[m], kind="stable")
        assert np.all(np.diff(q[m, order].astype(int)) >= 0)  # monotone in x
    err = np.abs(q.astype(np.float64) * s[:, None] - xf)
    # |q - y/s| <= 1/2 + half an fp32 ulp of the quotient (< 128): at most 1/2 + 2^-18
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 2.0 ** -17))


def test_int8_power_of_two_scaling(orc):
    x, xf = _rows(34)
    q, s = orc.quantize_i8(x)
    for e in (-5, 3, 17):
        x2 = W.bits(torch.from_numpy(xf * np.float32(2.0 ** e)).to(torch.bfloat16))
        q2, s2 = orc.quantize_i8(x2)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (s * np.float32(2.0 ** e)).astype(np.float32))


def test_int8_requantization_is_idempotent(orc):
    x, xf = _rows(35, M=64, K=1024)
    q, s = orc.quantize_i8(x)
    y2 = (q.astype(np.float32) * s[:, None]).astype(np.float32)
    q2, s2 = orc.quantize_f32_i8(y2)
    assert np.array_equal(q2, q)
    ulp = np.spacing(s)
    assert np.all(np.abs(s2.astype(np.float64) - s) <= ulp)


def test_zero_rows_give_zero_scale_and_codes(orc):
    x, _ = _rows(36, M=4, K=256)
    x = x.copy()
    x[1] = 0
    x[3] = 0x8000  # -0.0
    q, s = orc.quantize_i8(x)
    assert s[1] == 0 and s[3] == 0 and not q[1].any() and not q[3].any()
    assert s[0] > 0 and s[2] > 0
    qf, sf = orc.quantize_fp8(x)
    assert sf[1] == 0 and sf[3] == 0
    assert np.all(orc.e4m3_decode(qf[1]) == 0) and np.all(orc.e4m3_decode(qf[3]) == 0)


def test_rotated_quantizer_is_rotation_then_quantizer(orc):
    wl = W.custom("linear", 24, 1024, 8, 128, outlier_frac=0.005, outlier_factor=50.0, seed=37)
    x = W.bits(W.make_inputs(wl).x)
    q, s = orc.quantize_i8(x, 128)
    q2, s2 = orc.quantize_f32_i8(orc.rotate(x, 128))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    qf, sf = orc.quantize_fp8(x, 128)
    qf2, sf2 = orc.quantize_f32_fp8(orc.rotate(x, 128))
    assert np.array_equal(qf, qf2) and np.array_equal(sf, sf2)


def test_fp8_scale_codes_and_torch_cast(orc):
    x, xf = _rows(38, M=32, K=1024)
    q, s = orc.quantize_fp8(x)
    dec = orc.e4m3_decode(q)
    assert np.all(np.abs(dec).max(axis=1) == 448.0)
    assert np.all((np.sign(dec) == np.sign(xf)) | (dec == 0))
    for m in range(xf.shape[0]):
        amax = Fraction(float(np.max(np.abs(xf[m]))))
        assert abs(Fraction(float(s[m])) - amax / 448) <= Fraction(float(np.spacing(np.float32(s[m])))) / 2
    # the code is torch's E4M3FN cast of the clamped fp32 quotient
    t = np.clip((xf / s[:, None]).astype(np.float32), -448, 448).astype(np.float32)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_decode(q), orc.e4m3_decode(ref))
    # and it is within half an E4M3 spacing of the scaled input
    spacing = np.where(np.abs(dec) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(dec), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(dec - xf / s[:, None].astype(np.float64)) <= spacing * 0.5 * (1 + 1e-6) + 1e-30)


def test_fp8_power_of_two_scaling(orc):
    x, xf = _rows(39)
    q, s = orc.quantize_fp8(x)
    x2 = W.bits(torch.from_numpy(xf * np.float32(2.0 ** -7)).to(torch.bfloat16))
    q2, s2 = orc.quantize_fp8(x2)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, (s * np.float32(2.0 ** -7)).astype(np.float32))
