"""Pins of the oracle's number codecs against library routines and published values.

bf16: torch's bfloat16 (decode all 65,536 codes; fp32 -> bf16 round to nearest
even) and a brute-force nearest search over every finite bf16 for fp64 inputs.
E4M3FN: torch's float8_e4m3fn (decode all 256 codes, encode) and the OCP OFP8
table in tests/golden/e4m3fn_values.json, which the FP8 W8A8 dynamic scheme of
the clef-flash-FP8 card (Quantization table) stores values in.
"""
import json
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

GOLDEN = Path(__file__).parent / "golden"


def _bf16_table():
    codes = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)
    return codes.view(torch.bfloat16).to(torch.float64).numpy()  # ascending, finite, >= 0


def test_bf16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint16)
    ours = orc.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_matches_torch_on_fp32(orc):
    g = np.random.default_rng(11)
    v = (g.standard_normal(200_000) * np.exp2(g.integers(-60, 60, 200_000))).astype(np.float32)
    ours = orc.bf16_from_f64(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _nearest_bf16_bruteforce(v, table):
    """Nearest finite bf16 by exhaustive distance over the candidates around v (ties: even code)."""
    out = np.empty(v.shape, dtype=np.uint16)
    for i, x in enumerate(v):
        mag = abs(x)
        j = int(np.searchsorted(table, mag))
        best, bestd = None, None
        for c in range(max(0, j - 2), min(len(table), j + 2)):
            d = abs(Fraction(float(table[c])) - Fraction(float(mag)))
            if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
        out[i] = best | (0x8000 if np.signbit(x) else 0)
    return out


def test_bf16_encode_fp64_bruteforce(orc):
    table = _bf16_table()
    g = np.random.default_rng(12)
    v = g.standard_normal(3000) * np.exp2(g.integers(-40, 40, 3000))
    ours = orc.bf16_from_f64(v)
    assert np.array_equal(ours, _nearest_bf16_bruteforce(v, table))


@pytest.mark.parametrize("value,code", [
    (1.0 + 2.0 ** -8, 0x3F80),                   # halfway 1 .. 1+2^-7: even is 1.0
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # halfway 1+2^-7 .. 1+2^-6: even is 1+2^-6
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # just above the tie
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -133, 0x0001),                       # smallest subnormal bf16
])
def test_bf16_encode_ties_and_edges(orc, value, code):
    assert int(orc.bf16_from_f64(np.array([value]))[0]) == code


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_golden_table(orc):
    gold = json.loads((GOLDEN / "e4m3fn_values.json").read_text())
    for row in gold["decode"]:
        got = float(orc.e4m3_decode(np.array([int(row["code"], 16)], dtype=np.uint8))[0])
        if row["value"] == "nan":
            assert np.isnan(got)
        else:
            assert got == row["value"] and np.signbit(got) == np.signbit(row["value"]), row
    for row in gold["encode_round_to_nearest_even"]:
        got = int(orc.e4m3_encode(np.array([row["input"]], dtype=np.float32))[0])
        assert got == int(row["code"], 16), row


def test_e4m3_encode_vs_torch_all_bf16_in_range(orc):
    vals = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals) & (vals.abs() <= 448)]
    ours = orc.e4m3_encode(vals.numpy())
    ref = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +0 and -0 are both zero; compare decoded values and signs
    assert np.array_equal(orc.e4m3_decode(ours), orc.e4m3_decode(ref))
    assert np.array_equal(ours, ref)


def test_e4m3_encode_vs_torch_random_fp32(orc):
    g = np.random.default_rng(13)
    n = 1_000_000
    t = (g.uniform(-1, 1, n) * np.exp2(g.uniform(-14, 8.8, n))).astype(np.float32)
    t = np.clip(t, -448, 448).astype(np.float32)
    ours = orc.e4m3_encode(t)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_is_nearest_bruteforce(orc):
    """Every code is the nearest E4M3FN value (exhaustive over the 127 non-negative codes)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    values = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    g = np.random.default_rng(14)
    t = np.clip(g.standard_normal(20000) * 60, -448, 448).astype(np.float32)
    ours = orc.e4m3_encode(t)
    dec = np.abs(orc.e4m3_decode(ours))
    dist = np.abs(np.abs(t.astype(np.float64))[:, None] - values[None, :])
    best = dist.min(axis=1)
    assert np.array_equal(np.abs(dec - np.abs(t.astype(np.float64))), best)
