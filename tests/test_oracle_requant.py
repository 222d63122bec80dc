"""Pins of the oracle's two-step quantization of the SwiGLU output (reading R7).

The next linear's per-token quantizer ("CLEF Calibrated INT8 ConvRot" card,
notes under the latency table) needs a row's amax over all of its columns; the
fused form quantizes 128-column blocks on their own scales first and rescales
them to the row scale afterwards.  What pins it:

* a row of one block: the second step is the identity, so the result is the
  (separately pinned) per-token quantizer's, bit for bit;
* any row: the row scale is the per-token quantizer's scale exactly, every code
  is within one step of single rounding, the block holding the row's amax keeps
  the single-rounding codes, and the dequantized error obeys the two-rounding
  bound |q s - y| <= s/2 + s_b/2;
* a worked example with hand-derived codes (tests/golden/two_step_requant.json)
  that fixes the tie rule and shows a case where the two steps differ from
  single rounding;
* zero rows and zero blocks.
"""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = Path(__file__).parent / "golden" / "two_step_requant.json"


def _h(M, N, seed, outlier_frac=0.01, factor=20.0):
    """SwiGLU-output-like bf16 bits [M, N] (silu(a) * b with outlier columns)."""
    wl = W.custom("linear", M, N, 8, x_kind="silu_product", outlier_frac=outlier_frac,
                  outlier_factor=factor, seed=seed)
    return W.bits(W.make_inputs(wl).x)


def _two_step(h, rot):
    qb, amax = oracle.block_quantize(h, rot)
    return oracle.requantize_blocks(qb, amax), qb, amax


@pytest.mark.parametrize("N,rot", [(128, 0), (128, 128), (64, 0), (96, 0)])
def test_one_block_rows_equal_the_per_token_quantizer(N, rot):
    h = _h(37, N, seed=11)
    (q, s), qb, amax = _two_step(h, rot)
    q1, s1 = oracle.quantize_i8(h, rot)
    np.testing.assert_array_equal(q, q1)
    np.testing.assert_array_equal(s, s1)
    np.testing.assert_array_equal(qb, q1)                       # step 1 alone already is it
    y = oracle.rotate(h, rot)
    np.testing.assert_array_equal(amax[:, 0], np.abs(y).max(axis=1))


@pytest.mark.parametrize("N,rot", [(1024, 0), (1024, 128), (320, 0), (2048, 128)])
def test_row_scale_step_bound_and_amax_block(N, rot):
    h = _h(53, N, seed=12 + N + rot)
    (q, s), qb, amax = _two_step(h, rot)
    q1, s1 = oracle.quantize_i8(h, rot)
    y = oracle.rotate(h, rot).astype(np.float64)
    # the row scale is the per-token scale of the whole (rotated) row, exactly
    np.testing.assert_array_equal(s, s1)
    d = q.astype(np.int32) - q1.astype(np.int32)
    assert np.abs(d).max() <= 1
    nblk = oracle.col_blocks(N)
    assert amax.shape == (53, nblk)
    # the block that holds the row's amax keeps single-rounding codes
    for m in range(53):
        b = int(np.argmax(amax[m]))
        lo, hi = 128 * b, min(128 * b + 128, N)
        np.testing.assert_array_equal(q[m, lo:hi], q1[m, lo:hi])
        np.testing.assert_array_equal(q[m, lo:hi], qb[m, lo:hi])
    # error of the two roundings: |q s - y| <= s/2 + s_b/2 (plus the fp32 quotient and
    # product errors, at most 127 * 2^-23 of a step each)
    s_b = (amax / np.float32(127)).astype(np.float64)
    sb_full = np.repeat(s_b, 128, axis=1)[:, :N]
    err = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None] - y)
    bound = 0.5 * s.astype(np.float64)[:, None] + 0.5 * sb_full
    assert np.all(err <= bound * (1 + 1e-4))
    # and single rounding would respect s/2: the two-step codes differ somewhere
    assert np.count_nonzero(d) > 0


def test_worked_example():
    g = json.loads(GOLDEN.read_text())
    N = g["N"]
    vals = np.zeros((1, N), dtype=np.float32)
    for k, v in g["h"].items():
        vals[0, int(k)] = v
    h = W.bits(torch.from_numpy(vals).bfloat16())
    (q, s), qb, amax = _two_step(h, 0)
    exp_qb = np.zeros(N, np.int8)
    for k, v in g["block_codes"].items():
        exp_qb[int(k)] = v
    exp_q = np.zeros(N, np.int8)
    for k, v in g["codes"].items():
        exp_q[int(k)] = v
    np.testing.assert_array_equal(qb[0], exp_qb)
    np.testing.assert_array_equal(amax[0], np.array(g["block_amax"], np.float32))
    np.testing.assert_array_equal(q[0], exp_q)
    assert s.view(np.uint32)[0] == int(g["s_tok_hex"], 16)
    exp_single = np.zeros(N, np.int8)
    for k, v in g["single_rounding_codes"].items():
        exp_single[int(k)] = v
    q1, s1 = oracle.quantize_i8(h, 0)
    np.testing.assert_array_equal(q1[0], exp_single)
    assert s1[0] == s[0]


def test_zero_rows_and_blocks():
    h = _h(6, 512, seed=13)
    h[1] = 0                       # whole row zero
    h[2, 128:256] = 0              # one block zero
    h[3, :] = 0
    h[3, 300] = 0x3F80             # a single 1.0
    for rot in (0, 128):
        (q, s), qb, amax = _two_step(h, rot)
        assert s[1] == 0 and not q[1].any() and not amax[1].any()
        if rot == 0:
            assert amax[2, 1] == 0 and not q[2, 128:256].any()
            assert np.count_nonzero(q[3]) == 1 and q[3, 300] == 127
        q1, s1 = oracle.quantize_i8(h, rot)
        np.testing.assert_array_equal(s, s1)


def test_whole_gateup_quant_is_swiglu_then_two_steps():
    wl = W.custom("gateup", 19, 256, 384, 0, bias=True, seed=21)
    inp = W.make_inputs(wl)
    x = W.bits(inp.x)
    wq, s_ch = oracle.quantize_i8(W.bits(inp.w), 0)
    b = W.bits(inp.bias)
    for rot_in, rot_out in ((0, 128), (128, 0)):
        q, s = oracle.gateup_swiglu_quant(x, wq, s_ch, b, rot_in, rot_out)
        h = oracle.gateup_swiglu(x, wq, s_ch, b, rot_in)
        q1, s1 = oracle.quantize_i8(h, rot_out)
        np.testing.assert_array_equal(s, s1)
        assert np.abs(q.astype(np.int32) - q1).max() <= 1
        (q2, s2), _, _ = _two_step(h, rot_out)
        np.testing.assert_array_equal(q, q2)
        np.testing.assert_array_equal(s, s2)
