"""Pins of the oracle's gate/up SwiGLU whose output is quantized for the next linear.

The down projection's activations are int8 codes of the SwiGLU output, made by
the same per-token activation quantizer that every INT8 projection's input goes
through ("CLEF Calibrated INT8 ConvRot" card, notes under the latency table),
applied after the paired gate/up epilogue ("Loading CLEF INT8", fuse_mlp).  The
oracle's ``gateup_swiglu_quant`` is checked here against a second, independent
evaluation of that definition written with numpy and scipy only:

* the activation quantizer: the rotation as scipy's dense Sylvester Hadamard
  matrix in fp64, the scale by numpy's IEEE float32 division, the codes by
  numpy's float32 quotient and round-half-even;
* the integer product by numpy's int64 matmul, the epilogue in fp64 with
  scipy's logistic function, and the bf16 rounding of the SwiGLU output by a
  nearest-value search over the bf16 table;
* the output quantizer again as above, with the next linear's rotation.

A mistake in the oracle's composition (rotating with the wrong block, skipping
the bf16 rounding of the SwiGLU output, quantizing per block instead of per
row, a swapped gate/up half) changes codes or scales and fails the comparison.
"""
import numpy as np
import pytest
import torch
from scipy.linalg import hadamard
from scipy.special import expit

import workloads as W

_BF16 = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double().numpy()
_H128 = hadamard(128).astype(np.float64)
_C = np.float64(np.sqrt(0.5)) / 8.0           # fl64(2^-3.5)


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _nearest_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to the even code) of finite fp64 values, by table search."""
    mag = np.abs(v)
    hi = np.clip(np.searchsorted(_BF16, mag, side="left"), 1, len(_BF16) - 1)
    lo = hi - 1
    d_lo, d_hi = mag - _BF16[lo], _BF16[hi] - mag     # exact (Sterbenz) for neighbours
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(mag == _BF16[hi], hi, pick)
    return (pick.astype(np.uint16) | np.where(np.signbit(v), 0x8000, 0).astype(np.uint16))


def _quantize_rows(bits: np.ndarray, rot: int):
    """Per-row int8 quantizer, numpy/scipy only: (codes int8, scales fp32)."""
    x = _bf16_values(bits)
    if rot:
        M, K = x.shape
        y = (x.reshape(M, K // 128, 128) @ _H128.T).reshape(M, K) * _C
        y = y.astype(np.float32)
    else:
        y = x.astype(np.float32)
    amax = np.max(np.abs(y), axis=1)
    s = (amax / np.float32(127)).astype(np.float32)      # IEEE float32 division
    with np.errstate(invalid="ignore", divide="ignore"):
        t = (y / s[:, None]).astype(np.float32)
    t = np.where(s[:, None] > 0, t, np.float32(0))
    q = np.clip(np.rint(t), -127, 127).astype(np.int8)   # rint: half to even
    return q, s


def _reference(x_bits, wq, s_ch, bias_bits, rot_in, rot_out):
    qx, sx = _quantize_rows(x_bits, rot_in)
    N = wq.shape[0] // 2
    acc = qx.astype(np.int64) @ wq.astype(np.int64).T
    b = np.zeros(2 * N) if bias_bits is None else _bf16_values(bias_bits)
    v = acc * sx[:, None].astype(np.float64) * s_ch[None, :].astype(np.float64) + b[None, :]
    g, u = v[:, :N], v[:, N:]
    h = _nearest_bf16_bits(g * expit(g) * u)
    return _quantize_rows(h, rot_out), h


CASES = [(9, 256, 256, 0, 128, True), (5, 384, 128, 128, 0, False), (12, 128, 384, 128, 128, True),
         (3, 256, 192, 0, 0, True)]


@pytest.mark.parametrize("M,K,N,rot_in,rot_out,has_bias", CASES)
def test_matches_independent_per_token_quantizer(orc, M, K, N, rot_in, rot_out, has_bias):
    wl = W.custom("gateup", M, K, N, rot_in, bias=has_bias, seed=M * 31 + N)
    inp = W.make_inputs(wl)
    x, bias = W.bits(inp.x), (W.bits(inp.bias) if has_bias else None)
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), rot_in)
    q, s = orc.gateup_swiglu_quant(x, wq, s_ch, bias, rot_in, rot_out)
    (q_ref, s_ref), h_ref = _reference(x, wq, s_ch, bias, rot_in, rot_out)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "row scales"
    assert np.array_equal(q, q_ref), f"{np.count_nonzero(q != q_ref)} codes differ"
    # the quantizer's codes reach +-127 in every row (per-row scale, not per block)
    assert np.all(np.abs(q).max(axis=1) == 127)
    # and the SwiGLU output it quantizes is the oracle's own gate/up epilogue
    assert np.array_equal(orc.gateup_swiglu(x, wq, s_ch, bias, rot_in), h_ref)


def test_unrounded_or_blockwise_variants_differ(orc):
    """The reference is sensitive to the two plausible mistakes: quantizing the fp64
    SwiGLU value instead of its bf16 rounding, and scaling each 128-column block on its
    own instead of the row."""
    M, K, N = 16, 256, 512
    wl = W.custom("gateup", M, K, N, 0, bias=True, seed=5)
    inp = W.make_inputs(wl)
    x, bias = W.bits(inp.x), W.bits(inp.bias)
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), 0)
    q, s = orc.gateup_swiglu_quant(x, wq, s_ch, bias, 0, 128)
    (q_ref, _), h_bits = _reference(x, wq, s_ch, bias, 0, 128)
    assert np.array_equal(q, q_ref)
    blockwise = np.concatenate([_quantize_rows(np.ascontiguousarray(h_bits[:, c:c + 128]), 128)[0]
                                for c in range(0, N, 128)], axis=1)
    assert not np.array_equal(q, blockwise)
    # fp64 SwiGLU values straight into the rotation (no bf16 rounding): other codes
    qx, sx = _quantize_rows(x, 0)
    acc = qx.astype(np.int64) @ wq.astype(np.int64).T
    v = acc * sx[:, None].astype(np.float64) * s_ch[None, :].astype(np.float64) + _bf16_values(bias)[None, :]
    h64 = v[:, :N] * expit(v[:, :N]) * v[:, N:]
    y = ((h64.reshape(M, N // 128, 128) @ _H128.T).reshape(M, N) * _C).astype(np.float32)
    s64 = (np.max(np.abs(y), axis=1) / np.float32(127)).astype(np.float32)
    q64 = np.rint((y / s64[:, None]).astype(np.float32)).astype(np.int8)
    assert not np.array_equal(q, q64)


def test_zero_rows_and_row_independence(orc):
    M, K, N = 7, 256, 256
    wl = W.custom("gateup", M, K, N, 0, bias=False, seed=8)
    inp = W.make_inputs(wl)
    x = W.bits(inp.x).copy()
    x[2] = 0
    wq, s_ch = orc.quantize_i8(W.bits(inp.w), 0)
    q, s = orc.gateup_swiglu_quant(x, wq, s_ch, None, 0, 128)
    assert s[2] == 0 and not q[2].any()
    q3, s3 = orc.gateup_swiglu_quant(np.ascontiguousarray(x[3:6]), wq, s_ch, None, 0, 128)
    assert np.array_equal(q3, q[3:6]) and np.array_equal(s3, s[3:6])
