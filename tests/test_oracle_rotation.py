"""Pins of the oracle's block rotation.

The pages name the rotation ("ConvRot", "CLEF Calibrated INT8 ConvRot" card,
Benefits list and latency-table notes) without defining it; the reading taken
is the normalized Sylvester Walsh-Hadamard transform H_128 / sqrt(128) on every
block of 128 consecutive input features, applied alike to activations and
weights.  These tests pin the oracle's version against scipy's Sylvester
Hadamard matrix (a library routine) and against the invariants that make the
rotation usable: orthogonality, symmetry (it is its own inverse), block
independence and x.W^T == (xR).(WR)^T.
"""
import numpy as np
import pytest
import torch
from scipy.linalg import hadamard

import workloads as W

C = np.sqrt(np.float64(0.5)) / 8  # fl64(2^-3.5): sqrt is correctly rounded, /8 is exact


def _bf16(a):
    return W.bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_rotation_matrix_is_scipy_sylvester(orc):
    eye = _bf16(np.eye(128, dtype=np.float32))
    R = orc.rotate(eye, 128)                       # row i = rotation of e_i = H[i, :] / sqrt(128)
    H = hadamard(128).astype(np.float64)
    assert np.array_equal(R, (H * C).astype(np.float32))


def test_rotation_constant_block_goes_to_first_coefficient(orc):
    x = _bf16(np.full((1, 256), 1.5, dtype=np.float32))
    y = orc.rotate(x, 128)[0]
    for b in (0, 128):
        assert y[b] == np.float32(1.5 * 128 * C)
        assert np.all(y[b + 1:b + 128] == 0)


def test_rotation_matches_dense_fp64_product(orc):
    wl = W.custom("linear", 64, 1024, 16, 128, outlier_frac=0.02, outlier_factor=50.0, seed=21)
    x = W.bits(W.make_inputs(wl).x)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    H = hadamard(128).astype(np.float64)
    ref = (xf.reshape(64, 8, 128) @ H.T * C).astype(np.float32).reshape(64, 1024)
    assert np.array_equal(orc.rotate(x, 128), ref)


def test_rotation_is_orthogonal_and_involutive(orc):
    R = orc.rotate(_bf16(np.eye(128, dtype=np.float32)), 128).astype(np.float64)
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-6, rtol=0)
    assert np.allclose(R @ R, np.eye(128), atol=1e-6, rtol=0)   # symmetric: its own inverse
    assert np.array_equal(R, R.T)


def test_rotation_blocks_are_independent(orc):
    g = np.random.default_rng(22)
    x = _bf16(g.standard_normal((4, 384)).astype(np.float32))
    whole = orc.rotate(x, 128)
    for b in range(3):
        part = orc.rotate(np.ascontiguousarray(x[:, 128 * b:128 * (b + 1)]), 128)
        assert np.array_equal(whole[:, 128 * b:128 * (b + 1)], part)


def test_rotation_preserves_norms_and_products(orc):
    wl = W.custom("linear", 32, 512, 48, 128, seed=23)
    inp = W.make_inputs(wl)
    x, w = W.bits(inp.x), W.bits(inp.w)
    xf = inp.x.double().numpy()
    wf = inp.w.double().numpy()
    xr = orc.rotate(x, 128).astype(np.float64)
    wr = orc.rotate(w, 128).astype(np.float64)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-6)
    ref = xf @ wf.T
    got = xr @ wr.T
    scale = np.abs(xf) @ np.abs(wf).T
    assert np.max(np.abs(got - ref) / scale) < 1e-6


def test_no_rotation_is_plain_widening(orc):
    g = np.random.default_rng(24)
    x = _bf16(g.standard_normal((3, 200)).astype(np.float32))
    y = orc.rotate(x, 0)
    ref = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(y, ref)
