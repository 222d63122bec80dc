"""Comparison helpers shared by the GPU parity tests (no arithmetic of the method).

Tolerances for the bf16 outputs (derived for a single final bf16 rounding of an
fp32 epilogue against the oracle's fp64 epilogue): every element within a
relative error of 1e-2, measured against max(|ref|, 1e-3 * rms(ref)) so that
outputs that cancel to near zero are judged on the tensor's scale; and at least
99.9 % of the elements within 2 bf16 ulps of the oracle (the ulp of the
oracle's value).  Quantized codes must match bit for bit, except that a code
may move by one step (a rounding tie decided differently) in at most 1e-4 of
the elements.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

REL_TOL = 1e-2
ULP_FRAC = 0.999
ULPS = 2
FLIP_BUDGET = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def compare_bf16(got_bits: np.ndarray, ref_bits: np.ndarray, what: str) -> dict:
    got, ref = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    denom = np.maximum(np.abs(ref), 1e-3 * rms)
    err = np.abs(got - ref)
    rel = np.where(denom > 0, err / np.where(denom > 0, denom, 1), err)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))) - 7)
    within = err <= ULPS * ulp
    stats = {"n": int(ref.size), "max_rel": float(rel.max()) if ref.size else 0.0,
             "frac_within_2ulp": float(within.mean()) if ref.size else 1.0,
             "frac_equal": float((got_bits == ref_bits).mean()) if ref.size else 1.0}
    say(f"  {what}: {stats}")
    assert stats["max_rel"] <= REL_TOL, f"{what}: max relative error {stats['max_rel']}"
    assert stats["frac_within_2ulp"] >= ULP_FRAC, f"{what}: only {stats['frac_within_2ulp']} within 2 ulp"
    return stats


def compare_codes_i8(got: np.ndarray, ref: np.ndarray, what: str) -> int:
    diff = got.astype(np.int16) - ref.astype(np.int16)
    flips = int(np.count_nonzero(diff))
    say(f"  {what}: {flips} flipped codes of {ref.size}")
    assert np.all(np.abs(diff) <= 1), f"{what}: a code differs by more than one step"
    assert flips <= FLIP_BUDGET * max(ref.size, 1), f"{what}: {flips} flips exceed the budget"
    return flips


def _e4m3_rank(codes: np.ndarray) -> np.ndarray:
    """Signed position on the E4M3FN number line (+0 and -0 both rank 0)."""
    mag = (codes & 0x7F).astype(np.int16)
    return np.where(codes & 0x80, -mag, mag)


def compare_codes_fp8(got: np.ndarray, ref: np.ndarray, what: str) -> int:
    diff = _e4m3_rank(got) - _e4m3_rank(ref)
    flips = int(np.count_nonzero(diff))
    say(f"  {what}: {flips} flipped codes of {ref.size}")
    assert np.all(np.abs(diff) <= 1), f"{what}: a code differs by more than one step"
    assert flips <= FLIP_BUDGET * max(ref.size, 1), f"{what}: {flips} flips exceed the budget"
    return flips


def sample_rows(M: int, n: int = 48, seed: int = 0, tile: int = 128) -> np.ndarray:
    """First/last rows, rows on each side of the first tile boundaries, plus a seeded sample."""
    fixed = {0, 1, M - 2, M - 1}
    for b in (tile, 2 * tile, (M // tile) * tile):
        fixed |= {b - 1, b}
    fixed = {r for r in fixed if 0 <= r < M}
    rng = np.random.default_rng(seed)
    rest = [r for r in rng.permutation(M)[: n * 2] if r not in fixed]
    rows = sorted(fixed | set(int(r) for r in rest[: max(0, n - len(fixed))]))
    return np.array(rows, dtype=np.int64)


def tile_choice(M: int, N: int) -> str:
    """The GEMM launcher's tile for M tokens x N weight rows (2N for gate/up): the least
    ceil(tiles / 256) * tile area / efficiency over 256x256 (1.0), 192x128 (0.9) and
    128x128 (0.8), ties to the larger tile.  256x256 launches run the persistent form
    when K >= 256 and the output is under 2^31 bytes."""
    def cost(bm, bn, eff):
        tiles = -(-M // bm) * -(-N // bn)
        return -(-tiles // 256) * bm * bn / eff
    c256, c192, c128 = cost(256, 256, 1.0), cost(192, 128, 0.9), cost(128, 128, 0.8)
    if c256 <= c192 and c256 <= c128:
        return "256x256"
    return "192x128" if c192 <= c128 else "128x128"
