"""Seeded synthetic inputs for the W8A8 projection workloads.

This module only draws random numbers and casts them to the input dtypes.  It
holds none of the method's arithmetic (no rotation, no scaling, no rounding to
int8 or fp8), so both the GPU library's tests and the CPU oracle can take their
inputs from it without sharing any of the computation.

The pages measure whole models on private text records (the "CLEF Calibrated
INT8 ConvRot" card's memory and latency tables: 298 to 2,270 tokens, batch 1,
and equal-length batches of 1,502-token records).  Those records are not
available; the seeded tensors below stand in for one decoder projection's
activations and weights at those token counts.

Recipe (per workload, one ``torch.Generator`` seeded with ``seed``), drawn in
this order, all in fp32 on the CPU:
  1. x_raw = randn(M, K)   -- for the down projection instead a = randn(M, K),
     b = randn(M, K) and x_raw = silu(a) * b (an MLP hidden state);
  2. outlier channels = randperm(K)[:round(p * K)];
  3. w_raw = randn(N_w, K) * sigma_w   (N_w = 2N for the packed gate/up pair);
  4. bias = randn(N_w) * 0.01 where the workload has a bias;
  5. x_raw[:, outliers] *= factor; x = bf16(x_raw), w = bf16(w_raw),
     bias = bf16(bias) (round to nearest even, torch's cast).
``N(0, s)`` means standard deviation ``s``.
"""
from __future__ import annotations

from dataclasses import dataclass
import math
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "linear" | "gateup" | "fp8"
    M: int
    K: int
    N: int                 # output features (per half for "gateup")
    rot_block: int         # 0 or 128
    sigma_w: float
    bias: bool
    outlier_frac: float    # fraction of K channels scaled
    outlier_factor: float
    x_kind: str = "normal"  # "normal" | "silu_product"
    seed: int = 0

    @property
    def n_w(self) -> int:
        """Rows of the (packed) weight matrix."""
        return 2 * self.N if self.kind == "gateup" else self.N

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.K))

    @property
    def ops(self) -> int:
        """Multiply-adds x2 of the contraction (all packed rows count)."""
        return 2 * self.M * self.n_w * self.K

    def with_m(self, M: int) -> "Workload":
        return Workload(self.name, self.kind, M, self.K, self.N, self.rot_block, self.sigma_w,
                        self.bias, self.outlier_frac, self.outlier_factor, self.x_kind, self.seed)


# The five workloads: a short 298-token input; a 1,502-token input with the
# block-128 rotation; the packed gate/up projection at 2,270 tokens; the down
# projection over 8 records of 1,502 tokens with rotation; an fp8 projection at
# 16,384 tokens.
WORKLOADS = {
    "short_298x1024x1024": Workload("short_298x1024x1024", "linear", 298, 1024, 1024, 0,
                                    0.02, True, 0.01, 20.0, seed=1000),
    "rot_1502x4096x4096": Workload("rot_1502x4096x4096", "linear", 1502, 4096, 4096, 128,
                                   0.02, True, 0.005, 50.0, seed=2000),
    "gateup_2270x5120x2x17408": Workload("gateup_2270x5120x2x17408", "gateup", 2270, 5120, 17408, 0,
                                         0.02, False, 0.01, 20.0, seed=3000),
    "down_12016x17408x5120": Workload("down_12016x17408x5120", "linear", 12016, 17408, 5120, 128,
                                      0.01, True, 0.0, 1.0, x_kind="silu_product", seed=4000),
    "fp8_16384x4096x12288": Workload("fp8_16384x4096x12288", "fp8", 16384, 4096, 12288, 0,
                                     0.02, False, 0.01, 20.0, seed=5000),
}
ORDER = list(WORKLOADS)


def custom(kind: str, M: int, K: int, N: int, rot_block: int = 0, *, bias: bool = True,
           sigma_w: float = 0.02, outlier_frac: float = 0.01, outlier_factor: float = 20.0,
           x_kind: str = "normal", seed: int = 7) -> Workload:
    """A workload of the same recipe at another shape (for the parity tests)."""
    return Workload(f"{kind}_{M}x{K}x{N}_r{rot_block}", kind, M, K, N, rot_block, sigma_w, bias,
                    outlier_frac, outlier_factor, x_kind, seed)


@dataclass
class Inputs:
    x: torch.Tensor                 # bf16 [M, K]
    w: torch.Tensor                 # bf16 [N_w, K]  (unquantized weight)
    bias: Optional[torch.Tensor]    # bf16 [N_w] or None
    outliers: torch.Tensor          # int64 channel indices


def make_inputs(wl: Workload, rows: Optional[int] = None) -> Inputs:
    """Draw the workload's tensors on the CPU.  ``rows`` keeps only the first rows of x
    (the draw is the same, so the kept rows equal the full draw's first rows)."""
    g = torch.Generator().manual_seed(wl.seed)
    M, K = wl.M, wl.K
    if wl.x_kind == "silu_product":
        a = torch.randn(M, K, generator=g)
        b = torch.randn(M, K, generator=g)
        x_raw = torch.nn.functional.silu(a) * b
        del a, b
    else:
        x_raw = torch.randn(M, K, generator=g)
    outliers = torch.randperm(K, generator=g)[: wl.n_outliers]
    w_raw = torch.randn(wl.n_w, K, generator=g) * wl.sigma_w
    bias = (torch.randn(wl.n_w, generator=g) * 0.01) if wl.bias else None
    if rows is not None:
        x_raw = x_raw[:rows]
    if len(outliers):
        x_raw[:, outliers] *= wl.outlier_factor
    return Inputs(x=x_raw.to(torch.bfloat16).contiguous(),
                  w=w_raw.to(torch.bfloat16).contiguous(),
                  bias=None if bias is None else bias.to(torch.bfloat16).contiguous(),
                  outliers=outliers)


def random_codes(shape, seed: int, lo: int = -127, hi: int = 127) -> torch.Tensor:
    """Uniform random int8 codes in [lo, hi] (inputs of the stand-alone GEMM tests)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int64).to(torch.int8)


def random_scales(n: int, seed: int, lo: float = 1e-4, hi: float = 1e-1) -> torch.Tensor:
    """Positive fp32 scales, log-uniform in [lo, hi]."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return torch.exp(torch.log(torch.tensor(lo)) + u * (torch.log(torch.tensor(hi)) - torch.log(torch.tensor(lo)))).float()


def bits(t: torch.Tensor):
    """numpy view of a CPU bf16 tensor's raw bit patterns (uint16)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a) -> torch.Tensor:
    """CPU bf16 tensor from a numpy uint16 array of bit patterns."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


# ------------------------------------------------------------------------------
# Draws made directly on a device, for the cases whose tensors are too large to
# draw on the CPU in a test's time (inputs of several GiB).  Both sides still take
# the same tensor: the oracle reads the rows it checks back from the device.

def _device_generator(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def device_normal_bf16(rows: int, K: int, seed: int, device, outlier_frac: float = 0.01,
                       outlier_factor: float = 20.0, sigma: float = 1.0) -> torch.Tensor:
    """bf16 [rows, K]: N(0, 1) drawn in bf16 on ``device`` and multiplied by ``sigma``
    (in bf16), then a seeded set of round(outlier_frac * K) columns multiplied by
    ``outlier_factor`` (in bf16)."""
    g = _device_generator(seed, device)
    x = torch.randn(rows, K, generator=g, dtype=torch.bfloat16, device=device)
    if sigma != 1.0:
        x *= sigma
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = torch.randperm(K, generator=g, device=device)[:n_out]
        x[:, cols] *= outlier_factor
    return x


def device_codes(shape, seed: int, device, lo: int = -127, hi: int = 127) -> torch.Tensor:
    """Uniform int8 codes in [lo, hi] drawn on ``device``."""
    g = _device_generator(seed, device)
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int8, device=device)


def device_e4m3_codes(shape, seed: int, device) -> torch.Tensor:
    """E4M3FN code bytes (uint8) drawn on ``device``: random sign, exponent field
    uniform in [4, 11] (magnitudes 2^-3 to 2^4 x 1.875) and mantissa field uniform in
    [0, 7], so every code is finite and the products stay in a moderate range."""
    g = _device_generator(seed, device)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32, device=device)
    expo = torch.randint(4, 12, shape, generator=g, dtype=torch.int32, device=device)
    mant = torch.randint(0, 8, shape, generator=g, dtype=torch.int32, device=device)
    return (sign * 128 + expo * 8 + mant).to(torch.uint8)


def device_scales(n: int, seed: int, device, lo: float = 1e-4, hi: float = 1e-1) -> torch.Tensor:
    """Positive fp32 scales, log-uniform in [lo, hi], drawn on ``device``."""
    g = _device_generator(seed, device)
    u = torch.rand(n, generator=g, dtype=torch.float64, device=device)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).float()


def device_bias_bf16(n: int, seed: int, device) -> torch.Tensor:
    """bf16 bias [n] ~ N(0, 0.01) drawn on ``device``."""
    g = _device_generator(seed, device)
    return (torch.randn(n, generator=g, dtype=torch.float32, device=device) * 0.01).to(torch.bfloat16)
