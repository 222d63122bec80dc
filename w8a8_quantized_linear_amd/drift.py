"""Quantization-drift diagnostics: how far the W8A8 projection lands from the
unquantized one, with and without the block rotation.

The Calibrated INT8 card's evaluation table reports drift as the relative L2
distance of the quantized model's outputs from the BF16 model's.  Here the same
measure is taken for one projection: ||y_q - y||_2 / ||y||_2, where y_q is this
library's output (quantizer + integer GEMM + epilogue on the GPU, the weight
quantized per output channel with the same rotation setting) and y is the
unquantized projection of the same bf16 inputs evaluated in fp64 on the host
(x W^T + b; for gate/up, silu(g) u of the unquantized g and u).  Rotation by an
orthonormal matrix leaves y unchanged, so every rotation setting is measured
against the same reference.  The fp64 reference is computed for a subset of
token rows (rows are independent), which keeps it cheap at any size.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np
import torch

from . import (w8a8_fp8_linear, w8a8_gateup_swiglu, w8a8_linear, w8a8_quantize_act,
               w8a8_quantize_act_fp8)


def _reference(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], kind: str) -> np.ndarray:
    xf = x.double().cpu().numpy()
    wf = w.double().cpu().numpy()
    y = xf @ wf.T
    if bias is not None:
        y = y + bias.double().cpu().numpy()[None, :]
    if kind == "gateup":
        n = w.shape[0] // 2
        g, u = y[:, :n], y[:, n:]
        y = g / (1.0 + np.exp(-g)) * u
    return y


def relative_l2(y_q: np.ndarray, y: np.ndarray) -> float:
    """||y_q - y||_2 / ||y||_2 over all elements."""
    return float(np.linalg.norm(y_q - y) / np.linalg.norm(y))


def drift(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, kind: str = "linear",
          rot_blocks: Iterable[int] = (0, 128), rows: Optional[Sequence[int]] = None) -> Dict[int, float]:
    """Relative L2 drift of the W8A8 path for each rotation setting.

    x: bf16 [M, K], w: bf16 [N_w, K] (the packed [2N, K] gate/up matrix for
    kind == "gateup"), bias: bf16 [N_w] or None; kind is "linear", "gateup" or
    "fp8".  Device tensors are used as they are; host tensors are copied to the
    current device.  rows selects the token rows that are compared (all rows if
    None); the GPU path always runs on the whole batch."""
    dev = torch.device("cuda")
    xd, wd = x.to(dev), w.to(dev)
    bd = None if bias is None else bias.to(dev)
    sel = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    ref = _reference(x[torch.as_tensor(sel)].cpu(), w.cpu(), None if bias is None else bias.cpu(), kind)
    out = {}
    for rot in rot_blocks:
        if kind == "fp8":
            wq, s_ch = w8a8_quantize_act_fp8(wd, rot)
            y = w8a8_fp8_linear(xd, wq, s_ch, bd, rot_block=rot)
        else:
            wq, s_ch = w8a8_quantize_act(wd, rot)
            fn = w8a8_gateup_swiglu if kind == "gateup" else w8a8_linear
            y = fn(xd, wq, s_ch, bd, rot_block=rot)
        torch.cuda.synchronize()
        out[rot] = relative_l2(y[torch.as_tensor(sel, device=dev)].double().cpu().numpy(), ref)
    return out
