"""Measurement aids for the benchmark and the design tests -- not part of the
W8A8 path and not part of the library's C ABI (``include/w8a8.h``).

``libw8a8_probe.so`` (built next to this file by ``w8a8_quantized_linear_amd/build.py``)
holds three kernels:

* ``mfma_rate`` -- the rate the matrix cores sustain with register operands and no
  memory traffic (int8 32x32x32 or bf16 32x32x16 MFMAs): the measured-clock
  ceiling the GEMM is set against (``bench.py --mfma-peak``);
* ``fp8_contraction`` -- an E4M3FN x E4M3FN contraction through the fp8 matrix
  instructions, or through exact widening to bf16, for measuring how accurately
  each sums its products;
* ``f64_mfma_layout`` -- the lane layout of the fp64 4x4x4 matrix instruction that
  the quantizer's rotation uses;
* ``stream`` -- the HBM rate of a kernel with the quantizer's traffic (2 bytes read,
  1 byte written per element) and no arithmetic, or of a plain copy: the achievable
  streaming ceiling the quantizer is set against (``bench.py --stream-peak``);
* ``lds`` -- the cost of the GEMM's MFMA operand reads from LDS under different
  placements of the 16-byte chunks of a row (``bench.py --lds-patterns``).
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

import torch

LIB_PATH = Path(__file__).resolve().parent / "libw8a8_probe.so"
if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is not built; run `python w8a8_quantized_linear_amd/build.py`")
_lib = ctypes.CDLL(str(LIB_PATH))
_lib.w8a8_probe_mfma_rate.restype = ctypes.c_int
_lib.w8a8_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
_lib.w8a8_probe_fp8_contraction.restype = ctypes.c_int
_lib.w8a8_probe_fp8_contraction.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
_lib.w8a8_probe_f64_mfma_layout.restype = ctypes.c_int
_lib.w8a8_probe_f64_mfma_layout.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
_lib.w8a8_probe_stream.restype = ctypes.c_int
_lib.w8a8_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
_lib.w8a8_probe_lds.restype = ctypes.c_int
_lib.w8a8_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

FP8_KINDS = {"fp8_32x32x16": 0, "f8f6f4_32x32x64": 1, "fp8_32x32x16_fp32_adds": 2, "bf16_widened": 3}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def mfma_rate(kind: str, iters: int, blocks: int = 1024, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One launch of the rate probe on the current stream: kind "int8" or "bf16".
    Returns the int32 sink [blocks * 256] (each lane's accumulator sum)."""
    k = {"int8": 0, "bf16": 1}[kind]
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    if sink.dtype != torch.int32 or not sink.is_cuda or not sink.is_contiguous() or sink.numel() < blocks * 256:
        raise ValueError("sink: a contiguous int32 device tensor of blocks * 256 elements")
    if _lib.w8a8_probe_mfma_rate(k, iters, blocks, sink.data_ptr(), _stream()) != 0:
        raise RuntimeError("w8a8_probe_mfma_rate: bad argument or launch failure")
    return sink


def fp8_contraction(kind: str, a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """C fp32 [M, N] = dec(a) . dec(b)^T for E4M3FN codes a [M, K], b [N, K] (uint8,
    contiguous, on the device; M, N multiples of 32, K of 64) through the route
    ``kind`` (a key of FP8_KINDS)."""
    for t, name in ((a, "a"), (b, "b")):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: a contiguous 2-D uint8 device tensor")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if _lib.w8a8_probe_fp8_contraction(FP8_KINDS[kind], a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K,
                                       _stream()) != 0:
        raise RuntimeError("w8a8_probe_fp8_contraction: unsupported shape or launch failure")
    return c


def f64_mfma_layout() -> torch.Tensor:
    """D [64 launches, 64 lanes] of v_mfma_f64_4x4x4f64 with A one-hot at lane L in
    launch L, B = lane + 1, C = 0 (fp64, on the device)."""
    out = torch.zeros((64, 64), dtype=torch.float64, device="cuda")
    if _lib.w8a8_probe_f64_mfma_layout(out.data_ptr(), _stream()) != 0:
        raise RuntimeError("w8a8_probe_f64_mfma_layout: launch failure")
    return out


STREAM_KINDS = {"bf16_to_byte": 0, "copy": 1}


def stream(kind: str, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """One launch of the streaming probe on the current stream.  x: contiguous bf16
    device tensor whose element count is a multiple of 8; y: contiguous device tensor
    of at least numel(x) bytes ("bf16_to_byte": the high byte of each element) or
    2 * numel(x) bytes ("copy")."""
    k = STREAM_KINDS[kind]
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.numel() % 8 != 0 or x.numel() == 0:
        raise ValueError("x: a contiguous bf16 device tensor, a positive multiple of 8 elements")
    need = x.numel() * (1 if k == 0 else 2)
    if not y.is_cuda or not y.is_contiguous() or y.numel() * y.element_size() < need or y.device != x.device:
        raise ValueError(f"y: a contiguous device tensor of at least {need} bytes on x's device")
    if _lib.w8a8_probe_stream(k, x.data_ptr(), y.data_ptr(), x.numel() // 8, _stream()) != 0:
        raise RuntimeError("w8a8_probe_stream: bad argument or launch failure")
    return y


LDS_PATTERNS = {"contiguous": 0, "rows_no_swizzle": 1, "rows_earlier_key": 2, "rows_gemm_key": 3}


def lds(pattern: str, iters: int, blocks: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One launch of the LDS read-pattern probe on the current stream (pattern: a key
    of LDS_PATTERNS).  Returns the int32 [blocks * 256] lane sums."""
    k = LDS_PATTERNS[pattern]
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    if out.dtype != torch.int32 or not out.is_cuda or not out.is_contiguous() or out.numel() < blocks * 256:
        raise ValueError("out: a contiguous int32 device tensor of blocks * 256 elements")
    if _lib.w8a8_probe_lds(k, iters, blocks, out.data_ptr(), _stream()) != 0:
        raise RuntimeError("w8a8_probe_lds: bad argument or launch failure")
    return out


def lds_expected(pattern: str, iters: int) -> list:
    """Host-side value of each of the 256 lane sums of one block (the same in every
    block): iters times the sum of the dword indices the lane reads, mod 2^32, as a
    signed int32."""
    k = LDS_PATTERNS[pattern]

    def key(r):
        return {2: ((r >> 1) ^ (r >> 3)) & 3, 3: (r ^ (r >> 2)) & 3}.get(k, 0)
    sums = []
    for tid in range(256):
        lane, wave = tid & 63, tid >> 6
        total = 0
        for t in range(8):
            if k == 0:
                off = (t * 1024 + lane * 16) % 16384
            else:
                row = (wave * 64 + t * 32 + (lane & 31)) % 256
                c = 2 * (t & 1) + (lane >> 5)
                off = (row * 4 + (c ^ key(row))) * 16
            total += sum(off // 4 + d for d in range(4))
        v = (total * iters) % (1 << 32)
        sums.append(v - (1 << 32) if v >= 1 << 31 else v)
    return sums
