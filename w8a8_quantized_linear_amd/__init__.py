"""Python binding of the MI355X W8A8 quantized projection library (``libw8a8.so``).

The functions below carry the names of the C entry points declared in
``include/w8a8.h`` and only marshal arguments: they check dtypes/devices,
allocate outputs as torch tensors on the current device, pass raw device
pointers plus ``torch.cuda.current_stream()`` to the C call and turn a non-OK
status into an exception.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  Importing this package without the built
library raises immediately.

Conventions: bf16 tensors are ``torch.bfloat16``; int8 codes ``torch.int8``;
E4M3FN codes ``torch.uint8`` (raw codes; view as ``torch.float8_e4m3fn`` if
desired); scales ``torch.float32``.  All tensors are contiguous, 16-byte
aligned and on the current CUDA (HIP) device.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "W8A8Error", "workspace_bytes", "packed_bytes", "unpack_rows",
    "w8a8_pack_weight", "w8a8_quantize_act", "w8a8_quantize_act_fp8", "w8a8_gemm_i32",
    "w8a8_gemm_dequant", "w8a8_gemm_swiglu", "w8a8_fp8_gemm_dequant", "w8a8_linear",
    "w8a8_gateup_swiglu", "w8a8_fp8_linear", "w8a8_linear_packed", "w8a8_gateup_swiglu_packed",
    "w8a8_fp8_linear_packed", "w8a8_quantize_act_packed", "w8a8_quantize_act_fp8_packed",
    "w8a8_gemm_dequant_packed", "w8a8_gemm_swiglu_packed", "w8a8_fp8_gemm_dequant_packed",
    "w8a8_swiglu", "block_amax_bytes", "swiglu_quant_workspace_bytes",
    "w8a8_gemm_swiglu_blockquant_packed", "w8a8_requantize_blocks_packed",
    "w8a8_gateup_swiglu_quant_packed",
]

LIB_PATH = Path(__file__).resolve().parent / "libw8a8.so"
if not LIB_PATH.exists():
    raise ImportError(
        f"{LIB_PATH} is not built; run `python w8a8_quantized_linear_amd/build.py` "
        "(hipcc, gfx950) first -- there is no non-HIP fallback")

_lib = ctypes.CDLL(str(LIB_PATH))
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "w8a8_status_string": (ctypes.c_char_p, [_I]),
    "w8a8_workspace_bytes": (_SZ, [_I64, _I64]),
    "w8a8_packed_bytes": (_SZ, [_I64, _I64]),
    "w8a8_pack_weight": (_I, [_P, _I64, _I64, _P, _P]),
    "w8a8_quantize_act": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "w8a8_quantize_act_fp8": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "w8a8_gemm_i32": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_gemm_dequant": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_gemm_swiglu": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_fp8_gemm_dequant": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_linear": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_gateup_swiglu": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_fp8_linear": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_quantize_act_packed": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "w8a8_quantize_act_fp8_packed": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "w8a8_gemm_dequant_packed": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_gemm_swiglu_packed": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_fp8_gemm_dequant_packed": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_swiglu": (_I, [_P, _P, _I64, _P, _I64, _I64, _P]),
    "w8a8_linear_packed": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_gateup_swiglu_packed": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_fp8_linear_packed": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "w8a8_block_amax_bytes": (_SZ, [_I64, _I64]),
    "w8a8_swiglu_quant_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w8a8_gemm_swiglu_blockquant_packed": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P, _P]),
    "w8a8_requantize_blocks_packed": (_I, [_P, _P, _I64, _I64, _P, _P]),
    "w8a8_gateup_swiglu_quant_packed": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, _P, _P, _SZ, _P]),
    "w8a8_mfma_probe": (_I, [_I, _I64, _I, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class W8A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.w8a8_status_string(status).decode()} (status {status})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise W8A8Error(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _want(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def workspace_bytes(M: int, K: int) -> int:
    return int(_lib.w8a8_workspace_bytes(M, K))


def packed_bytes(rows: int, K: int) -> int:
    return int(_lib.w8a8_packed_bytes(rows, K))


def unpack_rows(packed: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """View-and-copy inverse of the packed layout (32-row x 64-byte blocks) for
    inspection: a flat byte tensor holding at least packed_bytes(rows, K) bytes
    -> [rows, K] in row-major order, same dtype and device."""
    n = packed_bytes(rows, K)
    blocks = packed.reshape(-1)[:n].reshape(-1, K // 64, 32, 64)   # [row block, k block, row, byte]
    return blocks.permute(0, 2, 1, 3).reshape(-1, K)[:rows].contiguous()


def w8a8_pack_weight(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row-major one-byte codes w [rows, K] (int8 or uint8) -> flat packed copy
    (packed_bytes(rows, K) elements of w's dtype)."""
    if w.dtype not in (torch.int8, torch.uint8):
        raise TypeError(f"w: expected int8 or uint8 codes, got {w.dtype}")
    _want(w, w.dtype, "w", 2)
    rows, K = w.shape
    n = packed_bytes(rows, K)
    wp = out if out is not None else torch.empty((max(n, 1),), dtype=w.dtype, device=w.device)
    if wp.numel() < n:
        raise ValueError("out is smaller than packed_bytes(rows, K)")
    _check(_lib.w8a8_pack_weight(_ptr(w), rows, K, _ptr(wp), _stream()), "w8a8_pack_weight")
    return wp


# ---------------------------------------------------------------- stage 1 ----
def w8a8_quantize_act(x: torch.Tensor, rot_block: int = 0,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Per-row int8 quantizer: x bf16 [M, K] -> (q int8 [M, K], s fp32 [M])."""
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    q, s = out if out is not None else (torch.empty((M, K), dtype=torch.int8, device=x.device),
                                        torch.empty((M,), dtype=torch.float32, device=x.device))
    _check(_lib.w8a8_quantize_act(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), _stream()),
           "w8a8_quantize_act")
    return q, s


def w8a8_quantize_act_fp8(x: torch.Tensor, rot_block: int = 0,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Per-row E4M3FN quantizer: x bf16 [M, K] -> (codes uint8 [M, K], s fp32 [M])."""
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    q, s = out if out is not None else (torch.empty((M, K), dtype=torch.uint8, device=x.device),
                                        torch.empty((M,), dtype=torch.float32, device=x.device))
    _check(_lib.w8a8_quantize_act_fp8(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), _stream()),
           "w8a8_quantize_act_fp8")
    return q, s


def _quant_packed(fname, x, rot_block, qdtype, out):
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    n = packed_bytes(M, K)
    q, s = out if out is not None else (torch.empty((max(n, 1),), dtype=qdtype, device=x.device),
                                        torch.empty((M,), dtype=torch.float32, device=x.device))
    if q.numel() < n:
        raise ValueError("q is smaller than packed_bytes(M, K)")
    _check(getattr(_lib, fname)(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), _stream()), fname)
    return q, s


def w8a8_quantize_act_packed(x: torch.Tensor, rot_block: int = 0, out=None):
    """Per-row int8 quantizer writing the packed layout: (q int8 flat, s fp32 [M])."""
    return _quant_packed("w8a8_quantize_act_packed", x, rot_block, torch.int8, out)


def w8a8_quantize_act_fp8_packed(x: torch.Tensor, rot_block: int = 0, out=None):
    """Per-row E4M3FN quantizer writing the packed layout: (codes uint8 flat, s fp32 [M])."""
    return _quant_packed("w8a8_quantize_act_fp8_packed", x, rot_block, torch.uint8, out)


# ------------------------------------------------------------ stages 2, 3 ----
def w8a8_gemm_i32(q: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None):
    """acc int32 [M, N] = q int8 [M, K] . w int8 [N, K]^T (exact)."""
    _want(q, torch.int8, "q", 2)
    _want(w, torch.int8, "w", 2)
    M, K = q.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("q and w disagree on K")
    acc = out if out is not None else torch.empty((M, N), dtype=torch.int32, device=q.device)
    _check(_lib.w8a8_gemm_i32(_ptr(q), _ptr(w), _ptr(acc), M, N, K, _stream()), "w8a8_gemm_i32")
    return acc


def _epi(fname, q, s_tok, w, s_ch, bias, n_out, qdtype, out):
    _want(q, qdtype, "q", 2)
    _want(w, qdtype, "w", 2)
    _want(s_tok, torch.float32, "s_tok", 1)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    M, K = q.shape
    if w.shape[1] != K or s_tok.shape[0] != M or s_ch.shape[0] != w.shape[0]:
        raise ValueError("inconsistent shapes")
    if bias is not None and bias.shape[0] != w.shape[0]:
        raise ValueError("bias length must equal the weight's rows")
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=q.device)
    _check(getattr(_lib, fname)(_ptr(q), _ptr(s_tok), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y),
                                M, n_out, K, _stream()), fname)
    return y


def w8a8_gemm_dequant(q, s_tok, w, s_ch, bias=None, out=None):
    """y bf16 [M, N] = (q . w^T) * s_tok * s_ch + bias, from int8 codes."""
    return _epi("w8a8_gemm_dequant", q, s_tok, w, s_ch, bias, w.shape[0], torch.int8, out)


def w8a8_gemm_swiglu(q, s_tok, w_gateup, s_ch, bias=None, out=None):
    """y bf16 [M, N] = silu(gate) * up over the packed [2N, K] int8 weight."""
    if w_gateup.shape[0] % 2:
        raise ValueError("packed gate/up weight needs an even number of rows")
    return _epi("w8a8_gemm_swiglu", q, s_tok, w_gateup, s_ch, bias, w_gateup.shape[0] // 2,
                torch.int8, out)


def w8a8_fp8_gemm_dequant(q, s_tok, w, s_ch, bias=None, out=None):
    """y bf16 [M, N] from E4M3FN codes (uint8) with fp32 accumulation."""
    return _epi("w8a8_fp8_gemm_dequant", q, s_tok, w, s_ch, bias, w.shape[0], torch.uint8, out)


def _epi_packed(fname, q, s_tok, w, s_ch, bias, M, n_out, K, qdtype, out):
    _want(q, qdtype, "q", 1)
    _want(w, qdtype, "w", 1)
    _want(s_tok, torch.float32, "s_tok", 1)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    rows = s_ch.shape[0]
    if s_tok.shape[0] != M or q.numel() < packed_bytes(M, K) or w.numel() < packed_bytes(rows, K):
        raise ValueError("inconsistent shapes")
    if bias is not None and bias.shape[0] != rows:
        raise ValueError("bias length must equal the weight's rows")
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=q.device)
    _check(getattr(_lib, fname)(_ptr(q), _ptr(s_tok), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y),
                                M, n_out, K, _stream()), fname)
    return y


def w8a8_gemm_dequant_packed(q_packed, s_tok, w_packed, s_ch, K, bias=None, out=None):
    """w8a8_gemm_dequant on packed operands; M = len(s_tok), N = len(s_ch)."""
    return _epi_packed("w8a8_gemm_dequant_packed", q_packed, s_tok, w_packed, s_ch, bias,
                       s_tok.shape[0], s_ch.shape[0], K, torch.int8, out)


def w8a8_gemm_swiglu_packed(q_packed, s_tok, w_gateup_packed, s_ch, K, bias=None, out=None):
    """w8a8_gemm_swiglu on packed operands; M = len(s_tok), N = len(s_ch) / 2."""
    return _epi_packed("w8a8_gemm_swiglu_packed", q_packed, s_tok, w_gateup_packed, s_ch, bias,
                       s_tok.shape[0], s_ch.shape[0] // 2, K, torch.int8, out)


def w8a8_fp8_gemm_dequant_packed(q_packed, s_tok, w_packed, s_ch, K, bias=None, out=None):
    """w8a8_fp8_gemm_dequant on packed operands; M = len(s_tok), N = len(s_ch)."""
    return _epi_packed("w8a8_fp8_gemm_dequant_packed", q_packed, s_tok, w_packed, s_ch, bias,
                       s_tok.shape[0], s_ch.shape[0], K, torch.uint8, out)


# ------------------------------------------------- unfused gate/up SwiGLU ----
def w8a8_swiglu(gate: torch.Tensor, up: torch.Tensor, out: Optional[torch.Tensor] = None):
    """y bf16 [M, N] = silu(gate) * up for bf16 [M, N] views with the same row stride
    (e.g. the two halves of a [M, 2N] projection: h[:, :N], h[:, N:])."""
    for t, name in ((gate, "gate"), (up, "up")):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_cuda:
            raise ValueError(f"{name}: expected a 2-D bf16 device tensor")
        if t.stride(1) != 1:
            raise ValueError(f"{name}: rows must be contiguous")
    if gate.shape != up.shape or gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must have the same shape and row stride")
    M, N = gate.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=gate.device)
    _check(_lib.w8a8_swiglu(_ptr(gate), _ptr(up), gate.stride(0), _ptr(y), M, N, _stream()),
           "w8a8_swiglu")
    return y


# ------------------------------------------------------------ whole paths ----
def _path(fname, x, w, s_ch, bias, rot_block, n_out, wdtype, workspace, out, w_rows=None):
    """w_rows is None for a row-major weight [rows, K]; for a packed weight (flat)
    it is the weight's row count."""
    _want(x, torch.bfloat16, "x", 2)
    _want(w, wdtype, "w", 1 if w_rows is not None else 2)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    M, K = x.shape
    rows = w.shape[0] if w_rows is None else w_rows
    if w_rows is None and w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    if w_rows is not None and w.numel() < packed_bytes(w_rows, K):
        raise ValueError("packed weight is smaller than packed_bytes(rows, K)")
    if s_ch.shape[0] != rows:
        raise ValueError("s_ch length must equal the weight's rows")
    if bias is not None and bias.shape[0] != rows:
        raise ValueError("bias length must equal the weight's rows")
    need = workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.bfloat16, device=x.device)
    _check(getattr(_lib, fname)(_ptr(x), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y), M, n_out, K,
                                rot_block, _ptr(workspace), workspace.numel(), _stream()), fname)
    return y


def w8a8_linear(x, w, s_ch, bias=None, rot_block=0, workspace=None, out=None):
    """y bf16 [M, N]: per-token int8 quantization of x (optionally rotated), int8 GEMM, dequant."""
    return _path("w8a8_linear", x, w, s_ch, bias, rot_block, w.shape[0], torch.int8, workspace, out)


def w8a8_gateup_swiglu(x, w_gateup, s_ch, bias=None, rot_block=0, workspace=None, out=None):
    """y bf16 [M, N]: quantize x, int8 GEMM against the packed [2N, K] gate/up weight, SwiGLU."""
    return _path("w8a8_gateup_swiglu", x, w_gateup, s_ch, bias, rot_block, w_gateup.shape[0] // 2,
                 torch.int8, workspace, out)


def w8a8_fp8_linear(x, w, s_ch, bias=None, rot_block=0, workspace=None, out=None):
    """y bf16 [M, N]: per-token E4M3FN quantization of x, fp8 GEMM, dequant."""
    return _path("w8a8_fp8_linear", x, w, s_ch, bias, rot_block, w.shape[0], torch.uint8, workspace, out)


def w8a8_linear_packed(x, w_packed, N, s_ch, bias=None, rot_block=0, workspace=None, out=None):
    """w8a8_linear with the weight [N, K] given in the packed layout (w8a8_pack_weight)."""
    return _path("w8a8_linear_packed", x, w_packed, s_ch, bias, rot_block, N, torch.int8, workspace,
                 out, w_rows=N)


def w8a8_gateup_swiglu_packed(x, w_gateup_packed, N, s_ch, bias=None, rot_block=0, workspace=None,
                              out=None):
    """w8a8_gateup_swiglu with the [2N, K] gate/up weight given in the packed layout."""
    return _path("w8a8_gateup_swiglu_packed", x, w_gateup_packed, s_ch, bias, rot_block, N, torch.int8,
                 workspace, out, w_rows=2 * N)


def w8a8_fp8_linear_packed(x, w_packed, N, s_ch, bias=None, rot_block=0, workspace=None, out=None):
    """w8a8_fp8_linear with the E4M3FN weight [N, K] given in the packed layout."""
    return _path("w8a8_fp8_linear_packed", x, w_packed, s_ch, bias, rot_block, N, torch.uint8,
                 workspace, out, w_rows=N)


# ------------------------ gate/up SwiGLU quantized for the next linear -------
def block_amax_bytes(M: int, N: int) -> int:
    return int(_lib.w8a8_block_amax_bytes(M, N))


def swiglu_quant_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.w8a8_swiglu_quant_workspace_bytes(M, N, K))


def w8a8_gemm_swiglu_blockquant_packed(q_packed, s_tok, w_gateup_packed, s_ch, K, bias=None,
                                       rot_out=0, want_h=False, codes=None, amax=None):
    """First step: returns (block codes, flat packed int8 [packed_bytes(M, N)];
    block amax fp32 [M, ceil(N / 128)]; h bf16 [M, N] or None).  M = len(s_tok),
    N = len(s_ch) / 2."""
    _want(q_packed, torch.int8, "q_packed", 1)
    _want(w_gateup_packed, torch.int8, "w_gateup_packed", 1)
    _want(s_tok, torch.float32, "s_tok", 1)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    M, rows = s_tok.shape[0], s_ch.shape[0]
    N = rows // 2
    if q_packed.numel() < packed_bytes(M, K) or w_gateup_packed.numel() < packed_bytes(rows, K):
        raise ValueError("inconsistent shapes")
    if bias is not None and bias.shape[0] != rows:
        raise ValueError("bias length must equal the weight's rows")
    dev = q_packed.device
    nblk = (N + 127) // 128
    codes = codes if codes is not None else torch.empty((max(packed_bytes(M, N), 1),), dtype=torch.int8, device=dev)
    amax = amax if amax is not None else torch.empty((M, nblk), dtype=torch.float32, device=dev)
    if codes.numel() < packed_bytes(M, N) or amax.numel() < M * nblk:
        raise ValueError("codes or amax too small")
    h = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if want_h else None
    _check(_lib.w8a8_gemm_swiglu_blockquant_packed(_ptr(q_packed), _ptr(s_tok), _ptr(w_gateup_packed),
                                                   _ptr(s_ch), _ptr(bias), M, N, K, rot_out, _ptr(codes),
                                                   _ptr(amax), _ptr(h), _stream()),
           "w8a8_gemm_swiglu_blockquant_packed")
    return codes, amax, h


def w8a8_requantize_blocks_packed(codes, amax, M, N, s_tok=None):
    """Second step, in place on `codes` (flat packed int8): returns s_tok fp32 [M]."""
    _want(codes, torch.int8, "codes", 1)
    _want(amax, torch.float32, "amax", 2)
    if codes.numel() < packed_bytes(M, N) or tuple(amax.shape) != (M, (N + 127) // 128):
        raise ValueError("inconsistent shapes")
    s = s_tok if s_tok is not None else torch.empty((M,), dtype=torch.float32, device=codes.device)
    _check(_lib.w8a8_requantize_blocks_packed(_ptr(codes), _ptr(amax), M, N, _ptr(s), _stream()),
           "w8a8_requantize_blocks_packed")
    return s


def w8a8_gateup_swiglu_quant_packed(x, w_gateup_packed, N, s_ch, bias=None, rot_in=0, rot_out=0,
                                    workspace=None, q_out=None, s_out=None):
    """Whole: returns (packed int8 codes [packed_bytes(M, N)], s_tok fp32 [M]) of the
    SwiGLU output, ready as the A operand of w8a8_gemm_dequant_packed (K = N)."""
    _want(x, torch.bfloat16, "x", 2)
    _want(w_gateup_packed, torch.int8, "w_gateup_packed", 1)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    M, K = x.shape
    if w_gateup_packed.numel() < packed_bytes(2 * N, K) or s_ch.shape[0] != 2 * N:
        raise ValueError("inconsistent shapes")
    if bias is not None and bias.shape[0] != 2 * N:
        raise ValueError("bias length must equal the weight's rows")
    dev = x.device
    need = swiglu_quant_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    q = q_out if q_out is not None else torch.empty((max(packed_bytes(M, N), 1),), dtype=torch.int8, device=dev)
    s = s_out if s_out is not None else torch.empty((M,), dtype=torch.float32, device=dev)
    if q.numel() < packed_bytes(M, N):
        raise ValueError("q_out too small")
    _check(_lib.w8a8_gateup_swiglu_quant_packed(_ptr(x), _ptr(w_gateup_packed), _ptr(s_ch), _ptr(bias), M, N,
                                                K, rot_in, rot_out, _ptr(q), _ptr(s), _ptr(workspace),
                                                workspace.numel(), _stream()),
           "w8a8_gateup_swiglu_quant_packed")
    return q, s


# ------------------------------------------------------- measurement aid ----
def w8a8_mfma_probe(kind: str, iters: int, blocks: int = 1024, sink: Optional[torch.Tensor] = None):
    """MFMA-only rate probe (not a step of the path): kind "int8" (32x32x32) or "bf16"
    (32x32x16).  Enqueues one launch on the current stream and returns the int32 sink
    [blocks * 256] (each lane's accumulator sum)."""
    k = {"int8": 0, "bf16": 1}[kind]
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    _want(sink, torch.int32, "sink", 1)
    if sink.numel() < blocks * 256:
        raise ValueError("sink: needs blocks * 256 elements")
    _check(_lib.w8a8_mfma_probe(k, iters, blocks, _ptr(sink), _stream()), "w8a8_mfma_probe")
    return sink
