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
    "w8a8_swiglu", "swiglu_quant_workspace_bytes", "w8a8_gateup_swiglu_quant_packed",
    "w8a8_gemm_i32_packed", "swiglu_quant_h", "w8a8_linear_packed_noalloc", "NOALLOC_MAX_WORKSPACE",
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
    "w8a8_gemm_i32_packed": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
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
    "w8a8_swiglu_quant_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w8a8_linear_packed_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "w8a8_gateup_swiglu_quant_packed": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, _P, _P, _SZ, _P]),
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


def _device_ok(t: torch.Tensor, name: str) -> None:
    """The library runs on the current HIP device and torch's current stream there."""
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _want(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    _device_ok(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _out(t: Optional[torch.Tensor], dtype: torch.dtype, numel: int, name: str, dev: torch.device,
         shape=None) -> torch.Tensor:
    """A caller-supplied output (checked: dtype, device, contiguity, at least `numel`
    elements, and `shape` when given), or a new tensor of `shape` (or `numel`
    elements, at least one)."""
    if t is None:
        return torch.empty(shape if shape is not None else (max(numel, 1),), dtype=dtype, device=dev)
    _want(t, dtype, name, t.dim())
    if t.device != dev:
        raise ValueError(f"{name}: is on {t.device}, the inputs on {dev}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")
    return t


def _workspace(t: Optional[torch.Tensor], need: int, dev: torch.device) -> torch.Tensor:
    """Caller-supplied workspace (a contiguous device tensor of at least `need` bytes,
    any dtype) or a new uint8 one."""
    if t is None:
        return torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if not isinstance(t, torch.Tensor):
        raise TypeError("workspace: expected a torch.Tensor")
    _device_ok(t, "workspace")
    if t.device != dev:
        raise ValueError(f"workspace: is on {t.device}, the inputs on {dev}")
    if not t.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace: needs {need} bytes, has {t.numel() * t.element_size()}")
    return t


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
    wp = _out(out, w.dtype, n, "out", w.device)
    _check(_lib.w8a8_pack_weight(_ptr(w), rows, K, _ptr(wp), _stream()), "w8a8_pack_weight")
    return wp


# ---------------------------------------------------------------- stage 1 ----
def w8a8_quantize_act(x: torch.Tensor, rot_block: int = 0,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Per-row int8 quantizer: x bf16 [M, K] -> (q int8 [M, K], s fp32 [M])."""
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, torch.int8, M * K, "q", x.device, shape=(M, K))
    s = _out(s0, torch.float32, M, "s", x.device, shape=(M,))
    _check(_lib.w8a8_quantize_act(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), _stream()),
           "w8a8_quantize_act")
    return q, s


def w8a8_quantize_act_fp8(x: torch.Tensor, rot_block: int = 0,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Per-row E4M3FN quantizer: x bf16 [M, K] -> (codes uint8 [M, K], s fp32 [M])."""
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, torch.uint8, M * K, "q", x.device, shape=(M, K))
    s = _out(s0, torch.float32, M, "s", x.device, shape=(M,))
    _check(_lib.w8a8_quantize_act_fp8(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), _stream()),
           "w8a8_quantize_act_fp8")
    return q, s


def _quant_packed(fname, x, rot_block, qdtype, out):
    _want(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    n = packed_bytes(M, K)
    q0, s0 = out if out is not None else (None, None)
    q = _out(q0, qdtype, n, "q", x.device)
    s = _out(s0, torch.float32, M, "s", x.device, shape=(M,))
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
    acc = _out(out, torch.int32, M * N, "out", q.device, shape=(M, N))
    _check(_lib.w8a8_gemm_i32(_ptr(q), _ptr(w), _ptr(acc), M, N, K, _stream()), "w8a8_gemm_i32")
    return acc


def w8a8_gemm_i32_packed(q_packed: torch.Tensor, w_packed: torch.Tensor, M: int, N: int, K: int,
                         out: Optional[torch.Tensor] = None):
    """acc int32 [M, N] from packed int8 codes (q_packed of M rows, w_packed of N rows):
    the accumulators of the packed GEMM that the whole paths run."""
    _want(q_packed, torch.int8, "q_packed", 1)
    _want(w_packed, torch.int8, "w_packed", 1)
    if q_packed.numel() < packed_bytes(M, K) or w_packed.numel() < packed_bytes(N, K):
        raise ValueError("packed operands smaller than packed_bytes(rows, K)")
    acc = _out(out, torch.int32, M * N, "out", q_packed.device, shape=(M, N))
    _check(_lib.w8a8_gemm_i32_packed(_ptr(q_packed), _ptr(w_packed), _ptr(acc), M, N, K, _stream()),
           "w8a8_gemm_i32_packed")
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
    y = _out(out, torch.bfloat16, M * n_out, "out", q.device, shape=(M, n_out))
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
    y = _out(out, torch.bfloat16, M * n_out, "out", q.device, shape=(M, n_out))
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
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{name}: expected a 2-D bf16 device tensor")
        _device_ok(t, name)
        if t.stride(1) != 1:
            raise ValueError(f"{name}: rows must be contiguous")
    if gate.shape != up.shape or gate.stride(0) != up.stride(0):
        raise ValueError("gate and up must have the same shape and row stride")
    M, N = gate.shape
    if gate.device != up.device:
        raise ValueError("gate and up must be on the same device")
    y = _out(out, torch.bfloat16, M * N, "out", gate.device, shape=(M, N))
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
    ws = _workspace(workspace, workspace_bytes(M, K), x.device)
    y = _out(out, torch.bfloat16, M * n_out, "out", x.device, shape=(M, n_out))
    _check(getattr(_lib, fname)(_ptr(x), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y), M, n_out, K,
                                rot_block, _ptr(ws), ws.numel() * ws.element_size(), _stream()), fname)
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


# Bytes of the library's fixed scratch array (W8A8_NOALLOC_MAX_WORKSPACE in w8a8.h).
NOALLOC_MAX_WORKSPACE = 64 << 20


def w8a8_linear_packed_noalloc(x, w_packed, N, s_ch, bias=None, rot_block=0, out=None):
    """w8a8_linear_packed with no workspace: the C entry point keeps the quantized
    activations in the library's fixed per-device scratch array and allocates nothing
    (y is allocated here only when `out` is not given).  Calls that overlap in time on
    one device race; workspace_bytes(M, K) must not exceed NOALLOC_MAX_WORKSPACE."""
    _want(x, torch.bfloat16, "x", 2)
    _want(w_packed, torch.int8, "w_packed", 1)
    _want(s_ch, torch.float32, "s_ch", 1)
    if bias is not None:
        _want(bias, torch.bfloat16, "bias", 1)
    M, K = x.shape
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("packed weight is smaller than packed_bytes(N, K)")
    if s_ch.shape[0] != N or (bias is not None and bias.shape[0] != N):
        raise ValueError("s_ch and bias lengths must equal N")
    y = _out(out, torch.bfloat16, M * N, "out", x.device, shape=(M, N))
    _check(_lib.w8a8_linear_packed_noalloc(_ptr(x), _ptr(w_packed), _ptr(s_ch), _ptr(bias), _ptr(y), M, N, K,
                                           rot_block, _stream()), "w8a8_linear_packed_noalloc")
    return y


# ------------------------ gate/up SwiGLU quantized for the next linear -------
def swiglu_quant_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.w8a8_swiglu_quant_workspace_bytes(M, N, K))


def swiglu_quant_h(workspace: torch.Tensor, M: int, N: int, K: int) -> torch.Tensor:
    """The bf16 SwiGLU output h [M, N] that w8a8_gateup_swiglu_quant_packed leaves in its
    workspace (a view; the workspace layout is fixed by the C header)."""
    off = workspace_bytes(M, K)
    raw = workspace.view(torch.uint8).reshape(-1)[off:off + 2 * M * N]
    return raw.view(torch.bfloat16).view(M, N)


def w8a8_gateup_swiglu_quant_packed(x, w_gateup_packed, N, s_ch, bias=None, rot_in=0, rot_out=0,
                                    workspace=None, q_out=None, s_out=None):
    """Returns (packed int8 codes [packed_bytes(M, N)], s_tok fp32 [M]): the per-token
    quantization (rotation rot_out) of the bf16 gate/up SwiGLU output, ready as the A
    operand of w8a8_gemm_dequant_packed for the down projection (K = N)."""
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
    ws = _workspace(workspace, swiglu_quant_workspace_bytes(M, N, K), dev)
    q = _out(q_out, torch.int8, packed_bytes(M, N), "q_out", dev)
    s = _out(s_out, torch.float32, M, "s_out", dev, shape=(M,))
    _check(_lib.w8a8_gateup_swiglu_quant_packed(_ptr(x), _ptr(w_gateup_packed), _ptr(s_ch), _ptr(bias), M, N,
                                                K, rot_in, rot_out, _ptr(q), _ptr(s), _ptr(ws),
                                                ws.numel() * ws.element_size(), _stream()),
           "w8a8_gateup_swiglu_quant_packed")
    return q, s
