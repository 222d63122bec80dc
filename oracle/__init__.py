"""CPU oracle for the W8A8 quantized decoder projection (TEST INFRASTRUCTURE).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``w8a8_oracle.cpp`` (plain C++17 loops, fp64 / int64);
this module only builds it with g++ and marshals numpy arrays through ctypes.
Every array argument is a C-contiguous numpy array; bf16 is carried as its
raw ``uint16`` bit pattern and E4M3FN as ``uint8`` codes.

What each call follows (pages on quantized Clef checkpoints):

* ``quantize_i8`` / ``quantize_fp8`` -- the per-token dynamic activation
  quantizer ("CLEF Calibrated INT8 ConvRot" card, latency-table notes;
  "clef-flash-FP8" card, Quantization table), also applied to the rows of a
  weight matrix for per-output-channel weight scales (same FP8 card, note
  after recipe.yaml: weight scales come straight from the weights).
* ``rotate`` -- the rotation the ConvRot quantizer applies first (INT8
  ConvRot card); its form is not given on the pages, the reading taken is a
  normalized Sylvester Walsh-Hadamard transform on blocks of 128 along K.
* ``gemm_i32`` / ``gemm_fp8`` -- the integer (fp8) contraction.
* ``gemm_dequant`` / ``gemm_swiglu`` / ``fp8_gemm_dequant`` -- the fused
  scale + bias (+ paired gate/up SwiGLU) epilogue (INT8 ConvRot card,
  Benefits list; "Loading CLEF INT8", fuse_mlp and packed gate/up).
* ``linear`` / ``gateup_swiglu`` / ``fp8_linear`` -- the whole path.
* ``swiglu_bf16`` / ``gateup_unfused`` -- the unfused gate/up path
  ("Loading CLEF INT8", fuse_mlp=False): SwiGLU applied to the separately
  rounded bf16 gate and up projections.
* ``gateup_swiglu_quant`` -- the SwiGLU output handed to the next (down)
  projection as int8 input: the per-token activation quantizer (INT8 ConvRot
  card, latency-table notes) applied to the bf16 output of the paired gate/up
  epilogue, with the next projection's rotation (reading R17 in the C++ header).

No function here carries a "parity unpinned" mark: each is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "w8a8_oracle.cpp"
_LIB_PATH = _HERE / "liboracle.so"

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with g++ (plain -O2, no intrinsics, no BLAS)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", str(_SRC), "-o", str(tmp)]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def default_threads() -> int:
    """Threads for the oracle: the OMP_NUM_THREADS share if set, else all cores, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # W8A8_ORACLE_LIB: a separately built copy (the mutation tests load copies of the
    # oracle with a planted mistake, to show that the pins catch it)
    alt = os.environ.get("W8A8_ORACLE_LIB")
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    sigs = {
        "orc_bf16_decode": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_bf16_from_f64": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_bf16_from_f64_array": (None, [P, I64, P, I]),
        "orc_e4m3_encode_array": (None, [P, I64, P, I]),
        "orc_rotate": (None, [P, I64, I64, I, P, I]),
        "orc_quantize_i8": (None, [P, I64, I64, I, P, P, I]),
        "orc_quantize_fp8": (None, [P, I64, I64, I, P, P, I]),
        "orc_quantize_f32_i8": (None, [P, I64, I64, P, P, I]),
        "orc_quantize_f32_fp8": (None, [P, I64, I64, P, P, I]),
        "orc_gemm_i32": (None, [P, P, I64, I64, I64, P, I]),
        "orc_gemm_fp8": (None, [P, P, I64, I64, I64, P, I]),
        "orc_gemm_dequant": (None, [P, P, P, P, P, P, I64, I64, I64, I]),
        "orc_gemm_swiglu": (None, [P, P, P, P, P, P, I64, I64, I64, I]),
        "orc_fp8_gemm_dequant": (None, [P, P, P, P, P, P, I64, I64, I64, I]),
        "orc_linear": (None, [P, P, P, P, P, I64, I64, I64, I, I]),
        "orc_gateup_swiglu": (None, [P, P, P, P, P, I64, I64, I64, I, I]),
        "orc_fp8_linear": (None, [P, P, P, P, P, I64, I64, I64, I, I]),
        "orc_swiglu_bf16": (None, [P, P, I64, P, I64, I64, I]),
        "orc_gateup_unfused": (None, [P, P, P, P, P, I64, I64, I64, I, I]),
        "orc_gateup_swiglu_quant": (None, [P, P, P, P, P, P, I64, I64, I64, I, I, I]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(a, dtype, shape, name):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {a.dtype}")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {shape}, got {a.shape}")
    return a


# ------------------------------------------------------------------ codecs --
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_bf16_decode(int(b)) for b in flat], dtype=np.float32).reshape(np.shape(bits))


def bf16_from_f64(v: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Nearest bf16 (ties to even) of finite fp64 values, as bit patterns."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.orc_bf16_from_f64_array(_ptr(v), v.size, _ptr(out), threads or default_threads())
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.orc_e4m3_decode(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def e4m3_encode(t: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Nearest E4M3FN code (ties to even) of float32 values already in [-448, 448]."""
    lib = _load()
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    lib.orc_e4m3_encode_array(_ptr(t), t.size, _ptr(out), threads or default_threads())
    return out


# --------------------------------------------------------------- stages -----
def rotate(x: np.ndarray, rot_block: int, threads: int | None = None) -> np.ndarray:
    """fp32 rows after the optional block-128 rotation (x: bf16 bits [M, K])."""
    lib = _load()
    M, K = x.shape
    x = _check(x, np.uint16, (M, K), "x")
    y = np.empty((M, K), dtype=np.float32)
    lib.orc_rotate(_ptr(x), M, K, rot_block, _ptr(y), threads or default_threads())
    return y


def quantize_i8(x: np.ndarray, rot_block: int = 0, threads: int | None = None):
    """Per-row symmetric int8 quantizer: returns (q int8 [M, K], s fp32 [M])."""
    lib = _load()
    M, K = x.shape
    x = _check(x, np.uint16, (M, K), "x")
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_quantize_i8(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), threads or default_threads())
    return q, s


def quantize_fp8(x: np.ndarray, rot_block: int = 0, threads: int | None = None):
    """Per-row symmetric E4M3FN quantizer: returns (q uint8 codes [M, K], s fp32 [M])."""
    lib = _load()
    M, K = x.shape
    x = _check(x, np.uint16, (M, K), "x")
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_quantize_fp8(_ptr(x), M, K, rot_block, _ptr(q), _ptr(s), threads or default_threads())
    return q, s


def quantize_f32_i8(y: np.ndarray, threads: int | None = None):
    """The int8 quantizer alone, on rows that are already fp32 (used by the pins)."""
    lib = _load()
    M, K = y.shape
    y = _check(y, np.float32, (M, K), "y")
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_quantize_f32_i8(_ptr(y), M, K, _ptr(q), _ptr(s), threads or default_threads())
    return q, s


def quantize_f32_fp8(y: np.ndarray, threads: int | None = None):
    """The E4M3FN quantizer alone, on rows that are already fp32 (used by the pins)."""
    lib = _load()
    M, K = y.shape
    y = _check(y, np.float32, (M, K), "y")
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_quantize_f32_fp8(_ptr(y), M, K, _ptr(q), _ptr(s), threads or default_threads())
    return q, s


def gemm_i32(q: np.ndarray, w: np.ndarray, threads: int | None = None) -> np.ndarray:
    lib = _load()
    M, K = q.shape
    N = w.shape[0]
    q = _check(q, np.int8, (M, K), "q")
    w = _check(w, np.int8, (N, K), "w")
    acc = np.empty((M, N), dtype=np.int32)
    lib.orc_gemm_i32(_ptr(q), _ptr(w), M, N, K, _ptr(acc), threads or default_threads())
    return acc


def gemm_fp8(q: np.ndarray, w: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Exact fp8 x fp8 dot products as fp64 [M, N]."""
    lib = _load()
    M, K = q.shape
    N = w.shape[0]
    q = _check(q, np.uint8, (M, K), "q")
    w = _check(w, np.uint8, (N, K), "w")
    acc = np.empty((M, N), dtype=np.float64)
    lib.orc_gemm_fp8(_ptr(q), _ptr(w), M, N, K, _ptr(acc), threads or default_threads())
    return acc


def _epilogue_call(fname, q, s_tok, w, s_ch, bias, n_out, qdtype, threads):
    lib = _load()
    M, K = q.shape
    Nw = w.shape[0]
    q = _check(q, qdtype, (M, K), "q")
    w = _check(w, qdtype, (Nw, K), "w")
    s_tok = _check(s_tok, np.float32, (M,), "s_tok")
    s_ch = _check(s_ch, np.float32, (Nw,), "s_ch")
    if bias is not None:
        bias = _check(bias, np.uint16, (Nw,), "bias")
    y = np.empty((M, n_out), dtype=np.uint16)
    getattr(lib, fname)(_ptr(q), _ptr(s_tok), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y),
                        M, n_out, K, threads or default_threads())
    return y


def gemm_dequant(q, s_tok, w, s_ch, bias=None, threads=None):
    """bf16 bits of q.w^T * s_tok * s_ch + bias (one rounding)."""
    return _epilogue_call("orc_gemm_dequant", q, s_tok, w, s_ch, bias, w.shape[0], np.int8, threads)


def gemm_swiglu(q, s_tok, w_gateup, s_ch, bias=None, threads=None):
    """bf16 bits of silu(gate) * up over the packed [2N, K] weight; output [M, N]."""
    assert w_gateup.shape[0] % 2 == 0
    return _epilogue_call("orc_gemm_swiglu", q, s_tok, w_gateup, s_ch, bias,
                          w_gateup.shape[0] // 2, np.int8, threads)


def fp8_gemm_dequant(q, s_tok, w, s_ch, bias=None, threads=None):
    return _epilogue_call("orc_fp8_gemm_dequant", q, s_tok, w, s_ch, bias, w.shape[0], np.uint8, threads)


def _path_call(fname, x, w, s_ch, bias, rot_block, n_out, wdtype, threads):
    lib = _load()
    M, K = x.shape
    Nw = w.shape[0]
    x = _check(x, np.uint16, (M, K), "x")
    w = _check(w, wdtype, (Nw, K), "w")
    s_ch = _check(s_ch, np.float32, (Nw,), "s_ch")
    if bias is not None:
        bias = _check(bias, np.uint16, (Nw,), "bias")
    y = np.empty((M, n_out), dtype=np.uint16)
    getattr(lib, fname)(_ptr(x), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(y), M, n_out, K,
                        rot_block, threads or default_threads())
    return y


def linear(x, w, s_ch, bias=None, rot_block=0, threads=None):
    return _path_call("orc_linear", x, w, s_ch, bias, rot_block, w.shape[0], np.int8, threads)


def gateup_swiglu(x, w_gateup, s_ch, bias=None, rot_block=0, threads=None):
    return _path_call("orc_gateup_swiglu", x, w_gateup, s_ch, bias, rot_block,
                      w_gateup.shape[0] // 2, np.int8, threads)


def fp8_linear(x, w, s_ch, bias=None, rot_block=0, threads=None):
    return _path_call("orc_fp8_linear", x, w, s_ch, bias, rot_block, w.shape[0], np.uint8, threads)


def swiglu_bf16(g, u, threads=None):
    """bf16 bits of silu(g) * u for bf16 bit arrays g, u [M, N] (one rounding)."""
    lib = _load()
    g = np.ascontiguousarray(g, dtype=np.uint16)
    u = np.ascontiguousarray(u, dtype=np.uint16)
    assert g.shape == u.shape and g.ndim == 2
    M, N = g.shape
    y = np.empty((M, N), dtype=np.uint16)
    lib.orc_swiglu_bf16(_ptr(g), _ptr(u), N, _ptr(y), M, N, threads or default_threads())
    return y


def gateup_unfused(x, w_gateup, s_ch, bias=None, rot_block=0, threads=None):
    """Unfused gate/up: linear onto the 2N packed rows (bf16), then swiglu_bf16 of its halves."""
    return _path_call("orc_gateup_unfused", x, w_gateup, s_ch, bias, rot_block,
                      w_gateup.shape[0] // 2, np.int8, threads)


# ------------------------------------ SwiGLU output quantized for the next linear --
def gateup_swiglu_quant(x, w_gateup, s_ch, bias=None, rot_in=0, rot_out=0, threads=None):
    """Gate/up SwiGLU whose bf16 output goes through the per-token int8 quantizer of
    the next linear (rotation rot_out): returns (q int8 [M, N], s fp32 [M])."""
    lib = _load()
    M, K = x.shape
    Nw = w_gateup.shape[0]
    assert Nw % 2 == 0
    N = Nw // 2
    x = _check(x, np.uint16, (M, K), "x")
    w = _check(w_gateup, np.int8, (Nw, K), "w")
    s_ch = _check(s_ch, np.float32, (Nw,), "s_ch")
    if bias is not None:
        bias = _check(bias, np.uint16, (Nw,), "bias")
    q = np.empty((M, N), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_gateup_swiglu_quant(_ptr(x), _ptr(w), _ptr(s_ch), _ptr(bias), _ptr(q), _ptr(s), M, N, K,
                                rot_in, rot_out, threads or default_threads())
    return q, s
