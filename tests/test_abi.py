"""Host-side tests of the C-ABI library: it loads, exports every entry point the
header declares, and rejects bad arguments before touching any device.

No kernel is launched here.  Argument checks run before the device check, so
the expected statuses come back on a machine without a GPU; pointers passed
are dummy, never dereferenced.
"""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "w8a8.h"
LIB = ROOT / "w8a8_quantized_linear_amd" / "libw8a8.so"

OK, NULLP, SHAPE, MISALIGNED, BADARG, DEVICE, LAUNCH, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7
A = 0x10000   # a 16-byte aligned dummy address (never dereferenced)
U = A + 8     # misaligned


@pytest.fixture(scope="module")
def lib():
    if not LIB.exists():
        import __graft_entry__
        __graft_entry__._hip_build_module().build()
    lib = ctypes.CDLL(str(LIB))
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "w8a8_status_string": (ctypes.c_char_p, [I]),
        "w8a8_workspace_bytes": (SZ, [I64, I64]),
        "w8a8_quantize_act": (I, [P, I64, I64, I, P, P, P]),
        "w8a8_quantize_act_fp8": (I, [P, I64, I64, I, P, P, P]),
        "w8a8_gemm_i32": (I, [P, P, P, I64, I64, I64, P]),
        "w8a8_gemm_i32_packed": (I, [P, P, P, I64, I64, I64, P]),
        "w8a8_gemm_dequant": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_gemm_swiglu": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_fp8_gemm_dequant": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_linear": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_gateup_swiglu": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_fp8_linear": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_packed_bytes": (SZ, [I64, I64]),
        "w8a8_pack_weight": (I, [P, I64, I64, P, P]),
        "w8a8_quantize_act_packed": (I, [P, I64, I64, I, P, P, P]),
        "w8a8_quantize_act_fp8_packed": (I, [P, I64, I64, I, P, P, P]),
        "w8a8_gemm_dequant_packed": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_gemm_swiglu_packed": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_fp8_gemm_dequant_packed": (I, [P, P, P, P, P, P, I64, I64, I64, P]),
        "w8a8_swiglu": (I, [P, P, I64, P, I64, I64, P]),
        "w8a8_linear_packed": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_gateup_swiglu_packed": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_fp8_linear_packed": (I, [P, P, P, P, P, I64, I64, I64, I, P, SZ, P]),
        "w8a8_swiglu_quant_workspace_bytes": (SZ, [I64, I64, I64]),
        "w8a8_gateup_swiglu_quant_packed": (I, [P, P, P, P, I64, I64, I64, I, I, P, P, P, SZ, P]),
        "w8a8_linear_packed_noalloc": (I, [P, P, P, P, P, I64, I64, I64, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


def declared_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    want = {"w8a8_status_string", "w8a8_workspace_bytes", "w8a8_quantize_act",
            "w8a8_quantize_act_fp8", "w8a8_gemm_i32", "w8a8_gemm_dequant", "w8a8_gemm_swiglu",
            "w8a8_fp8_gemm_dequant", "w8a8_linear", "w8a8_gateup_swiglu", "w8a8_fp8_linear",
            "w8a8_packed_bytes", "w8a8_pack_weight", "w8a8_linear_packed",
            "w8a8_gateup_swiglu_packed", "w8a8_fp8_linear_packed", "w8a8_quantize_act_packed",
            "w8a8_quantize_act_fp8_packed", "w8a8_gemm_dequant_packed", "w8a8_gemm_swiglu_packed",
            "w8a8_fp8_gemm_dequant_packed", "w8a8_swiglu", "w8a8_swiglu_quant_workspace_bytes",
            "w8a8_gateup_swiglu_quant_packed", "w8a8_gemm_i32_packed"}
    assert want <= set(declared_symbols())


def test_measurement_aids_are_not_in_the_library():
    """The MFMA rate and fp8-accuracy probes live in the bench-only probe library."""
    import subprocess
    syms = subprocess.run(["nm", "-D", "--defined-only", str(LIB)], capture_output=True, text=True).stdout
    assert "w8a8_" in syms and "probe" not in syms
    probe = ROOT / "w8a8_quantized_linear_amd" / "probe" / "libw8a8_probe.so"
    psyms = subprocess.run(["nm", "-D", "--defined-only", str(probe)], capture_output=True, text=True).stdout
    assert "w8a8_probe_mfma_rate" in psyms and "w8a8_probe_fp8_contraction" in psyms


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert lib.w8a8_status_string(s).decode().startswith("W8A8_")
    assert b"unknown" in lib.w8a8_status_string(99)


def test_packed_and_workspace_bytes(lib):
    # packed codes: rows rounded up to a multiple of 32
    assert lib.w8a8_packed_bytes(0, 128) == 0
    assert lib.w8a8_packed_bytes(1, 128) == 32 * 128
    assert lib.w8a8_packed_bytes(32, 4096) == 32 * 4096
    assert lib.w8a8_packed_bytes(1502, 4096) == 1504 * 4096
    # workspace: packed codes, then the fp32 scales, each on a 256-byte boundary
    assert lib.w8a8_workspace_bytes(0, 128) == 0
    assert lib.w8a8_workspace_bytes(1, 128) == 32 * 128 + 256
    assert lib.w8a8_workspace_bytes(12016, 17408) == 12032 * 17408 + ((12016 * 4 + 255) // 256) * 256
    assert lib.w8a8_workspace_bytes(3, 64) % 256 == 0


def test_quantize_argument_checks(lib):
    q = lib.w8a8_quantize_act
    assert q(None, 4, 128, 0, A, A, None) == NULLP
    assert q(A, 4, 128, 0, None, A, None) == NULLP
    assert q(A, 4, 128, 0, A, None, None) == NULLP
    assert q(A, -1, 128, 0, A, A, None) == SHAPE
    assert q(A, 4, 0, 0, A, A, None) == SHAPE
    assert q(A, 4, 24, 0, A, A, None) == SHAPE               # K % 32
    assert q(A, 4, 48, 0, A, A, None) == SHAPE
    assert q(A, 4, 131072 + 16, 0, A, A, None) == SHAPE      # K > max
    assert q(A, 4, 64, 128, A, A, None) == SHAPE             # rotation needs K % 128
    assert q(A, 4, 128, 64, A, A, None) == BADARG            # rot_block not 0/128
    assert q(U, 4, 128, 0, A, A, None) == MISALIGNED
    assert q(A, 4, 128, 0, U, A, None) == MISALIGNED
    assert q(A, 0, 128, 0, A, A, None) == OK                 # M == 0: nothing enqueued
    assert lib.w8a8_quantize_act_fp8(A, 0, 256, 128, A, A, None) == OK
    assert lib.w8a8_quantize_act_fp8(A, 4, 200, 128, A, A, None) == SHAPE
    for qp in (lib.w8a8_quantize_act_packed, lib.w8a8_quantize_act_fp8_packed):
        assert qp(A, 4, 96, 0, A, A, None) == SHAPE          # packed codes need K % 64
        assert qp(A, 4, 128, 0, None, A, None) == NULLP
        assert qp(A, 4, 128, 0, U, A, None) == MISALIGNED
        assert qp(A, 0, 64, 0, A, A, None) == OK


def test_gemm_argument_checks(lib):
    g = lib.w8a8_gemm_dequant
    assert g(None, A, A, A, None, A, 4, 8, 128, None) == NULLP
    assert g(A, None, A, A, None, A, 4, 8, 128, None) == NULLP
    assert g(A, A, A, None, None, A, 4, 8, 128, None) == NULLP
    assert g(A, A, A, A, None, None, 4, 8, 128, None) == NULLP
    assert g(A, A, A, A, None, A, 4, 8, 64, None) == SHAPE    # K % 128
    assert g(A, A, A, A, None, A, 4, 12, 128, None) == SHAPE  # N % 8
    assert g(A, A, A, A, None, A, 4, 0, 128, None) == SHAPE
    assert g(A, A, A, A, None, A, -2, 8, 128, None) == SHAPE
    assert g(A, A, A, A, None, A, 4, 8, 131072 + 128, None) == SHAPE
    assert g(A, A, A, A, U, A, 4, 8, 128, None) == MISALIGNED  # bias
    assert g(A, A, U, A, None, A, 4, 8, 128, None) == MISALIGNED
    assert g(A, A, A, A, None, A, 0, 8, 128, None) == OK
    assert lib.w8a8_gemm_i32(A, A, None, 4, 8, 128, None) == NULLP
    assert lib.w8a8_gemm_i32(A, A, A, 0, 8, 128, None) == OK
    assert lib.w8a8_gemm_swiglu(A, A, A, A, None, A, 4, 8, 100, None) == SHAPE
    assert lib.w8a8_fp8_gemm_dequant(A, A, A, A, None, A, 4, 8, 256, None) in (OK, DEVICE)
    for gp in (lib.w8a8_gemm_dequant_packed, lib.w8a8_gemm_swiglu_packed, lib.w8a8_fp8_gemm_dequant_packed):
        assert gp(None, A, A, A, None, A, 4, 8, 128, None) == NULLP
        assert gp(A, A, A, A, None, A, 4, 8, 64, None) == SHAPE
        assert gp(A, A, A, A, None, A, 4, 12, 128, None) == SHAPE
        assert gp(A, A, A, A, None, A, 0, 8, 128, None) == OK


def test_whole_path_argument_checks(lib):
    f = lib.w8a8_linear
    ws = lib.w8a8_workspace_bytes(4, 256)
    assert f(A, A, A, None, A, 4, 8, 256, 0, None, ws, None) == NULLP
    assert f(None, None, None, None, None, 0, 8, 256, 0, None, 0, None) == OK  # M == 0 reads nothing
    assert f(A, A, A, None, A, 4, 8, 256, 0, A, ws - 1, None) == BADARG   # workspace too small
    assert f(A, A, A, None, A, 4, 8, 256, 3, A, ws, None) == BADARG      # rot_block
    assert f(A, A, A, None, A, 4, 8, 192, 0, A, ws, None) == SHAPE       # K % 128
    assert f(A, A, A, None, A, 4, 8, 256, 0, U, ws, None) == MISALIGNED
    assert f(A, A, A, None, A, 0, 8, 256, 0, A, 0, None) == OK
    assert lib.w8a8_gateup_swiglu(A, A, A, None, A, 4, 8, 256, 128, A, ws - 256, None) == BADARG
    assert lib.w8a8_fp8_linear(A, A, None, None, A, 4, 8, 256, 0, A, ws, None) == NULLP
    for g in (lib.w8a8_linear_packed, lib.w8a8_gateup_swiglu_packed, lib.w8a8_fp8_linear_packed):
        assert g(A, None, A, None, A, 4, 8, 256, 0, A, ws, None) == NULLP
        assert g(A, A, A, None, A, 4, 8, 256, 0, A, ws - 1, None) == BADARG
        assert g(A, A, A, None, A, 4, 12, 256, 0, A, ws, None) == SHAPE
        assert g(None, None, None, None, None, 0, 8, 256, 0, None, 0, None) == OK


def test_swiglu_argument_checks(lib):
    f = lib.w8a8_swiglu
    assert f(None, A, 16, A, 4, 16, None) == NULLP
    assert f(A, A, 16, None, 4, 16, None) == NULLP
    assert f(A, A, 16, A, 4, 12, None) == SHAPE        # N % 8
    assert f(A, A, 8, A, 4, 16, None) == SHAPE         # ld < N
    assert f(A, A, 20, A, 4, 16, None) == SHAPE        # ld % 8
    assert f(A, A, 16, A, -1, 16, None) == SHAPE
    assert f(U, A, 16, A, 4, 16, None) == MISALIGNED
    assert f(A, U, 16, A, 4, 16, None) == MISALIGNED
    assert f(None, None, 32, None, 0, 16, None) == OK  # M == 0


def test_pack_weight_argument_checks(lib):
    p = lib.w8a8_pack_weight
    assert p(None, 4, 128, A, None) == NULLP
    assert p(A, 4, 128, None, None) == NULLP
    assert p(A, 4, 96, A, None) == SHAPE          # K % 64
    assert p(A, 4, 0, A, None) == SHAPE
    assert p(A, -1, 128, A, None) == SHAPE
    assert p(A, 4, 131072 + 64, A, None) == SHAPE
    assert p(U, 4, 128, A, None) == MISALIGNED
    assert p(A, 4, 128, U, None) == MISALIGNED
    assert p(None, 0, 128, None, None) == OK      # nothing to pack


def test_swiglu_quant_sizes_and_argument_checks(lib):
    ws = lib.w8a8_swiglu_quant_workspace_bytes(4, 256, 512)
    assert ws == lib.w8a8_workspace_bytes(4, 512) + 4 * 256 * 2     # x codes + scales, then bf16 h
    assert lib.w8a8_swiglu_quant_workspace_bytes(3, 192, 512) == lib.w8a8_workspace_bytes(3, 512) + 1280
    assert lib.w8a8_swiglu_quant_workspace_bytes(0, 256, 512) == 0
    g = lib.w8a8_gateup_swiglu_quant_packed
    assert g(A, A, A, None, 4, 256, 512, 0, 128, A, A, A, ws - 1, None) == BADARG
    assert g(A, A, A, None, 4, 256, 512, 3, 128, A, A, A, ws, None) == BADARG   # rot_in
    assert g(A, A, A, None, 4, 256, 512, 0, 64, A, A, A, ws, None) == BADARG    # rot_out
    assert g(A, A, A, None, 4, 256, 512, 0, 128, None, A, A, ws, None) == NULLP
    assert g(A, A, A, None, 4, 256, 512, 0, 128, A, None, A, ws, None) == NULLP
    assert g(A, A, A, None, 4, 256, 512, 0, 128, A, A, U, ws, None) == MISALIGNED
    assert g(A, A, A, U, 4, 256, 512, 0, 128, A, A, A, ws, None) == MISALIGNED  # bias
    assert g(A, A, A, None, 4, 192, 512, 0, 128, A, A, A, ws, None) == SHAPE    # rotation: N % 128
    assert g(A, A, A, None, 4, 200, 512, 0, 0, A, A, A, ws, None) == SHAPE      # N % 64
    assert g(A, A, A, None, 4, 256, 320, 0, 0, A, A, A, ws, None) == SHAPE      # K % 128
    assert g(A, A, A, None, 4, 131072 + 128, 512, 0, 0, A, A, A, 1 << 40, None) == SHAPE  # N too long
    assert g(None, None, None, None, 0, 256, 512, 0, 0, None, None, None, 0, None) == OK


def test_noalloc_argument_checks(lib):
    """The entry point without a workspace: the allocating entry point's checks, and the
    fixed scratch limit (64 MiB) right after the shapes."""
    f = lib.w8a8_linear_packed_noalloc
    assert b"scratch" in lib.w8a8_status_string(SCRATCH)
    assert f(A, A, A, None, A, 4, 8, 192, 0, None) == SHAPE                    # K % 128
    assert f(A, A, A, None, A, 4, 8, 256, 3, None) == BADARG                   # rot_block
    assert f(None, None, None, None, None, 0, 8, 256, 0, None) == OK           # M == 0
    assert f(A, A, A, None, None, 4, 8, 256, 0, None) == NULLP
    assert f(A, A, U, None, A, 4, 8, 256, 0, None) == MISALIGNED
    assert f(A, A, A, U, A, 4, 8, 256, 0, None) == MISALIGNED                  # bias
    # 12,016 x 17,408: 209 MB of codes, beyond the 64 MiB array (before any pointer check)
    assert f(None, None, None, None, None, 12016, 5120, 17408, 128, None) == SCRATCH
    # the boundary: 4,096 x 16,384 codes are 64 MiB, plus 16 KiB of scales -> too large;
    # 4,064 rows fit
    assert lib.w8a8_workspace_bytes(4096, 16384) == (64 << 20) + 16384
    assert f(A, A, A, None, A, 4096, 8, 16384, 0, None) == SCRATCH
    assert lib.w8a8_workspace_bytes(4064, 16384) <= 64 << 20
    import torch
    if not torch.cuda.is_available():
        assert f(A, A, A, None, A, 4064, 8, 16384, 0, None) == DEVICE


def test_packed_i32_argument_checks(lib):
    g = lib.w8a8_gemm_i32_packed
    assert g(None, A, A, 4, 8, 128, None) == NULLP
    assert g(A, A, None, 4, 8, 128, None) == NULLP
    assert g(A, A, A, 4, 8, 64, None) == SHAPE
    assert g(A, A, A, 4, 12, 128, None) == SHAPE
    assert g(A, U, A, 4, 8, 128, None) == MISALIGNED
    assert g(A, A, A, 0, 8, 128, None) == OK


def test_valid_call_without_gpu_reports_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert lib.w8a8_quantize_act(A, 4, 128, 0, A, A, None) == DEVICE
    assert lib.w8a8_gemm_i32(A, A, A, 4, 8, 128, None) == DEVICE
    assert lib.w8a8_pack_weight(A, 4, 128, A, None) == DEVICE
    assert lib.w8a8_gemm_i32_packed(A, A, A, 4, 8, 128, None) == DEVICE
    ws = lib.w8a8_swiglu_quant_workspace_bytes(4, 256, 512)
    assert lib.w8a8_gateup_swiglu_quant_packed(A, A, A, None, 4, 256, 512, 0, 128, A, A, A, ws, None) == DEVICE


def test_probe_argument_checks():
    """The bench-only probes refuse bad arguments before launching anything."""
    probe = ROOT / "w8a8_quantized_linear_amd" / "probe" / "libw8a8_probe.so"
    pl = ctypes.CDLL(str(probe))
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    pl.w8a8_probe_mfma_rate.restype, pl.w8a8_probe_mfma_rate.argtypes = I, [I, I64, I, P, P]
    r = pl.w8a8_probe_mfma_rate
    assert r(2, 10, 1, A, None) == -1 and r(0, 0, 1, A, None) == -1 and r(1, 10, 0, A, None) == -1
    assert r(0, 10, 1, None, None) == -1 and r(0, (1 << 40) + 1, 1, A, None) == -1
    pl.w8a8_probe_fp8_contraction.restype = I
    pl.w8a8_probe_fp8_contraction.argtypes = [I, P, P, P, I64, I64, I64, P]
    c = pl.w8a8_probe_fp8_contraction
    assert c(0, A, A, A, 33, 32, 64, None) == -1      # M % 32
    assert c(0, A, A, A, 32, 32, 96, None) == -1      # K % 64
    assert c(5, A, A, A, 32, 32, 64, None) == -1      # kind
    assert c(0, None, A, A, 32, 32, 64, None) == -1
    pl.w8a8_probe_stream.restype, pl.w8a8_probe_stream.argtypes = I, [I, P, P, I64, P]
    st = pl.w8a8_probe_stream
    assert st(2, A, A, 8, None) == -1 and st(0, None, A, 8, None) == -1 and st(1, A, None, 8, None) == -1
    assert st(0, A, A, 0, None) == -1 and st(0, A, A, -1, None) == -1
    pl.w8a8_probe_lds.restype, pl.w8a8_probe_lds.argtypes = I, [I, I, I, P, P]
    ld = pl.w8a8_probe_lds
    assert ld(4, 1, 1, A, None) == -1 and ld(-1, 1, 1, A, None) == -1 and ld(0, 0, 1, A, None) == -1
    assert ld(0, 1, 0, A, None) == -1 and ld(3, 1, 1, None, None) == -1
