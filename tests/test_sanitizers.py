"""CPU AddressSanitizer + UndefinedBehaviorSanitizer builds (g++, host code only):

* the oracle (``oracle/w8a8_oracle.cpp``) driven through every entry point on small
  seeded inputs (``tests/sanitize/oracle_driver.cpp``);
* the C ABI's host validation (``w8a8_quantized_linear_amd/csrc/api.cpp``) with
  host-only launcher stand-ins (``tests/sanitize/launcher_stubs.cpp``), driven
  through the argument cases of the ABI tests (``tests/sanitize/abi_driver.cpp``)
  and linked against the HIP runtime (no GPU needed: every call returns before a
  launch).

Each binary must build and exit 0 with no sanitizer report."""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-pthread"]
ROCM = Path("/opt/rocm")


def _build_and_run(tmp_path, name, sources, extra, env_extra):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = tmp_path / name
    cmd = ["g++", *SAN, *extra, *map(str, sources), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, f"build failed:\n{res.stderr[-3000:]}"
    env = dict(os.environ, **env_extra)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, f"{name} failed ({run.returncode}):\n{run.stdout[-2000:]}\n{run.stderr[-4000:]}"
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, run.stderr[-4000:]
    return run.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "oracle_san",
                         [ROOT / "oracle" / "w8a8_oracle.cpp", ROOT / "tests" / "sanitize" / "oracle_driver.cpp"],
                         [], {"ASAN_OPTIONS": "detect_leaks=1"})
    assert "oracle ran clean" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not (ROCM / "lib" / "libamdhip64.so").exists():
        pytest.skip("HIP runtime not installed")
    import torch
    if torch.cuda.is_available():
        pytest.skip("the driver expects the no-device status that valid calls return without a GPU")
    csrc = ROOT / "w8a8_quantized_linear_amd" / "csrc"
    out = _build_and_run(tmp_path, "abi_san",
                         [csrc / "api.cpp", ROOT / "tests" / "sanitize" / "launcher_stubs.cpp",
                          ROOT / "tests" / "sanitize" / "abi_driver.cpp"],
                         ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM / 'include'}", f"-I{ROOT / 'include'}", f"-I{csrc}",
                          f"-L{ROCM / 'lib'}", "-lamdhip64", f"-Wl,-rpath,{ROCM / 'lib'}"],
                         # the HIP runtime's own allocations outlive main: leak checks off
                         {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "all argument checks as expected" in out
