"""Build ``libw8a8.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

    python w8a8_quantized_linear_amd/build.py

(run as a script: importing the package loads the library this produces).

Every HIP source is compiled with packed-fp32 instruction selection disabled
and the correctly rounded fp32 divide the quantizer relies on.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libw8a8.so"
BUILD_DIR = PKG / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["quantize.hip", "gemm.hip", "swiglu.hip", "short.hip", "scratch.hip", "api.cpp"]
# Per-source flags.  The quantizer's fp64 matrix instructions (the rotation's
# cross-quarter transform) take the VGPR form: their results feed vector
# instructions, and results in accumulation registers would cost two copies per
# value and, at 12,016 x 17,408, the third wave per SIMD.
EXTRA = {"quantize.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# measurement aids for the benchmark and the design tests (not the library's C ABI)
PROBE_DIR = PKG / "probe"
PROBE_SOURCES = ["mfma_probe.hip", "fp8_contraction.hip", "f64_mfma_layout.hip", "stream_probe.hip",
                 "lds_probe.hip"]
PROBE_LIB = PROBE_DIR / "libw8a8_probe.so"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, folder: Path = CSRC, tag: str = "") -> Path:
    obj = BUILD_DIR / (tag + src.rsplit(".", 1)[0] + ".o")
    obj.unlink(missing_ok=True)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", str(folder / src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out: Path) -> Path:
    tmp = out.with_suffix(".so.tmp")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    # every kernel launched from host code must have its stub in the library
    nm = subprocess.run(["nm", "--undefined-only", str(tmp)], capture_output=True, text=True)
    missing = [l for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if nm.returncode != 0 or missing:
        raise RuntimeError("link produced a library with undefined kernel stubs:\n" + "\n".join(missing))
    os.replace(tmp, out)
    return out


def build() -> Path:
    """Build libw8a8.so (the library) and probe/libw8a8_probe.so (measurement aids)."""
    BUILD_DIR.mkdir(exist_ok=True)
    jobs = [(src, CSRC, "") for src in SOURCES] + [(src, PROBE_DIR, "probe_") for src in PROBE_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
