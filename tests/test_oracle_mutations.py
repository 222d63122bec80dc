"""The pins are strong enough: copies of the oracle with one plausible mistake planted
each (on the CPU) must fail the ``-m "not gpu"`` oracle pins.

Each mutant is the oracle's C++ source with one textual change, compiled with the
oracle's own g++ flags into a temporary library; the pin files then run in a child
pytest process that loads it (``W8A8_ORACLE_LIB``), and must report a failure.  The
unmutated source must pass the same run (the control).
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "w8a8_oracle.cpp"
PINS = sorted(str(p) for p in (ROOT / "tests").glob("test_oracle_*.py") if p.name != Path(__file__).name)

# (name, text to replace, replacement): each a mistake someone could make writing the oracle
MUTANTS = [
    ("fp8 epilogue scaled by 2 (wrong power-of-two shift)",
     "dequant(a, 18, s_tok[m], s_ch[n], bias, n)", "dequant(a, 17, s_tok[m], s_ch[n], bias, n)"),
    ("int8 codes rounded half away from zero",
     "float r = std::nearbyint(t);", "float r = std::round(t);"),
    ("int8 scale amax / 128",
     "float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    ("Hadamard sign of i | j instead of i & j",
     "__builtin_popcount((unsigned)(i & j))", "__builtin_popcount((unsigned)(i | j))"),
    ("rotation without the 1/sqrt(128) normalization",
     "y[b + j] = (float)(acc * c);", "y[b + j] = (float)acc;"),
    ("bias dropped from the epilogue",
     "if (bias) v += (double)bf16_to_f32(bias[n]);", "(void)bias;"),
    ("SwiGLU gate and up swapped",
     "y[e] = f64_to_bf16(silu_times(g, u));", "y[e] = f64_to_bf16(silu_times(u, g));"),
    ("fp8 quotient clamped to 240 instead of 448",
     "if (t > 448.0f) t = 448.0f;", "if (t > 240.0f) t = 240.0f;"),
    ("SwiGLU output quantized with the input's rotation instead of the next linear's",
     "orc_quantize_i8(h.data(), M, N, rot_out, q, s, nthreads);",
     "orc_quantize_i8(h.data(), M, N, rot_in, q, s, nthreads);"),
]


def _build(src_text: str, out: Path) -> Path:
    src = out.with_suffix(".cpp")
    src.write_text(src_text)
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math", "-ffp-contract=off",
           str(src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    return out


def _run_pins(lib: Path) -> subprocess.CompletedProcess:
    env = dict(os.environ, W8A8_ORACLE_LIB=str(lib), OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS", "8"))
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *PINS]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_control_passes(tmp_path):
    res = _run_pins(_build(SRC.read_text(), tmp_path / "control.so"))
    assert res.returncode == 0, res.stdout[-3000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    text = SRC.read_text()
    assert text.count(old) == 1, f"mutation site not unique: {old!r}"
    res = _run_pins(_build(text.replace(old, new), tmp_path / "mutant.so"))
    assert res.returncode != 0, f"no pin caught: {name}\n{res.stdout[-2000:]}"
    failed = [l for l in res.stdout.splitlines() if l.startswith("FAILED")]
    print(f"{name}: caught by {failed[:1]}")
