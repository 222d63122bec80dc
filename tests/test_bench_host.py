"""bench.py's host logic, on the CPU: the one-GPU refusal, the HBM-traffic summary
built from rocprofv3 counter files (calibration scaling, per-dispatch sums, the
average per launch), and the rule that stored traffic is reported only for the
kernel sources it was measured on."""
import csv
import json
import shutil
import subprocess
import sys

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]
ADD = ("void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float>, "
       "std::array<char*, 2ul> >(int, at::native::CUDAFunctorOnSelf_add<float>, std::array<char*, 2ul>)")
FILL = ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
        "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)")
GEMM = ("void w8a8::(anonymous namespace)::gemm_tile<192, 128, 2, 2, 64, 4, (w8a8::Epi)1, false, true, true>"
        "(unsigned char const*, float const*, unsigned char const*, float const*, unsigned short const*, "
        "void*, long, long, long, int, int, w8a8::(anonymous namespace)::QuantOut)")
PERSIST = ("void w8a8::(anonymous namespace)::gemm_persist<(w8a8::Epi)1, false, true, true>"
           "(unsigned char const*, float const*, unsigned char const*, float const*, unsigned short const*, "
           "void*, long, long, long, int, int)")
QUANT = "void w8a8::(anonymous namespace)::quantize_rows<128, 1, true, false>(unsigned short const*, long)"


def _write_run(d, counter, rows):
    """rows: (dispatch id, kernel name, value); several rows of one dispatch are summed
    (rocprofv3 reports a counter per hardware instance in some configurations)."""
    d.mkdir(parents=True)
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for i, (disp, name, val) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Correlation_Id=i + 1, Dispatch_Id=disp, Agent_Id="Agent 1", Kernel_Name=name,
                     Counter_Name=counter, Counter_Value=val)
            w.writerow(r)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(bench.ROOT / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_pmc_summary_scales_each_counter_by_its_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "feedfacecafebeef")
    cal_kib = bench.CALIBRATION_BYTES / 1024.0
    # FETCH_SIZE reads half of the calibration copy's bytes (factor 2); the fill that
    # precedes it is smaller and must not be taken for the calibration kernel
    _write_run(tmp_path / "f", "FETCH_SIZE", [
        (1, FILL, 17.5), (2, ADD, cal_kib / 2), (3, QUANT, 900.0),
        (4, GEMM, 1000.0), (4, GEMM, 500.0),          # dispatch 4: two instances, 1500 KiB
        (5, GEMM, 2500.0),                            # dispatch 5: 2500 KiB
    ])
    # WRITE_SIZE is exact (factor 1)
    _write_run(tmp_path / "w", "WRITE_SIZE", [
        (1, FILL, 64.0), (2, ADD, cal_kib), (3, QUANT, 300.0), (4, GEMM, 120.0), (5, GEMM, 80.0),
    ])
    rec = bench.pmc_summary("wl", str(tmp_path / "f"), str(tmp_path / "w"))
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["gemm_dispatches"] == 2
    assert rec["fetch_kib_per_launch"] == pytest.approx(2000.0)
    assert rec["write_kib_per_launch"] == pytest.approx(100.0)
    assert rec["gemm_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2 + 100.0 * 1024)
    assert rec["gemm_kernel"] == "w8a8::gemm_tile<192, 128, 2, 2, 64, 4, (w8a8::Epi)1, false, true, true>"
    assert rec["sources_digest"] == "feedfacecafebeef"


def test_pmc_summary_finds_the_persistent_gemm(tmp_path, monkeypatch):
    """256 x 256 workloads run gemm_persist; its dispatches are the GEMM's."""
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0123456789abcdef")
    cal_kib = bench.CALIBRATION_BYTES / 1024.0
    _write_run(tmp_path / "f", "FETCH_SIZE", [(1, ADD, cal_kib / 2), (2, QUANT, 900.0), (3, PERSIST, 4000.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [(1, ADD, cal_kib), (2, QUANT, 300.0), (3, PERSIST, 250.0)])
    rec = bench.pmc_summary("wl", str(tmp_path / "f"), str(tmp_path / "w"))
    assert rec["gemm_kernel"] == "w8a8::gemm_persist<(w8a8::Epi)1, false, true, true>"
    assert rec["gemm_dispatches"] == 1
    # the quantizer of the same runs, each counter scaled by its own factor (2 and 1)
    assert rec["quantizer_kernel"] == "w8a8::quantize_rows<128, 1, true, false>"
    assert rec["quantizer_bytes_per_launch"] == pytest.approx((2 * 900.0 + 300.0) * 1024.0)
    assert rec["gemm_bytes_per_launch"] == pytest.approx(4000.0 * 1024 * 2 + 250.0 * 1024)


def test_pmc_summary_without_a_gemm_dispatch_fails(tmp_path):
    _write_run(tmp_path / "f", "FETCH_SIZE", [(1, ADD, 1.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [(1, ADD, 1.0)])
    with pytest.raises(SystemExit):
        bench.pmc_summary("wl", str(tmp_path / "f"), str(tmp_path / "w"))


def test_stored_traffic_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_wl.json").write_text(
        json.dumps({"sources_digest": "aaaa", "gemm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "aaaa")
    assert bench.stored_traffic("wl") == 123.0
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "bbbb")
    assert bench.stored_traffic("wl") is None
    assert bench.stored_traffic("other") is None


def test_sources_digest_ignores_comments_and_tracks_code(tmp_path, monkeypatch):
    csrc = bench.ROOT / "w8a8_quantized_linear_amd" / "csrc"
    dst = tmp_path / "w8a8_quantized_linear_amd" / "csrc"
    shutil.copytree(csrc, dst)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    base = bench.kernel_sources_digest()
    assert base == (monkeypatch.undo() or bench.kernel_sources_digest())   # the copy digests like the tree
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    g = dst / "gemm.hip"
    g.write_text(g.read_text() + "\n// a trailing comment\n/* and a\n   block comment */\n\n")
    assert bench.kernel_sources_digest() == base
    g.write_text(g.read_text() + "\nstatic int w8a8_digest_probe = 1;\n")
    assert bench.kernel_sources_digest() != base
