"""Benchmark of the W8A8 quantized projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over one batch: the per-token
quantizer (stage 1) followed by the int8 GEMM with its fused epilogue (stages 2
and 3) -- the two kernels ``w8a8_linear_packed`` / ``w8a8_gateup_swiglu_packed`` /
``w8a8_fp8_linear_packed`` enqueue (activation codes written in the packed
layout, weight packed once at load time), launched here through their stage
entry points (``w8a8_quantize_act*_packed`` and the ``*_packed`` GEMMs).  Inputs
(activations, quantized and packed weights, scales, bias) are resident in HBM
before the timed region; successive steps rotate through enough copies of them
(>= 512 MiB in total) that no step finds its operands in the 256 MiB
last-level cache.

Before timing, W untimed warmup steps run (by default as many as fill about
0.25 s: the GPU raises its clock over the first tens of milliseconds of
sustained load, and steps timed inside that ramp run up to 13% slow).  The
timed region runs exactly K steps with nothing else enqueued.  Then each
library call of the step runs on its own, its K launches back to back between
two HIP events on the launch stream, which gives the per-kernel average launch
durations (events between the kernels of a step would idle the GPU for a few
microseconds each, so they stay out of both measurements).

Before the warmup steps, steps run untimed for about 0.3 s whatever W is (the
clock ramp; reported as ``clock_ramp_steps``), so that an explicit small W does
not put the timed steps inside the ramp.

Other paths (--path): the unfused gate/up chain, the whole-path call as one
library call, and for gate/up workloads the SwiGLU output quantized for the next
linear (swiglu-quant: the three kernels of ``w8a8_gateup_swiglu_quant_packed``);
the ops counted stay those of the GEMM.

Prints one JSON line: metric = TOPS of the whole path (2*M*N_w*K ops per step
over the step time), the roofline of the dominant kernel (the GEMM) with its
event-timed average duration, the quantizer's bandwidth, and the CPU oracle
timed on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

DEFAULT_WORKLOAD = "down_12016x17408x5120"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP8_TFLOPS = 5000.0     # dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 MFMA (the E4M3FN GEMM runs on it)
PEAK_HBM_GBS = 8000.0        # HBM3E 8 TB/s
ROTATION_BYTES = 512 << 20
CALIBRATION_BYTES = 256 << 20   # plain device copy run before the warmup (counter calibration)
WARMUP_SECONDS = 0.25           # default untimed warmup: the GPU's clock ramps up under load
RAMP_SECONDS = 0.3              # untimed steps before the warmup steps (clock ramp), always run
# Context only (not this metric): the INT8 card's whole-model batch-1 forward on an H100
# 80 GB at 2,270 tokens ("CLEF Calibrated INT8 ConvRot" card, latency table).
H100_CONTEXT = {"hardware": "H100 80 GB", "workload": "whole model, batch 1, 2,270 input tokens",
                "int8_cute_ms": 170.62, "bf16_ms": 241.09,
                "source": "CLEF Calibrated INT8 ConvRot card, latency table",
                "note": "context only: a whole-model latency, not a measurement of this kernel path"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as fill about 0.25 s, at least 40: "
                         "the GPU raises its clock over the first tens of milliseconds of sustained "
                         "load, and steps timed before that run up to 13%% slow)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--shard", type=int, default=1, metavar="P",
                    help="time one GPU's share of the workload split P ways, on this one GPU: token "
                         "rows (ceil(M / P)) for the linear and fp8 workloads, output columns (N / P of "
                         "each of gate and up, so the SwiGLU stays local) for gate/up; nothing else changes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("fused", "unfused", "single", "swiglu-quant"),
                    default="fused",
                    help="fused: quantizer and GEMM with its fused epilogue, timed per kernel; "
                         "unfused (gate/up workloads): the fuse_mlp=False chain -- GEMM onto the 2N "
                         "packed rows with the dequant epilogue, then w8a8_swiglu; single (int8): "
                         "the whole-path entry point as one call (one kernel for short batches); "
                         "swiglu-quant (gate/up): the SwiGLU output quantized for the next linear "
                         "(w8a8_gateup_swiglu_quant_packed: the fused SwiGLU GEMM writing bf16 h, then "
                         "the per-token quantizer on h)")
    ap.add_argument("--rot-out", type=int, choices=(0, 128), default=128,
                    help="rotation block of the next linear's input for the swiglu-quant path "
                         "(the down projection rotates by 128)")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="instead of the workload: the rate the matrix cores sustain with register "
                         "operands and no memory traffic (int8 32x32x32 and bf16 32x32x16 MFMAs), "
                         "after a ramp-up launch -- the measured-clock ceiling for the GEMM")
    ap.add_argument("--lds-patterns", action="store_true",
                    help="instead of the workload line: the time of the GEMM's MFMA operand reads "
                         "from LDS (ds_read_b128 of 32 rows x 2 chunks) with no swizzle, the earlier "
                         "swizzle key and the GEMM's key, against contiguous 16-byte reads")
    ap.add_argument("--stream-peak", action="store_true",
                    help="instead of the workload line: on each workload's activation shape, the HBM "
                         "rate of a kernel with the quantizer's traffic and no arithmetic (2 bytes read, "
                         "1 written per element), of a plain bf16 copy, and of the library's quantizer "
                         "itself, event-timed in one process after a clock ramp -- the achievable "
                         "streaming ceiling the quantizer is set against")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the workload line: the vendor library's GEMM on each large workload's "
                         "shape (hipBLASLt through torch: torch._int_mm, int8 -> int32, for the int8 "
                         "workloads; torch._scaled_mm with row-wise scales, E4M3FN -> bf16, for fp8) "
                         "beside this library's GEMM on the same codes (w8a8_gemm_i32_packed, or the "
                         "fp8 dequant GEMM), event-timed after a clock ramp -- context for the GEMM's "
                         "roofline fraction")
    ap.add_argument("--drift", action="store_true",
                    help="instead of timing: relative L2 drift of every workload's W8A8 output from "
                         "the fp64 unquantized projection, without and with the block rotation")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script into "
                         "profiles/traffic_<workload>.json and exit")
    return ap.parse_args()


def kernel_sources_digest() -> str:
    """Digest of the sources of the kernels the stored counter records cover (the GEMM
    and the activation quantizer), with comments and blank lines removed (a comment
    edit does not change a kernel)."""
    import re
    h = hashlib.sha256()
    for name in ("gemm.hip", "internal.h", "epilogue_math.h", "quantize.hip", "quant_math.h"):
        text = (ROOT / "w8a8_quantized_linear_amd" / "csrc" / name).read_text()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str = "gemm"):
    """HBM bytes per launch of the GEMM (or, with kernel="quantizer", of the activation
    quantizer) from the committed rocprofv3 counter runs, if they were taken on the
    current kernel sources; else None."""
    p = ROOT / "profiles" / f"traffic_{workload}.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text())
    if rec.get("sources_digest") != kernel_sources_digest():
        return None
    return rec.get(f"{kernel}_bytes_per_launch")


def _pmc_per_kernel(run_dir: str, counter: str):
    """Mean counter value (KiB per dispatch) per kernel name from a rocprofv3 csv run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        per_dispatch = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name), v in per_dispatch.items():
            vals.setdefault(name, []).append(v)
    return vals


def pmc_summary(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """HBM bytes per GEMM launch from FETCH_SIZE / WRITE_SIZE, each scaled by the factor
    that makes the calibration copy read / write exactly CALIBRATION_BYTES."""
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")

    def pick(d, pred):
        ks = [k for k in d if pred(k)]
        if not ks:
            raise SystemExit(f"no kernel matching in {sorted(d)[:5]}")
        return ks
    # the calibration add reads and writes CALIBRATION_BYTES (the largest elementwise
    # kernel in the run); the GEMM is gemm_persist (256 x 256 tiles) or gemm_tile
    copy_k = max(pick(fetch, lambda k: "elementwise" in k.lower()), key=lambda k: max(fetch[k]))
    gemm_k = pick(fetch, lambda k: "gemm_tile" in k or "gemm_persist" in k)[0]
    copy_w = max(pick(write, lambda k: "elementwise" in k.lower()), key=lambda k: max(write[k]))
    f_copy, w_copy = max(fetch[copy_k]), max(write[copy_w])
    f_factor = CALIBRATION_BYTES / (f_copy * 1024.0)
    w_factor = CALIBRATION_BYTES / (w_copy * 1024.0)
    f_gemm = sum(fetch[gemm_k]) / len(fetch[gemm_k])
    w_gemm = sum(write[gemm_k]) / len(write[gemm_k])

    def short(k):
        return k.split(">(")[0].replace("(anonymous namespace)::", "").removeprefix("void ") + ">"
    rec = {"workload": workload, "sources_digest": kernel_sources_digest(),
           "gemm_kernel": short(gemm_k), "gemm_dispatches": len(fetch[gemm_k]),
           "fetch_kib_per_launch": f_gemm, "write_kib_per_launch": w_gemm,
           "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
           "fetch_factor": f_factor, "write_factor": w_factor,
           "gemm_bytes_per_launch": f_gemm * 1024.0 * f_factor + w_gemm * 1024.0 * w_factor}
    # the activation quantizer of the same runs (the first quantizer kernel of the step;
    # a path that also quantizes the SwiGLU output launches a second one, reported apart)
    quant = sorted(k for k in fetch if "quantize_rows" in k and k in write)
    for i, k in enumerate(quant):
        f_q = sum(fetch[k]) / len(fetch[k])
        w_q = sum(write[k]) / len(write[k])
        tag = "quantizer" if i == 0 else f"quantizer{i + 1}"
        rec[f"{tag}_kernel"] = short(k)
        rec[f"{tag}_dispatches"] = len(fetch[k])
        rec[f"{tag}_bytes_per_launch"] = f_q * 1024.0 * f_factor + w_q * 1024.0 * w_factor
    return rec


def cpu_baseline(wl, inp, unfused=False, rot_out=None):
    """The CPU oracle, as it stands, on the whole workload (all rows), on this host."""
    import numpy as np
    import oracle
    import workloads as W
    threads = oracle.default_threads()
    x, w = W.bits(inp.x), W.bits(inp.w)
    bias = None if inp.bias is None else W.bits(inp.bias)
    fp8 = wl.kind == "fp8"
    wq, s_ch = (oracle.quantize_fp8 if fp8 else oracle.quantize_i8)(w, wl.rot_block, threads)
    # bounded sample: all rows when the whole pass is cheap enough, else a row slice
    rows = wl.M if wl.M * wl.n_w * wl.K <= 60 * 10 ** 9 else max(1, int(60 * 10 ** 9 // (wl.n_w * wl.K)))
    xs = np.ascontiguousarray(x[:rows])
    fn = {"linear": oracle.linear, "gateup": oracle.gateup_unfused if unfused else oracle.gateup_swiglu,
          "fp8": oracle.fp8_linear}[wl.kind]
    # whole passes until about 10 s of CPU time (all threads) have been spent
    passes, t0, c0 = 0, time.perf_counter(), time.process_time()
    while True:
        if rot_out is not None:   # gate/up SwiGLU whose output is quantized for the next linear
            oracle.gateup_swiglu_quant(xs, wq, s_ch, bias, wl.rot_block, rot_out, threads)
        else:
            fn(xs, wq, s_ch, bias, wl.rot_block, threads)
        passes += 1
        if time.process_time() - c0 >= 10.0 or passes >= 20:
            break
    dt, cpu = time.perf_counter() - t0, time.process_time() - c0
    ops = 2 * rows * wl.n_w * wl.K * passes
    host_cores = os.cpu_count() or 1
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "host_cores": host_cores,
            "threads": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.M} token rows, {passes} pass(es) (quantize + GEMM + epilogue), "
                      f"{dt:.2f} s wall, {cpu:.1f} s CPU on {threads} threads of a {host_cores}-core host "
                      "(the threads are the process's CPU share)"}


def mfma_peak(torch, blocks=768, launch_s=0.2):
    """Sustained MFMA rate from the register-operand probe (bench-only probe library): grow the iteration
    count until a launch takes ~50 ms, run one ~launch_s launch untimed (the clock ramps
    up under load), then time three and take the median."""
    import statistics
    import w8a8_quantized_linear_amd.probe as probe
    out = {}
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    for kind, ops_each, peak, unit in (("int8", 65536, PEAK_INT8_TOPS, "TOPS"),
                                       ("bf16", 32768, PEAK_BF16_TFLOPS, "TFLOP/s")):
        def launch_ms(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            probe.mfma_rate(kind, iters, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        iters = 256
        while (ms := launch_ms(iters)) < 50.0:
            iters *= 4
        iters = max(1, int(iters * launch_s * 1e3 / ms))
        launch_ms(iters)                                  # ramp-up, untimed
        ms = statistics.median(launch_ms(iters) for _ in range(3))
        rate = blocks * 4 * iters * 4 * ops_each / (ms * 1e-3) / 1e12
        out[kind] = {"value": rate, "unit": unit, "peak": peak, "frac": rate / peak,
                     "launch_ms": ms, "iters": iters, "blocks": blocks}
    return out


def stream_peak(torch, W, lib, names, launches=50):
    """Achievable streaming rate next to the quantizer, per activation shape: the
    bench-only streaming probe (bf16 -> one byte per element; bf16 copy) and the
    library's quantizer (packed codes), each cycling through enough input/output
    copies that the last-level cache cannot serve them, after a clock ramp; median of
    three timed runs of `launches` back-to-back launches."""
    import statistics
    import w8a8_quantized_linear_amd.probe as probe
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for name in names:
        wl = W.WORKLOADS[name]
        M, K = wl.M, wl.K
        fp8 = wl.kind == "fp8"
        x0 = W.make_inputs(wl).x.to(dev)
        copies = max(2, -(-ROTATION_BYTES // (5 * M * K)))
        xs = [x0] + [x0.clone() for _ in range(copies - 1)]
        ys = [torch.empty((2 * M * K,), dtype=torch.uint8, device=dev) for _ in range(copies)]
        qs = [torch.empty((lib.packed_bytes(M, K),), dtype=torch.uint8, device=dev) for _ in range(copies)]
        ss = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(copies)]
        qfn = lib._lib.w8a8_quantize_act_fp8_packed if fp8 else lib._lib.w8a8_quantize_act_packed

        def quantize(i):
            st = qfn(xs[i].data_ptr(), M, K, wl.rot_block, qs[i].data_ptr(), ss[i].data_ptr(), stream)
            if st != 0:
                raise RuntimeError(f"quantizer: status {st}")
        runs = {"probe_bf16_to_byte": (3 * M * K, lambda i: probe.stream("bf16_to_byte", xs[i], ys[i])),
                "probe_copy": (4 * M * K, lambda i: probe.stream("copy", xs[i], ys[i])),
                "quantizer": (3 * M * K + 4 * M, quantize)}
        t = time.perf_counter()
        i = 0
        while time.perf_counter() - t < RAMP_SECONDS:   # clock ramp, untimed
            for _, fn in runs.values():
                fn(i % copies)
            i += 1
            torch.cuda.synchronize()
        rec = {"stream_peak": name, "M": M, "K": K, "rot_block": wl.rot_block, "codes": "e4m3fn" if fp8 else "int8"}
        for key, (nbytes, fn) in runs.items():
            us = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for j in range(launches):
                    fn(j % copies)
                e1.record()
                torch.cuda.synchronize()
                us.append(e0.elapsed_time(e1) / launches * 1e3)
            u = statistics.median(us)
            rec[key] = {"us": u, "bytes": nbytes, "gbs": nbytes / u / 1e3, "frac_of_8tbs": nbytes / u / 1e3 / PEAK_HBM_GBS}
        rec["quantizer_vs_probe"] = rec["quantizer"]["gbs"] / rec["probe_bf16_to_byte"]["gbs"]
        print(json.dumps(rec), flush=True)
        del xs, ys, qs, ss, x0
        torch.cuda.empty_cache()


def lds_patterns(torch, blocks=512, iters=4096, launches=5):
    """Per-launch time of the LDS read-pattern probe (bench-only probe library) for each
    chunk placement, after an untimed launch of each; median of three timed runs."""
    import statistics
    import w8a8_quantized_linear_amd.probe as probe
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    reads = blocks * 256 * 8 * iters            # ds_read_b128 per launch, lane-wise
    rec = {"lds_patterns": {"blocks": blocks, "iters": iters, "reads_of_16_bytes": reads}}
    for name in probe.LDS_PATTERNS:
        probe.lds(name, iters, blocks, out)
        torch.cuda.synchronize()
        us = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(launches):
                probe.lds(name, iters, blocks, out)
            e1.record()
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) / launches * 1e3)
        u = statistics.median(us)
        rec[name] = {"us": u, "tb_per_s": reads * 16 / u / 1e6}
    base = rec["contiguous"]["us"]
    for name in probe.LDS_PATTERNS:
        rec[name]["time_vs_contiguous"] = rec[name]["us"] / base
    print(json.dumps(rec), flush=True)


def vendor_gemm(torch, W, lib, names, launches=20):
    """Per-launch time of the vendor GEMM and of this library's GEMM on the same codes."""
    dev = torch.device("cuda:0")

    def per_launch_us(fn):
        t = time.perf_counter()
        while time.perf_counter() - t < RAMP_SECONDS:   # clock ramp, untimed
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches * 1e3

    for name in names:
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl)
        M, K, Nw = wl.M, wl.K, wl.n_w
        fp8 = wl.kind == "fp8"
        quant = lib.w8a8_quantize_act_fp8 if fp8 else lib.w8a8_quantize_act
        q, s_tok = quant(inp.x.to(dev), wl.rot_block)
        w, s_ch = quant(inp.w.to(dev), wl.rot_block)
        qp, wp = lib.w8a8_pack_weight(q), lib.w8a8_pack_weight(w)
        ops = 2 * M * Nw * K
        rec = {"vendor_gemm": name, "M": M, "K": K, "weight_rows": Nw, "ops": ops}
        if fp8:
            a8, b8 = q.view(torch.float8_e4m3fn), w.view(torch.float8_e4m3fn)
            sa, sb = s_tok.view(M, 1).contiguous(), s_ch.view(1, Nw).contiguous()
            out = torch.empty((M, Nw), dtype=torch.bfloat16, device=dev)
            vendor = ("torch._scaled_mm (hipBLASLt), E4M3FN x E4M3FN, row-wise scales -> bf16",
                      lambda: torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16))
            ours = [("library", ("w8a8_fp8_gemm_dequant_packed (bf16 output)",
                                 lambda: lib.w8a8_fp8_gemm_dequant_packed(qp, s_tok, wp, s_ch, K, out=out)))]
        else:
            acc = torch.empty((M, Nw), dtype=torch.int32, device=dev)
            out = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
            gemm = lib.w8a8_gemm_swiglu_packed if wl.kind == "gateup" else lib.w8a8_gemm_dequant_packed
            vendor = ("torch._int_mm (hipBLASLt), int8 x int8 -> int32", lambda: torch._int_mm(q, w.t()))
            ours = [("library_i32", ("w8a8_gemm_i32_packed (int32 output, as the vendor call)",
                                     lambda: lib.w8a8_gemm_i32_packed(qp, wp, M, Nw, K, out=acc))),
                    ("library", (f"{gemm.__name__} (the path's GEMM: fused epilogue, bf16 output)",
                                 lambda: gemm(qp, s_tok, wp, s_ch, K, out=out)))]
        for key, (what, fn) in [("vendor", vendor)] + ours:
            try:
                us = per_launch_us(fn)
                rec[key] = {"call": what, "us_per_launch": us, "tops": ops / us / 1e6}
            except Exception as e:   # a library without the kernel on this build: say so
                rec[key] = {"call": what, "error": repr(e)[:200]}
        print(json.dumps(rec), flush=True)
        del q, w, qp, wp
        torch.cuda.empty_cache()


def traffic_key(workload: str, path: str) -> str:
    """Name of the stored counter record of a workload's GEMM on a bench path."""
    return workload + ("-unfused" if path == "unfused" else "") + ("-swiglu-quant" if path == "swiglu-quant" else "")


def main():
    args = parse()
    if args.pmc_summary:
        key = traffic_key(args.workload, args.path)
        rec = pmc_summary(key, *args.pmc_summary)
        out = ROOT / "profiles" / f"traffic_{key}.json"
        out.write_text(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(across GPUs the projection would shard by token rows, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import w8a8_quantized_linear_amd as lib

    if args.mfma_peak:
        print(json.dumps({"mfma_peak": mfma_peak(torch)}))
        return
    if args.vendor_gemm:
        vendor_gemm(torch, W, lib, [n for n in W.ORDER if W.WORKLOADS[n].M >= 2048])
        return
    if args.stream_peak:
        stream_peak(torch, W, lib, [n for n in W.ORDER if W.WORKLOADS[n].M >= 2048])
        return
    if args.lds_patterns:
        lds_patterns(torch)
        return
    if args.drift:
        import numpy as np
        from w8a8_quantized_linear_amd.drift import drift
        for name in W.ORDER:
            wl = W.WORKLOADS[name]
            inp = W.make_inputs(wl)
            rng = np.random.default_rng(wl.seed)
            rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, size=min(wl.M, 62), replace=False)]))
            t0 = time.perf_counter()
            d = drift(inp.x, inp.w, inp.bias, wl.kind, (0, 128), rows)
            print(json.dumps({"drift": "relative L2 vs fp64 unquantized projection", "workload": name,
                              "kind": wl.kind, "workload_rot_block": wl.rot_block,
                              "rows_compared": int(len(rows)),
                              "rel_l2": {str(k): v for k, v in d.items()},
                              "seconds": round(time.perf_counter() - t0, 2)}), flush=True)
        return

    wl = W.WORKLOADS[args.workload]
    if args.shard > 1:
        import dataclasses
        P = args.shard
        if wl.kind == "gateup":
            if wl.N % (8 * P):
                print(f"bench.py: N = {wl.N} does not split into {P} column shards of a multiple of 8",
                      file=sys.stderr)
                sys.exit(2)
            wl = dataclasses.replace(wl, N=wl.N // P, name=f"{wl.name}-columns-1of{P}")
        else:
            wl = dataclasses.replace(wl, M=-(-wl.M // P), name=f"{wl.name}-rows-1of{P}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # untimed elementwise kernel of known size (reads and writes CALIBRATION_BYTES):
    # the reference the HBM byte counters are scaled by
    calib_src = torch.zeros(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.add(calib_src, 1.0, out=calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst
    unfused = args.path == "unfused"
    single = args.path == "single"
    quantout = args.path == "swiglu-quant"
    if (unfused or quantout) and wl.kind != "gateup":
        print(f"bench.py: --path {args.path} applies to gate/up workloads only", file=sys.stderr)
        sys.exit(2)
    if single and wl.kind == "fp8":
        print("bench.py: --path single applies to int8 workloads only", file=sys.stderr)
        sys.exit(2)
    inp = W.make_inputs(wl)
    fp8 = wl.kind == "fp8"
    quant = lib.w8a8_quantize_act_fp8 if fp8 else lib.w8a8_quantize_act
    M, K, Nw = wl.M, wl.K, wl.n_w
    n_out = wl.N

    # resident operands, several copies so that consecutive steps do not hit in cache
    x0 = inp.x.to(dev)
    wq_rows, s_ch0 = quant(inp.w.to(dev), wl.rot_block)
    wq0 = lib.w8a8_pack_weight(wq_rows)       # load-time packing, outside the timed region
    del wq_rows
    bias0 = None if inp.bias is None else inp.bias.to(dev)
    per_copy = M * K * 2 + Nw * K + M * K + M * n_out * 2 + 4 * (M + Nw)
    copies = max(2, -(-ROTATION_BYTES // per_copy))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
    qs = [torch.empty((lib.packed_bytes(M, K),), dtype=torch.uint8 if fp8 else torch.int8, device=dev)
          for _ in range(copies)]
    ss = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(copies)]
    ys = [torch.empty((M, n_out), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    # unfused: the bf16 gate/up projection [M, 2N] between the GEMM and the SwiGLU pass
    hs = [torch.empty((M, Nw), dtype=torch.bfloat16, device=dev) for _ in range(copies)] if unfused else []
    # swiglu-quant: the next linear's input codes (packed) + scales
    if quantout:
        cs = [torch.empty((lib.packed_bytes(M, n_out),), dtype=torch.int8, device=dev) for _ in range(copies)]
        s2 = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    L = lib._lib
    stream = torch.cuda.current_stream().cuda_stream
    qfn = L.w8a8_quantize_act_fp8_packed if fp8 else L.w8a8_quantize_act_packed
    gfn = {"linear": L.w8a8_gemm_dequant_packed, "gateup": L.w8a8_gemm_swiglu_packed,
           "fp8": L.w8a8_fp8_gemm_dequant_packed}[wl.kind]
    bptr = None if bias0 is None else bias0.data_ptr()
    sch = s_ch0.data_ptr()
    qargs = [(xs[i].data_ptr(), M, K, wl.rot_block, qs[i].data_ptr(), ss[i].data_ptr(), stream)
             for i in range(copies)]
    if unfused:
        gfn = L.w8a8_gemm_dequant_packed
        gargs = [(qs[i].data_ptr(), ss[i].data_ptr(), wqs[i].data_ptr(), sch, bptr, hs[i].data_ptr(),
                  M, Nw, K, stream) for i in range(copies)]
        sargs = [(hs[i].data_ptr(), hs[i].data_ptr() + 2 * n_out, Nw, ys[i].data_ptr(), M, n_out, stream)
                 for i in range(copies)]
    else:
        gargs = [(qs[i].data_ptr(), ss[i].data_ptr(), wqs[i].data_ptr(), sch, bptr, ys[i].data_ptr(),
                  M, n_out, K, stream) for i in range(copies)]
    # calls[c]: the library calls of one step on operand copy c, in order
    calls = [[(qfn, qargs[i]), (gfn, gargs[i])] for i in range(copies)]
    if unfused:
        for i in range(copies):
            calls[i].append((L.w8a8_swiglu, sargs[i]))
    if single:
        wsz = lib.workspace_bytes(M, K)
        wss = [torch.empty((wsz,), dtype=torch.uint8, device=dev) for _ in range(copies)]
        pfn = L.w8a8_linear_packed if wl.kind == "linear" else L.w8a8_gateup_swiglu_packed
        calls = [[(pfn, (xs[i].data_ptr(), wqs[i].data_ptr(), sch, bptr, ys[i].data_ptr(), M, n_out, K,
                         wl.rot_block, wss[i].data_ptr(), wsz, stream))] for i in range(copies)]
    if quantout:   # the kernels w8a8_gateup_swiglu_quant_packed enqueues, h in ys
        for i in range(copies):
            calls[i].append((L.w8a8_quantize_act_packed,
                             (ys[i].data_ptr(), M, n_out, args.rot_out, cs[i].data_ptr(), s2[i].data_ptr(),
                              stream)))
    def step(i):
        st = 0
        for fn, a in calls[i % copies]:
            st |= fn(*a)
        if st:
            raise RuntimeError(f"library call failed with status {st}")

    # clock ramp: untimed steps for about RAMP_SECONDS, whatever the warmup count
    t_r, ramp = time.perf_counter(), 0
    while time.perf_counter() - t_r < RAMP_SECONDS:
        for _ in range(8):
            step(ramp)
            ramp += 1
        torch.cuda.synchronize()
    if args.warmup is not None:
        warmup = args.warmup
        for i in range(warmup):
            step(i)
    else:
        # 40 steps, the last 20 timed to estimate a step, then enough more to fill ~0.25 s
        for i in range(20):
            step(i)
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        for i in range(20, 40):
            step(i)
        torch.cuda.synchronize()
        per_step = max((time.perf_counter() - t_w) / 20, 1e-6)
        warmup = 40 + int(WARMUP_SECONDS / per_step)
        for i in range(40, warmup):
            step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, nothing else enqueued between the kernels.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Per-kernel durations: each library call of the step on its own, its K
    # launches of the timed steps (same operand copies, same order) back to back
    # on the launch stream between two HIP events.  (An event recorded between
    # the kernels of a step is a command-processor packet that idles the GPU for
    # a few microseconds, so per-kernel figures get passes of their own.)
    per_call = []
    for j in range(len(calls[0])):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        st = 0
        for i in range(args.steps):
            fn, a = calls[i % copies][j]
            st |= fn(*a)
        e1.record()
        torch.cuda.synchronize()
        if st:
            raise RuntimeError(f"library call failed with status {st}")
        per_call.append(e0.elapsed_time(e1) / args.steps * 1e-3)

    def avg(j):  # s per launch of call j
        return per_call[j]
    tq = avg(0)                       # quantizer (or the single whole-path call)
    tg = avg(1) if not single else tq  # GEMM
    ms_per_step = wall / args.steps * 1e3
    ops = 2 * M * Nw * K
    q_bytes = 2 * M * K + M * K + 4 * M                      # read bf16 x, write codes + scales
    out_cols = Nw if unfused else n_out                      # the unfused GEMM writes [M, 2N]
    out_bytes = M * out_cols * 2                             # bf16 output
    g_bytes = M * K + Nw * K + 4 * (M + Nw) + out_bytes + (0 if bias0 is None else 2 * Nw)
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_INT8_TOPS
    # (a stored record covers the GEMM kernel alone, not the single whole-path call)
    traffic = None if single else stored_traffic(traffic_key(wl.name, args.path))
    q_traffic = None if single else stored_traffic(traffic_key(wl.name, args.path), "quantizer")

    out = {
        "metric": "W8A8 linear TOPS incl. quant+dequant, % int8 MFMA peak; quantizer GB/s",
        "value": ops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "i8",
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": wl.name, "M": M, "K": K, "N": n_out, "weight_rows": Nw,
                   "rot_block": wl.rot_block,
                   "path": wl.kind + ("-unfused" if unfused else "") + ("-single-call" if single else "")
                   + (f"-{args.path}-rot{args.rot_out}" if quantout else ""),
                   "parallelism": "single GPU" if args.shard == 1 else
                   f"one GPU's share of {args.shard} ({'gate/up columns' if wl.kind == 'gateup' else 'token rows'})",
                   "operand_copies": copies, "clock_ramp_steps": ramp},
        "pct_of_peak": 100.0 * ops / (ms_per_step * 1e-3) / (peak * 1e12),
        "roofline": {"bound": "mfma", "achieved": ops / tg / 1e12, "peak": peak, "unit": "TFLOP/s",
                     "frac": ops / tg / 1e12 / peak, "traffic": traffic,
                     "kernel": "gemm_persist / gemm_tile (GEMM + fused epilogue)", "avg_launch_us": tg * 1e6,
                     "algorithmic_bytes": g_bytes},
        "quantizer": {"bound": "hbm", "achieved": q_bytes / tq / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": q_bytes / tq / 1e9 / PEAK_HBM_GBS, "avg_launch_us": tq * 1e6,
                      "algorithmic_bytes": q_bytes, "traffic": q_traffic},
    }
    if single:
        del out["quantizer"]
        out["roofline"]["kernel"] = ("whole-path call: one kernel (quantizer + GEMM + epilogue) for "
                                     "short batches, else the quantizer and the GEMM")
        out["roofline"]["algorithmic_bytes"] = q_bytes + g_bytes - M * K - 4 * M   # codes not re-read
    if unfused:
        tsw = avg(2)
        sw_bytes = 6 * M * n_out                             # read gate + up, write y (bf16)
        out["swiglu"] = {"bound": "hbm", "achieved": sw_bytes / tsw / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": sw_bytes / tsw / 1e9 / PEAK_HBM_GBS,
                         "avg_launch_us": tsw * 1e6, "algorithmic_bytes": sw_bytes}
        out["roofline"]["kernel"] = "gemm_persist / gemm_tile (GEMM + dequant epilogue onto 2N columns)"
    if quantout:
        th = avg(2)
        qh_bytes = 2 * M * n_out + M * n_out + 4 * M
        out["quantizer_h"] = {"bound": "hbm", "achieved": qh_bytes / th / 1e9, "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": qh_bytes / th / 1e9 / PEAK_HBM_GBS,
                              "avg_launch_us": th * 1e6, "algorithmic_bytes": qh_bytes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, unfused, args.rot_out if quantout else None)
    out["context_h100"] = H100_CONTEXT
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
