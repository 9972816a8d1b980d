"""Throughput of the fused GEMM + ReLU on one MI355X.

One step = one gemm_relu call (every stage of the hot path: tile rasterisation,
global->LDS pipeline, MFMA contraction, ReLU, convert, store) over inputs
already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                    [--workload NAME] [--no-cpu-baseline]

Before the W counted warm-up calls, calls of the same step run untimed for at
least MS milliseconds (default 300; the line reports how many as
settle.calls): the chip's power-managed clock falls within 0.2 s of idling
and takes 50-100 ms of load to recover, so without it a short warm-up after
the host-side input generation times the clock ramp, not the kernel.
    python bench.py --table      # one JSON line per workload (warm and cold L2/MALL)
    python bench.py --vendor     # the vendor GEMM (+ a separate ReLU) beside it, per workload

Default workload: fp16 GEMM+ReLU at M = N = K = 8192 (row-major A and B,
uniform[-1, 1] inputs from a fixed seed, fp32 accumulation, fp16 output) — the
shape of the pages' headline GEMM figure.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_TFLOPS_F16 = 2516.6      # MI355X dense fp16/bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_TFLOPS_F8 = 5033.2       # MI355X dense fp8 MFMA: 256 CU x 8192 flop/clk x 2.4 GHz
PEAK_TFLOPS_F4 = 10066.3      # MI355X dense fp4 / fp6 MFMA: 256 CU x 16384 flop/clk x 2.4 GHz
HBM_GBPS = 8000.0
METRIC = "TFLOP/s and % of MI355X fp16 MFMA peak, fp16 GEMM+ReLU 8192³"
KERNEL_SOURCES = ["dense_tiled_gemm_relu_amd/csrc/gemm_relu_kernel.hpp",
                  "dense_tiled_gemm_relu_amd/csrc/configs.hpp",
                  "dense_tiled_gemm_relu_amd/csrc/gemm_relu_api.hip",
                  "dense_tiled_gemm_relu_amd/csrc/inst_i16.hip"]


def _code_only(text):
    """Source text without comments and blank space: a comment edit does not
    change the kernel a counter summary was taken on."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


HBM_PEAK_GBS = 8000.0      # MI355X HBM3E


def roofline(flops, nbytes, kernel_ms, peak_tflops, traffic):
    """The roofline record of one launch: MFMA-bound when the algorithmic
    intensity (flops per algorithmic byte) is above the ridge point of the input
    type's peak and 8 TB/s, HBM-bound below it (achieved = algorithmic bytes per
    launch over the launch's duration)."""
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9)
    rec = {"intensity": round(flops / nbytes, 1), "ridge": round(ridge, 1)}
    if flops / nbytes >= ridge:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        rec.update(bound="mfma", achieved=round(achieved, 2), peak=peak_tflops, unit="TFLOP/s",
                   frac=round(achieved / peak_tflops, 4))
    else:
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
        rec.update(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                   frac=round(achieved / HBM_PEAK_GBS, 4))
    rec.update(traffic=traffic, algorithmic_bytes=int(nbytes), kernel_ms=round(kernel_ms, 5))
    return rec


def measured_traffic(workload, launches_per_record=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def measured_cycles(workload):
    """Shader-clock cycles per launch (GRBM_GUI_ACTIVE of one XCD) from the
    committed counter summary, if it was taken on the current kernel sources;
    else None.  A launch takes the same number of cycles at any clock (measured:
    the same count for 930 us and 797 us dispatches), so cycles / duration is
    the clock the launch ran at."""
    path = os.path.join(ROOT, "profiles", "cycles_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("cycles_per_launch")


def ingest_cycles(workload, pmc_dir):
    """GRBM_GUI_ACTIVE per launch of the GEMM kernel (sum of the XCD rows / 8)
    and the launch durations from one rocprofv3 --pmc GRBM_GUI_ACTIVE
    --kernel-trace run -> profiles/cycles_<workload>.json, stamped with the
    kernel source hash."""
    import csv
    import glob
    g = _pmc_per_dispatch(pmc_dir, "GRBM_GUI_ACTIVE", "gemm_relu_kernel")
    dur = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "gemm_relu_kernel" in r["Kernel_Name"]:
                dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    d = [dur[k] for k in sorted(dur)]
    per_xcd = [x / 8.0 for x in g]
    cyc = sorted(per_xcd)[len(per_xcd) // 2]
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "cycles_per_launch": int(cyc), "launches": len(per_xcd),
           "cycles_min": int(min(per_xcd)), "cycles_max": int(max(per_xcd))}
    if len(d) == len(per_xcd):
        mhz = [c / t / 1e6 for c, t in zip(per_xcd, d)]
        rec.update(clock_mhz_first=round(mhz[0]), clock_mhz_last=round(mhz[-1]),
                   duration_us_first=round(d[0] * 1e6, 1), duration_us_last=round(d[-1] * 1e6, 1))
    path = os.path.join(ROOT, "profiles", "cycles_%s.json" % workload)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


COPY_BYTES = 256 * 1024 * 1024


def calibrate_copy():
    """Three plain device copies of COPY_BYTES (torch copy_), for scaling the
    FETCH_SIZE / WRITE_SIZE counters: the copy reads and writes exactly
    COPY_BYTES per dispatch."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copied %d bytes x 3" % COPY_BYTES)


def _pmc_per_dispatch(csv_dir, counter, kernel_substr):
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no %s rows for %s under %s" % (counter, kernel_substr, csv_dir))
    v = sorted(vals.items(), key=lambda kv: int(kv[0]))
    return [x for _, x in v]


def ingest_traffic(workload, fetch_dir, write_dir, copyf_dir, copyw_dir):
    """HBM bytes per launch of the GEMM kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain copy of COPY_BYTES.  Writes
    profiles/traffic_<workload>.json stamped with the kernel source hash."""
    f = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", "gemm_relu_kernel")[1:]   # drop first (cold)
    w = _pmc_per_dispatch(write_dir, "WRITE_SIZE", "gemm_relu_kernel")[1:]
    cf = _pmc_per_dispatch(copyf_dir, "FETCH_SIZE", "copyBuffer")
    cw = _pmc_per_dispatch(copyw_dir, "WRITE_SIZE", "copyBuffer")
    kib = 1024.0
    fetch_scale = COPY_BYTES / (sum(cf) / len(cf) * kib)
    write_scale = COPY_BYTES / (sum(cw) / len(cw) * kib)
    fetch = sum(f) / len(f) * kib * fetch_scale
    write = sum(w) / len(w) * kib * write_scale
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
           "hbm_bytes_per_launch": int(fetch + write),
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "raw_fetch_kib": [round(x) for x in f], "raw_write_kib": [round(x) for x in w]}
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w, A, B, target_s=15.0):
    """The oracle, untuned, on a bounded sample of the same workload: the first
    R rows of A against all of B (R x N x K multiply-adds), R sized so the run
    takes about target_s seconds on this host's cores."""
    import oracle
    M, N, K, ic, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["transB"]
    rows_a = A.reshape(M, K)
    # The fixed cost (decoding all of B) hides the per-row cost in a short run,
    # so grow the row count until one run lasts at least ~60% of target_s.
    R = min(M, 16)
    for _ in range(5):
        t = time.perf_counter()
        _, threads = oracle.gemm_relu_ref(rows_a[:R], B, R, N, K, ic, tb, return_threads=True)
        dt = time.perf_counter() - t
        if dt >= 0.6 * target_s or R >= M:
            break
        R = int(min(M, max(R + 1, R * target_s / max(dt, 1e-3))))
    flops = 2.0 * R * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "cpu_model": host_cpu()[0], "kind": "oracle",
            "sample": "rows 0..%d of A (%d x %d x %d multiply-adds of the %s workload, "
                      "binary64), %.2f s wall" % (R - 1, R, N, K, w["name"], dt)}


def cpu_baseline_mx(w, target_s=15.0):
    """The block-scaled oracle on the first R rows of A against all of B."""
    import oracle
    M, N, K, fmt = w["M"], w["N"], w["K"], w["in_dtype"]
    A, SA, B, SB = wl.mx_inputs(M, N, K, fmt, w["index"], w["dist"])
    R = 1
    for _ in range(6):
        rows = np.repeat(np.arange(R), N)
        cols = np.tile(np.arange(N), R)
        t = time.perf_counter()
        oracle.gemm_relu_mx_ref(A, SA, B, SB, M, N, K, fmt, rows=rows, cols=cols)
        dt = time.perf_counter() - t
        if dt >= 0.6 * target_s or R >= M:
            break
        R = int(min(M, max(R + 1, R * target_s / max(dt, 1e-3))))
    flops = 2.0 * R * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count())),
            "cpu_model": host_cpu()[0], "kind": "oracle",
            "sample": "rows 0..%d of A (%d x %d x %d block-scaled multiply-adds of the %s "
                      "workload, binary64), %.2f s wall" % (R - 1, R, N, K, w["name"], dt)}


def cpu_baseline_sp(w, target_s=15.0):
    """The 2:4 sparse oracle on the first R rows of A against all of B
    (dense-equivalent flops, as the GPU figure)."""
    import oracle
    M, N, K, ic, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["transB"]
    As, E, B = wl.sp_inputs(M, N, K, ic, tb, w["index"])
    R = 1
    for _ in range(6):
        rows = np.repeat(np.arange(R), N)
        cols = np.tile(np.arange(N), R)
        t = time.perf_counter()
        oracle.gemm_relu_sp_ref(As, E, B, M, N, K, ic, tb, rows=rows, cols=cols)
        dt = time.perf_counter() - t
        if dt >= 0.6 * target_s or R >= M:
            break
        R = int(min(M, max(R + 1, R * target_s / max(dt, 1e-3))))
    flops = 2.0 * R * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count())),
            "cpu_model": host_cpu()[0], "kind": "oracle",
            "sample": "rows 0..%d of A (%d x %d x %d dense-equivalent multiply-adds of the %s "
                      "workload, binary64), %.2f s wall" % (R - 1, R, N, K, w["name"], dt)}


def host_cpu():
    """(model name, logical CPUs this process may run on) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_table(names=None):
    """The oracle, untuned, over the whole of each plain workload (every output
    element), once on all host threads (OMP_NUM_THREADS if set) and, for the two smallest
    square workloads, once on one thread: one JSON line per run.  A CPU
    baseline for the GPU figures, not a target."""
    import oracle
    model, ncpu = host_cpu()
    # explicit counts: a one-thread run leaves OpenMP's default at one thread
    all_threads = int(os.environ.get("OMP_NUM_THREADS") or ncpu)
    order = sorted(wl.WORKLOADS, key=lambda n: wl.WORKLOADS[n]["index"])
    names = names or [n for n in order if not (wl.WORKLOADS[n].get("mx") or
                                                wl.WORKLOADS[n].get("sparse") or
                                                wl.WORKLOADS[n]["in_dtype"] in wl.FP8)]
    for name in names:
        w = wl.WORKLOADS[name]
        M, N, K, ic, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["transB"]
        A, B = wl.workload_inputs(name)
        runs = [all_threads] + ([1] if name in ("gemm_relu_f16_256", "gemm_relu_f16_4096") else [])
        for threads in runs:
            t = time.perf_counter()
            _, used = oracle.gemm_relu_ref(A, B, M, N, K, ic, tb, threads=threads,
                                           return_threads=True)
            dt = time.perf_counter() - t
            rec = {"workload": name, "M": M, "N": N, "K": K, "threads": int(used),
                   "oracle_s": round(dt, 6), "oracle_gflops": round(2.0 * M * N * K / dt / 1e9, 3),
                   "host_cpu": model, "host_cpus": ncpu}
            print(json.dumps(rec), flush=True)


def peak_tflops(in_dtype, sparse=False):
    if sparse:
        return PEAK_TFLOPS_F16_SPARSE
    if in_dtype == wl.MX_E2M1:
        return PEAK_TFLOPS_F4
    if in_dtype in wl.FP8 or in_dtype in (wl.MX_E4M3, wl.MX_E5M2):
        return PEAK_TFLOPS_F8
    return PEAK_TFLOPS_F16


PEAK_TFLOPS_F16_SPARSE = 2 * PEAK_TFLOPS_F16   # 2:4 sparse fp16/bf16, dense-equivalent flops


def ceiling_kind(in_dtype, sparse=False, plan=None):
    """probe_mfma_rate kind matching an input type and tile configuration: 0
    fp16 32x32x16, 1 E4M3, 2 E2M1 (scaled MFMA), 3 E4M3 on the scaled MFMA, 4
    the 2:4 sparse fp16 form, 5 fp16 16x16x32 (the 16x16-block tiles)."""
    if sparse:
        return 4
    if plan is not None and ("_i16" in plan or plan.endswith("_16")):
        return 5
    if in_dtype == wl.MX_E2M1:
        return 2
    if in_dtype in (wl.MX_E4M3, wl.MX_E5M2):
        return 3
    return 1 if in_dtype in wl.FP8 else 0


def workload_call(gr, name, stream, workspace=False):
    """(call, C tensor, tile config, algorithmic bytes) for one workload, its
    inputs uploaded: plain ones through gemm_relu (through gemm_relu_ws with a
    zeroed workspace of gemm_relu_workspace_size bytes when `workspace`),
    block-scaled ones through gemm_relu_mx."""
    import torch
    w = wl.WORKLOADS[name]
    M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
    Cd = torch.empty((M, N), dtype=torch_dtype(oc), device="cuda")
    if w.get("mx"):
        arrs = wl.mx_inputs(M, N, K, ic, w["index"], w["dist"])
        Ad, SAd, Bd, SBd = (torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda() for x in arrs)

        def call():
            gr.gemm_relu_mx(Ad, SAd, Bd, SBd, Cd, M, N, K, ic, oc, stream)
        plan = gr.gemm_relu_mx_plan(Ad, SAd, Bd, SBd, Cd, M, N, K, ic, oc)
        nbytes = sum(int(x.size) for x in arrs) + M * N * wl.elem_bytes(oc)
        return call, Cd, plan, nbytes, (Ad, SAd, Bd, SBd)
    if w.get("sparse"):
        As, E, B = wl.sp_inputs(M, N, K, ic, tb, w["index"])
        Ad = to_device(As, ic, (M, K // 2))
        Ed = torch.from_numpy(E).cuda()
        Bd = to_device(B, ic, wl.b_shape(M, N, K, tb))

        def call():
            gr.gemm_relu_sp(Ad, Ed, Bd, Cd, M, N, K, ic, oc, tb, stream)
        plan = gr.gemm_relu_sp_plan(Ad, Ed, Bd, Cd, M, N, K, ic, oc, tb)
        nbytes = 2 * (M * K // 2 + K * N) + E.size + M * N * wl.elem_bytes(oc)
        return call, Cd, plan, nbytes, (Ad, Ed, Bd)
    A, B = wl.workload_inputs(name)
    Ad = to_device(A, ic, (M, K))
    Bd = to_device(B, ic, wl.b_shape(M, N, K, tb))
    nbytes = wl.elem_bytes(ic) * (M * K + K * N) + M * N * wl.elem_bytes(oc)
    if workspace:
        need = gr.gemm_relu_workspace_size(M, N, K, ic, oc, tb)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")

        def call():
            gr.gemm_relu_ws(Ad, Bd, Cd, M, N, K, ic, oc, tb, ws, need, stream)
        plan = gr.gemm_relu_ws_plan(Ad, Bd, Cd, M, N, K, ic, oc, tb, ws, need)
        return call, Cd, plan, nbytes, (Ad, Bd, ws)

    def call():
        gr.gemm_relu(Ad, Bd, Cd, M, N, K, ic, oc, tb, stream)
    plan = gr.gemm_relu_plan(Ad, Bd, Cd, M, N, K, ic, oc, tb)
    return call, Cd, plan, nbytes, (Ad, Bd)


def torch_dtype(code):
    import torch
    return {wl.F16: torch.float16, wl.BF16: torch.bfloat16, wl.F32: torch.float32,
            wl.F8E4M3: torch.float8_e4m3fn, wl.F8E5M2: torch.float8_e5m2}[code]


def to_device(bits, code, shape):
    """Storage patterns (uint16 or uint8) -> a CUDA tensor of the input type."""
    import torch
    bits = np.ascontiguousarray(bits).reshape(shape)
    raw = bits.view(np.uint8) if code in wl.FP8 else bits.view(np.int16)
    return torch.from_numpy(raw).cuda().view(torch_dtype(code))


def mfma_ceiling(gr, stream, blocks=1024, steps=2048, kind=0):
    """MFMA-only throughput on random operands with no memory traffic (the probe
    library's probe_mfma_rate: 4 waves per CU, each streaming the 32 MFMAs of
    one step of a 128x128 wave tile; kind 0: fp16 32x32x16, 1: E4M3 32x32x64,
    2: E2M1 32x32x64 on the scaled MFMA with unit scales, 3: E4M3 on the scaled
    MFMA, 4: the 2:4 sparse fp16 32x32x32 form, counted at its dense-equivalent
    flops; 5: fp16 16x16x32, the same step as 64 MFMAs).  The chip is
    power-limited, so this, not 2.4 GHz x the instruction rate, is what the
    contraction step alone can reach on this machine now.  None if the probe
    library is not built."""
    import ctypes
    import torch
    if not os.path.exists(gr.PROBE_LIB_PATH):
        return None
    lib = ctypes.CDLL(gr.PROBE_LIB_PATH)
    lib.probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    if kind == 2:                               # random E2M1 nibbles, 16 bytes per lane
        src = torch.randint(0, 256, (blocks * 8 * 256 * 16,), dtype=torch.uint8, device="cuda")
    else:
        per_lane = {1: 32, 3: 32, 4: 16}.get(kind, 8)   # operand elements per lane
        src = torch.empty(blocks * 8 * 256 * per_lane, dtype=torch.float32, device="cuda")
        src = src.uniform_(-1, 1).to(torch.float8_e4m3fn if kind in (1, 3) else torch.float16)
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    st = stream.cuda_stream

    def run(n):
        rc = lib.probe_mfma_rate(src.data_ptr(), src.numel() * src.element_size(), out.data_ptr(),
                                 ticks.data_ptr(), blocks, n, kind, st)
        if rc != 0:
            raise RuntimeError("probe_mfma_rate failed: %d" % rc)

    run(steps // 8)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run(steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) * 1e-3
    t = ticks.view(blocks, 2).double()
    cycles = t[:, 0].mean().item()
    clock_mhz = (t[:, 0] / t[:, 1]).mean().item() * 100.0
    # flops of one 128x128x32 (fp16) or 128x128x128 (8-bit) wave step, per wave and step
    flops = blocks * 4 * steps * 32 * (32 * 32 * {0: 16, 4: 32, 5: 16}.get(kind, 64) * 2)
    mfmas = steps * 32 * (2 if kind == 5 else 1)    # kind 5: 16x16x32, half the MACs each
    return {"tflops": round(flops / sec / 1e12, 1), "clock_mhz": round(clock_mhz),
            "cycles_per_mfma": round(cycles / mfmas, 2),
            "kind": "MFMA-only, random %s operands, no memory traffic (probe_mfma_rate)"
                    % ("fp16", "E4M3", "E2M1 (unit block scales)", "E4M3 (unit block scales)",
                       "fp16, 2:4 sparse (dense-equivalent flops)", "fp16, 16x16x32 form")[kind]}


TABLE_WARMUP_S = 0.5


def table(gr):
    """One JSON line per workload: median per-call kernel time over 5 trials of
    20 back-to-back calls (HIP events on the launch stream, after at least 10
    and at least TABLE_WARMUP_S seconds of warm-up calls),
    and a cold-cache time (each sample after a 512 MiB read that evicts the
    256 MiB MALL and the L2s).  A kernel that follows an event record starts
    some microseconds later than one that follows another kernel, so the cold
    time is a difference: events around [a one-block fill kernel, the call]
    less events around the fill kernel alone, medians of 20 samples each (the
    single-call event time is reported beside it).  Plain workloads for which
    gemm_relu_ws splits K get a second line, timed through it."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    # cache eviction for the cold times: a READ of 512 MiB, which leaves the
    # 256 MiB MALL and the L2s holding clean lines of another buffer.  (Writing
    # it instead leaves them dirty, and the timed kernel's misses then pay for
    # their write-back: measured on the skinny 64x8192x8192 workload, 58 us
    # after a 512 MiB write against 43 us after a 512 MiB read; a plain
    # 134 MB streaming read, 52 against 26 us.)
    flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    ceilings = {k: mfma_ceiling(gr, stream, kind=k) for k in (0, 1, 2, 3, 4, 5)}
    print(json.dumps({"mfma_ceiling": ceilings[0], "mfma_ceiling_fp8": ceilings[1],
                      "mfma_ceiling_mxfp4": ceilings[2], "mfma_ceiling_mxfp8": ceilings[3],
                      "mfma_ceiling_sparse_f16": ceilings[4], "mfma_ceiling_f16_16x16": ceilings[5]}),
          flush=True)
    tiny = torch.zeros(64, dtype=torch.float32, device="cuda")

    def cold_sample(fn):
        torch.sum(flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tiny.fill_(1.0)
        if fn is not None:
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    runs = []
    for name in sorted(wl.WORKLOADS, key=lambda n: wl.WORKLOADS[n]["index"]):
        w = wl.WORKLOADS[name]
        runs.append((name, False))
        if not w.get("mx") and not w.get("sparse") and gr.gemm_relu_workspace_size(
                w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]) > 0:
            runs.append((name, True))
    for name, with_ws in runs:
        w = wl.WORKLOADS[name]
        M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
        call, Cd, plan, nbytes, keep = workload_call(gr, name, stream, workspace=with_ws)
        ceiling = ceilings[ceiling_kind(ic, w.get("sparse", False), plan)]
        peak = peak_tflops(ic, w.get("sparse", False))

        # warm-up by time, not by count: the power-limited clock takes tens of
        # milliseconds to settle, far longer than 10 calls of a small workload
        n, t_end = 0, time.perf_counter() + TABLE_WARMUP_S
        while n < 10 or time.perf_counter() < t_end:
            call()
            n += 1
            if n % 10 == 0:
                torch.cuda.synchronize()
        trials = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            trials.append(e0.elapsed_time(e1) * 1e3 / 20)
        with_call, fill_only, raw = [], [], []
        for i in range(20):
            with_call.append(cold_sample(call))
            fill_only.append(cold_sample(None))
            torch.sum(flush)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            raw.append(e0.elapsed_time(e1) * 1e3)
        t = statistics.median(trials)
        tc = statistics.median(with_call) - statistics.median(fill_only)
        flops = 2.0 * M * N * K
        print(json.dumps({
            "workload": name, "M": M, "N": N, "K": K, "in": wl.DTYPE_NAMES[ic],
            "out": wl.DTYPE_NAMES[oc], "transB": tb,
            "entry": "gemm_relu_ws" if with_ws else "gemm_relu",
            "tile_config": plan,
            "t_median_us": round(t, 2), "t_trials_us": [round(x, 2) for x in trials],
            "tflops": round(flops / t / 1e6, 1),
            "pct_peak": round(100 * flops / t / 1e6 / peak, 2), "peak_tflops": peak,
            "pct_of_mfma_ceiling": (round(100 * flops / t / 1e6 / ceiling["tflops"], 1)
                                    if ceiling else None),
            "algorithmic_GBps": round(nbytes / t / 1e3, 1),
            "pct_hbm": round(100 * nbytes / t / 1e3 / HBM_GBPS, 2),
            "t_cold_median_us": round(tc, 2), "tflops_cold": round(flops / tc / 1e6, 1),
            "cold_GBps": round(nbytes / tc / 1e3, 1), "pct_hbm_cold": round(100 * nbytes / tc / 1e3 / HBM_GBPS, 2),
            "t_cold_single_event_us": round(statistics.median(raw), 2)}),
            flush=True)
        del keep, Cd


def profile_workloads(gr, calls):
    """`calls` synchronised calls of each workload in index order, nothing else
    on the GPU in between: the dispatch list a counter run attributes to
    workloads (printed as JSON, one line per workload)."""
    import torch
    stream = torch.cuda.current_stream()
    for name in sorted(wl.WORKLOADS, key=lambda n: wl.WORKLOADS[n]["index"]):
        call, Cd, plan, nbytes, keep = workload_call(gr, name, stream)
        torch.cuda.synchronize()
        for _ in range(calls):
            call()
            torch.cuda.synchronize()
        print(json.dumps({"workload": name, "tile_config": plan, "calls": calls}), flush=True)
        del keep, Cd


def vendor(gr):
    """Context for the fused kernel: each plain (not block-scaled, not sparse)
    workload timed through the vendor GEMM (torch.mm / torch._scaled_mm, which
    dispatch to hipBLASLt on this image) without and with a separate ReLU, and
    through gemm_relu, on the same resident inputs in the same process; one JSON
    line per workload.  The three are warmed up together for at least
    TABLE_WARMUP_S seconds (the clock is shared, and it takes tens of
    milliseconds to settle), then timed in 5 rounds of one trial each, in an
    order that rotates from round to round; a trial is 20 back-to-back calls.
    Each figure is the median of its 5 trials."""
    import torch
    stream = torch.cuda.current_stream()

    def trial_us(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / 20

    def median_us(fns):
        names = list(fns)
        n, t_end = 0, time.perf_counter() + TABLE_WARMUP_S
        while n < 10 or time.perf_counter() < t_end:
            for k in names:
                fns[k]()
            n += 1
            if n % 10 == 0:
                torch.cuda.synchronize()
        trials = {k: [] for k in names}
        for r in range(5):
            for k in names[r % len(names):] + names[:r % len(names)]:
                trials[k].append(trial_us(fns[k]))
        return {k: statistics.median(v) for k, v in trials.items()}

    for name in sorted(wl.WORKLOADS, key=lambda n: wl.WORKLOADS[n]["index"]):
        w = wl.WORKLOADS[name]
        if w.get("mx") or w.get("sparse"):
            continue
        M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
        call, Cd, plan, nbytes, keep = workload_call(gr, name, stream)
        Ad, Bd = keep
        Bkn = Bd.t() if tb else Bd             # (K, N) operand of the product, a view
        rec = {"workload": name, "tile_config": plan}
        try:
            if ic in wl.FP8:
                one = torch.ones((), device="cuda")
                Bcm = Bkn.t().contiguous().t()   # column-major (K, N), as the fp8 GEMM takes it
                vfn = lambda: torch._scaled_mm(Ad, Bcm, scale_a=one, scale_b=one,
                                               out_dtype=torch_dtype(oc))
                rec["vendor"] = "torch._scaled_mm (unit scales)"
            elif oc == wl.F32 and ic != wl.F32:
                vfn = lambda: torch.mm(Ad, Bkn, out_dtype=torch.float32)
                rec["vendor"] = "torch.mm, fp32 out_dtype"
            else:
                vfn = lambda: torch.mm(Ad, Bkn)
                rec["vendor"] = "torch.mm"
            out = vfn()
            torch.cuda.synchronize()
            med = median_us({"ours": call, "vendor": vfn, "vendor_relu": lambda: torch.relu_(vfn())})
            rec.update(ours_us=round(med["ours"], 2), vendor_us=round(med["vendor"], 2),
                       vendor_relu_us=round(med["vendor_relu"], 2))
            # same result up to the summation order: the largest difference
            # after ReLU, relative to the largest output
            call()
            torch.cuda.synchronize()
            ref = torch.relu(out.float())
            rec["max_rel_diff"] = float((Cd.float() - ref).abs().max() / ref.abs().max().clamp_min(1e-30))
        except Exception as exc:               # a vendor path this image does not offer
            rec["vendor_error"] = repr(exc)[:160]
            rec["ours_us"] = round(median_us({"ours": call})["ours"], 2)
        flops = 2.0 * M * N * K
        for k in ("ours_us", "vendor_us", "vendor_relu_us"):
            if k in rec:
                rec[k.replace("_us", "_tflops")] = round(flops / rec[k] / 1e6, 1)
        print(json.dumps(rec), flush=True)
        del keep, Cd


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    # Before the counted warm-up: calls of the same step for at least this
    # long.  The power-managed clock drops within 0.2 s of idle and needs
    # 50-100 ms of load to come back (measured: the first 10 calls of a fresh
    # process average 1108 us, calls 60-400 about 798 us), so a short
    # warm-up right after the host-side input generation would time the ramp.
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--workload", default="gemm_relu_f16_8192", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--table", action="store_true",
                    help="time every workload (warm and cold caches), one JSON line each")
    ap.add_argument("--profile-workloads", type=int, default=0, metavar="CALLS",
                    help="run CALLS synchronised calls of every workload (for counter runs under "
                         "rocprofv3); prints the dispatch order")
    ap.add_argument("--vendor", action="store_true",
                    help="time the vendor GEMM (with and without a separate ReLU) beside "
                         "gemm_relu on every plain workload, one JSON line each")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the oracle over every plain workload on the host cores "
                         "(no GPU), one JSON line per run")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only the plain copy used to scale HBM byte counters")
    ap.add_argument("--ingest-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPYF", "COPYW"),
                    help="rocprofv3 --pmc output dirs -> profiles/traffic_<workload>.json")
    ap.add_argument("--ingest-cycles", metavar="PMC_DIR",
                    help="rocprofv3 --pmc GRBM_GUI_ACTIVE --kernel-trace output dir -> "
                         "profiles/cycles_<workload>.json")
    args = ap.parse_args()
    if args.ingest_traffic:
        ingest_traffic(args.workload, *args.ingest_traffic)
        return
    if args.ingest_cycles:
        ingest_cycles(args.workload, args.ingest_cycles)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.cpu_table:
        cpu_table()
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused GEMM+ReLU has no multi-GPU path in this "
              "library (an M or N split of C would need no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_tiled_gemm_relu_amd as gr

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(gr.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if args.table:
        table(gr)
        return
    if args.profile_workloads:
        profile_workloads(gr, args.profile_workloads)
        return
    if args.vendor:
        vendor(gr)
        return

    w = dict(wl.WORKLOADS[args.workload], name=args.workload)
    M, N, K, ic, oc, tb = w["M"], w["N"], w["K"], w["in_dtype"], w["out_dtype"], w["transB"]
    stream = torch.cuda.current_stream()
    step, Cd, plan, nbytes, keep = workload_call(gr, args.workload, stream)
    sparse = w.get("sparse", False)
    peak = peak_tflops(ic, sparse)

    settle_calls, t_end = 0, time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        step()
        settle_calls += 1
        if settle_calls % 8 == 0:
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` calls, synchronised on both sides; HIP
    # events on the launch stream give the kernels' own average duration
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    flops = 2.0 * M * N * K
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    metric = METRIC if args.workload == "gemm_relu_f16_8192" else (
        "TFLOP/s and %% of MI355X %s MFMA peak, %s" %
        ("2:4 sparse fp16/bf16 (dense-equivalent)" if sparse else
         {PEAK_TFLOPS_F4: "fp4", PEAK_TFLOPS_F8: "fp8"}.get(peak, "fp16/bf16"),
         args.workload))
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "calls": settle_calls},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.DTYPE_NAMES[ic],
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "in": wl.DTYPE_NAMES[ic], "out": wl.DTYPE_NAMES[oc], "transB": tb,
                   "accumulate": "f32", "inputs": w["dist"], "tile_config": plan},
        "roofline": roofline(flops, nbytes, kernel_ms, peak, measured_traffic(args.workload)),
    }
    cycles = measured_cycles(args.workload)
    if cycles is not None:
        out["clock"] = {"mhz": round(cycles / (kernel_ms * 1e-3) / 1e6),
                        "source": "shader cycles per launch (GRBM_GUI_ACTIVE per XCD, "
                                  "profiles/cycles_%s.json) / kernel_ms" % args.workload}
    ceiling = mfma_ceiling(gr, stream, kind=ceiling_kind(ic, sparse, plan))
    if ceiling is not None:
        out["mfma_ceiling"] = dict(ceiling, frac=round(achieved / ceiling["tflops"], 4))
    if not args.no_cpu_baseline:
        if w.get("mx"):
            out["cpu_baseline"] = cpu_baseline_mx(w)
        elif w.get("sparse"):
            out["cpu_baseline"] = cpu_baseline_sp(w)
        else:
            A, B = wl.workload_inputs(args.workload)
            out["cpu_baseline"] = cpu_baseline(w, A, B)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
