#!/usr/bin/env python3
"""Throughput of C = A.B on one MI355X through the C ABI (gemm_run).

One step = one gemm_run over the whole workload (default: bf16 8192^3 with
bf16 output, A and B i.i.d. N(0,1)).  Inputs are generated on the host from
fixed seeds and are resident in HBM before timing starts; the timed region is
K back-to-back launches on one stream between two HIP events, after W
untimed warmups.  TFLOP/s counts 2MNK per step.

Printed: one JSON line with the contract fields plus
  roofline      the GEMM kernel against the dense bf16/fp16 MFMA peak;
  repeats       the timed launches cut into five equal repeats (events on the
                launch stream): mean, median, min and max of their per-launch
                means;
  cold_l2       single launches of the main workload, each after reading a
                512 MiB buffer so that neither the L2s nor the Infinity Cache
                hold A or B (the repeated launches above run warm);
  cpu_baseline  the CPU fp64 oracle timed on a bounded sample of output rows
                of the same workload on this host (and those rows checked
                against the GPU result);
  observed      the three denominators of the measurement: a window of
                back-to-back launches during which amd-smi samples the eight
                XCD shader clocks and socket power, giving FLOP/clk/CU at the
                clock the chip held (against 4096 nominal) and the fraction
                of the spec peak at that clock; and the same window for the
                MFMA-only loop of bench_probe.hip on the same kind of operand
                data (the practical MFMA ceiling), giving the fraction of the
                probe-measured peak;
  secondary     the same measurement on bf16 4096^3;
  other_configs the same on the other workloads (fp16 2048^3, the ragged
                fp16 3000x5000x4099 shape, fp16 256^3, and the 8-bit float
                E4M3 8192^3 -> bf16 with B column-major, against the dense
                fp8 peak of 5.0 PFLOP/s).
Before the warmups of each workload, untimed launches run for about
--settle-ms so that the timed launches see a settled shader clock.

Other modes: --copy-calibration (the plain copy that scales the HBM byte
counters), --loop-seconds (one workload back to back, or the MFMA-only loop of
bench_probe.hip: mfma_probe_bf16_data, mfma_probe_f16_data, mfma_probe_e4m3_data)
and --power-sample (that loop in a child process, with amd-smi power and clock
samples taken by this process, which never touches the GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) at 4096³ and 8192³ bf16/fp16; % of MFMA peak"
PEAK_TFLOPS = 2500.0        # MI355X published dense fp16/bf16 MFMA peak
HBM_GBPS = 8000.0           # MI355X published HBM3E bandwidth
CODES = {("f16", "f32"): 0, ("f16", "f16"): 1, ("bf16", "f32"): 2, ("bf16", "bf16"): 3,
         ("e4m3", "f32"): 4, ("e4m3", "f16"): 5, ("e4m3", "bf16"): 6,
         ("e5m2", "f32"): 7, ("e5m2", "f16"): 8, ("e5m2", "bf16"): 9}
EIGHT_BIT = ("e4m3", "e5m2")
PEAK8_TFLOPS = 5000.0       # MI355X published dense fp8 MFMA peak
N_CU = 256                  # MI355X compute units (8 XCDs x 32)
FLOP_PER_CLK_CU = 4096      # dense fp16/bf16 MFMA FLOP per clock per CU (nominal)
FLOP_PER_CLK_CU8 = 8192     # dense fp8
PROBE_LIB = os.path.join(ROOT, "libdhpt_bench_probe.so")
TRAFFIC_SOURCE = ("profiles/hbm_traffic.json: rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0 per launch, "
                  "looked up by workload, instance and a hash of the kernel sources; not measured in this run")
# The sources each kernel family is compiled from, with the instance table
# (which holds the tile visit order): a counter summary stays valid for a
# workload while these are unchanged.
FAMILY_SOURCES = {
    "dl": ["dense_half_precision_tiled_amd/csrc/gemm_common.h",
           "dense_half_precision_tiled_amd/csrc/gemm_dl_kernel.h",
           "dense_half_precision_tiled_amd/csrc/gemm_internal.h",
           "dense_half_precision_tiled_amd/csrc/gemm_instances.hip"],
    "dl8": ["dense_half_precision_tiled_amd/csrc/gemm_common.h",
            "dense_half_precision_tiled_amd/csrc/gemm_dl_kernel.h",
            "dense_half_precision_tiled_amd/csrc/gemm_internal.h",
            "dense_half_precision_tiled_amd/csrc/gemm_instances.hip"],
    "ks": ["dense_half_precision_tiled_amd/csrc/gemm_instances.hip",
           "dense_half_precision_tiled_amd/csrc/gemm_common.h",
           "dense_half_precision_tiled_amd/csrc/gemm_ks_kernel.h",
           "dense_half_precision_tiled_amd/csrc/gemm_internal.h"],
}


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed, so
    that rewording a comment does not count as a change of the kernel (the
    sources hold no string literal with comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in FAMILY_SOURCES[family]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def describe(w, layout=None) -> str:
    lay = layout or w.get("layout", "row")
    return "%s GEMM C=A.B M=%d N=%d K=%d %s, %s inputs, fp32 accumulate, %s output" % (
        w["fmt"], w["M"], w["N"], w["K"],
        "A row-major, B column-major" if lay == "col" else "row-major",
        "U[-1,1)" if w["law"] == "uniform" else "N(0,1)", w["out"])


def peak_for(w) -> float:
    return PEAK8_TFLOPS if w["fmt"] in EIGHT_BIT else PEAK_TFLOPS


def upload(bits, torch):
    import numpy as np
    return torch.from_numpy(bits.view(np.int16) if bits.dtype.itemsize == 2 else bits.view(np.int8)).cuda()


def measure(G, torch, name, steps, warmup, instance=None, layout=None, settle_ms=200.0, entry="run", relu=0,
            splits=4):
    """Upload a workload, run one correctness launch into a poisoned C, let
    the clock settle (untimed launches for about settle_ms), run `warmup`
    untimed launches, then time `steps` launches.  Returns a dict with the
    timing and the buffers.
    layout "col" stores B column-major (its transpose row-major) and calls
    gemm_run_ex; "row" calls gemm_run; None takes the workload's own.
    entry "ws" calls gemm_run_ws instead, with a zeroed workspace of
    gemm_workspace_size() bytes allocated here (before timing); entry
    "splitk" calls gemm_run_splitk with `splits` pieces of K and its
    workspace, allocated here too.  relu = 1 applies ReLU through gemm_run_ex
    (the general-epilogue kernels)."""
    import numpy as np
    from dense_half_precision_tiled_amd import inputs
    A, B, w = inputs.workload_inputs(name)
    M, N, K = w["M"], w["N"], w["K"]
    code = CODES[(w["fmt"], w["out"])]
    layout = layout or w.get("layout", "row")
    col = layout == "col"
    tA, tB = upload(A, torch), upload(np.ascontiguousarray(B.T) if col else B, torch)
    odt = torch.float32 if w["out"] == "f32" else torch.int16
    tC = torch.full((M, N), -1, dtype=torch.int32 if odt == torch.float32 else torch.int16,
                    device="cuda")                      # all-ones bits: NaN poison
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    ldb = K if col else N
    args = (M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), ldb, tC.data_ptr(), N, s)
    ex_tail = (1.0, 0.0, None, relu, s)
    force_ex = bool(relu)                    # ReLU: through gemm_run_ex, whatever the B layout
    ws = torch.zeros(G.gemm_workspace_size() // 4, dtype=torch.int32, device="cuda") if entry == "ws" else None
    lay_code = G.GEMM_B_COL_MAJOR if col else G.GEMM_B_ROW_MAJOR
    ws_args = (args[:4] + (lay_code,) + args[4:-1] + (1.0, 0.0, None, relu) +
               ((ws.data_ptr(), G.gemm_workspace_size(), s) if ws is not None else ()))
    sk_ws, sk_args = None, None
    if entry == "splitk":
        need = G.gemm_splitk_workspace_size(M, N, K, splits)
        if need < 0:
            raise RuntimeError("gemm_splitk_workspace_size: %s" % G.gemm_strerror(need))
        sk_ws = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")
        sk_args = (args[:4] + (lay_code,) + args[4:-1] + (1.0, 0.0, None, relu, splits, sk_ws.data_ptr(),
                                                          sk_ws.numel() * 4, s))

    def launch(_keep=(tA, tB, tC, ws, sk_ws)):
        # the closure owns the buffers whose addresses `args` holds, so they
        # stay allocated for as long as it can be called
        if sk_args is not None:
            st = G.gemm_run_splitk(*sk_args)
        elif ws is not None:
            st = G.gemm_run_ws(*ws_args) if instance is None else G.gemm_run_instance_ws(instance, *ws_args)
        elif col or force_ex:
            a = args[:4] + (lay_code,) + args[4:-1] + ex_tail
            st = G.gemm_run_ex(*a) if instance is None else G.gemm_run_instance_ex(instance, *a)
        else:
            st = G.gemm_run(*args) if instance is None else G.gemm_run_instance(instance, *args)
        if st != 0:
            raise RuntimeError("gemm_run failed: %s" % G.gemm_strerror(st))

    launch()
    torch.cuda.synchronize()
    # The shader clock ramps up over tens of milliseconds of load; without
    # this, short kernels are timed partly at idle clocks.
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(8):
            launch()
        n_settle += 8
        torch.cuda.synchronize()
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    # The timed launches are cut into up to five equal repeats by events on
    # the launch stream; the step time is over all of them, and the spread of
    # the per-repeat means is reported beside it.
    nrep = max(1, min(5, steps))
    bounds = [round(i * steps / nrep) for i in range(nrep + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    evs[0].record(stream)
    t0 = time.perf_counter()
    for i in range(nrep):
        for _ in range(bounds[i + 1] - bounds[i]):
            launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / max(steps, 1)
    rep_ms = [evs[i].elapsed_time(evs[i + 1]) / (bounds[i + 1] - bounds[i])
              for i in range(nrep) if bounds[i + 1] > bounds[i]]
    flops = 2.0 * M * N * K
    if sk_args is not None:
        inst = None
    elif instance is not None:
        inst = instance
    elif ws is not None:
        inst = G.gemm_select_instance_ws(*ws_args[:-1])
    elif col or force_ex:
        inst = G.gemm_select_instance_ex(M, N, K, code, lay_code, tA.data_ptr(), K,
                                         tB.data_ptr(), ldb, tC.data_ptr(), N, 1.0, 0.0, None, relu)
    else:
        inst = G.gemm_select_instance(M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N,
                                      tC.data_ptr(), N)
    return {"name": name, "w": w, "layout": layout, "entry": "gemm_run_splitk" if sk_args is not None else
            "gemm_run_ws" if ws is not None else ("gemm_run_ex" if col or force_ex else "gemm_run"), "relu": relu,
            "A": A, "B": B, "C": tC, "ms": ms, "rep_ms": rep_ms,
            "launch": launch,
            "wall_s": wall, "settle_launches": n_settle,
            "tflops": flops / (ms * 1e-3) / 1e12,
            "instance": ("splitk_%d" % splits if splits else "splitk_auto") if inst is None else
            G.gemm_instance_name(inst),
            "alg_bytes": (1 if w["fmt"] in EIGHT_BIT else 2) * (M * K + K * N) + (4 if w["out"] == "f32" else 2) * M * N}


def repeats(res):
    import statistics
    r = res["rep_ms"]
    return {"n": len(r), "ms_mean": round(statistics.mean(r), 5), "ms_median": round(statistics.median(r), 5),
            "ms_min": round(min(r), 5), "ms_max": round(max(r), 5)}


def measure_cold(torch, res, launches: int, flush_bytes: int = 512 << 20):
    """Single launches with cold caches: before each, read a buffer larger
    than the L2s and the Infinity Cache together (a sum over it, so the
    caches hold only clean lines of that buffer), then time the one launch
    with events on its stream."""
    import statistics
    flush = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        total = flush.sum()
        e0.record(stream)
        res["launch"]()
        e1.record(stream)
        torch.cuda.synchronize()
        if int(total.item()) != flush_bytes // 4:
            raise RuntimeError("flush buffer read back wrong")
        times.append(e0.elapsed_time(e1))
    del flush
    w = res["w"]
    ms = statistics.mean(times)
    return {"launches": launches, "flush_bytes": flush_bytes, "ms_mean": round(ms, 5),
            "ms_median": round(statistics.median(times), 5),
            "value": round(2.0 * w["M"] * w["N"] * w["K"] / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}


def traffic_from_profiles(name: str, instance_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when that summary is missing, was taken on another kernel, or on
    other sources of the kernel's family."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    entry = d.get("workloads", {}).get(name)
    family = instance_name.split("_")[0]
    if entry is None or family not in FAMILY_SOURCES or entry.get("instance") != instance_name:
        return None
    if entry.get("source_hash") != kernel_source_hash(family):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(res, budget_s: float):
    """Time the CPU oracle on a sample of output rows of the same workload and
    check those rows of the GPU result against it."""
    import numpy as np
    import torch
    import oracle
    w = res["w"]
    M, N, K = w["M"], w["N"], w["K"]
    threads = oracle.default_threads()
    rng = np.random.Generator(np.random.PCG64(1234))
    # Each call pays a fixed cost (decoding B) plus a cost per round of
    # `threads` rows (the rows of a round run in parallel, one per thread):
    # time one and three rounds to separate them, then size the sample to the
    # budget in whole rounds.
    times = []
    for n in (threads, 3 * threads):
        rows = rng.integers(0, M, min(n, M)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.gemm_rows_f64(res["A"], res["B"], rows, w["fmt"], threads)
        times.append(time.perf_counter() - t0)
    per_round = max((times[1] - times[0]) / 2.0, 1e-6)
    fixed = max(times[0] - per_round, 0.0)
    rounds = max(1, int((budget_s - fixed) / per_round))
    nrows = int(min(M, rounds * threads))
    rows = np.array(sorted(set(rng.choice(M, max(nrows - 2, 0), replace=False).tolist()) | {0, M - 1}), dtype=np.int64)
    t0 = time.perf_counter()
    r = oracle.gemm_rows_f64(res["A"], res["B"], rows, w["fmt"], threads)
    t = time.perf_counter() - t0
    raw = res["C"].cpu().numpy()
    if w["out"] == "f32":
        y = raw.view(np.float32).astype(np.float64)[rows]
    elif w["out"] == "f16":
        y = raw.view(np.float16).astype(np.float64)[rows]
    else:
        y = (raw.view(np.uint16)[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    check = oracle.compare(y, r, K, w["out"])
    flops = 2.0 * rows.size * N * K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d output rows (all %d columns, full K=%d), fp64 triple loop, %.1f s"
                      % (rows.size, M, N, K, t),
            "seconds": round(t, 3),
            "parity_on_sample": {"ok": check["ok"], "max_abs": check["max_abs"],
                                 "max_rel": check["max_rel"], "n_bad": check["n_bad"]},
            "single_thread": single_thread_oracle()}


def single_thread_oracle():
    """Per-core figure: the whole fp16 256^3 product on one host thread."""
    from dense_half_precision_tiled_amd import inputs
    import oracle
    A, B, w = inputs.workload_inputs("f16_256")
    best = float("inf")
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemm_f64(A, B, w["fmt"], 1)
        best = min(best, time.perf_counter() - t0)
    return {"workload": "fp16 256x256x256, full product", "threads": 1,
            "value": round(2.0 * w["M"] * w["N"] * w["K"] / best / 1e9, 3), "unit": "GFLOP/s",
            "seconds": round(best, 4)}


def smi_sample():
    """(socket power W, [gfx clock MHz per XCD]) from amd-smi, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout)
        d = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [float(d["clock"][k]["clk"]["value"]) for k in d["clock"] if k.startswith("gfx_")]
        return float(d["power"]["socket_power"]["value"]), clks
    except Exception:          # no amd-smi, a changed JSON layout: report no clock
        return None


def clock_window(torch, launch, flops_per_launch: float, seconds: float) -> dict:
    """Launch back to back for about `seconds` (batches of 8 on the current
    stream, timed with events over the whole window) while a thread samples
    the XCD clocks and socket power.  Returns the rate and the samples'
    statistics (clock None when amd-smi gave nothing)."""
    import statistics
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            x = smi_sample()
            if x is None:
                return
            samples.append(x)
            stop.wait(0.05)

    stream = torch.cuda.current_stream()
    launch()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, t0 = 0, time.perf_counter()
    e0.record(stream)
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            launch()
        n += 8
        torch.cuda.synchronize()
    e1.record(stream)
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    ms = e0.elapsed_time(e1)
    out = {"seconds": round(ms * 1e-3, 3), "launches": n,
           "tflops": round(n * flops_per_launch / (ms * 1e-3) / 1e12, 2), "smi_samples": len(samples)}
    busy = [x for x in samples if statistics.mean(x[1]) > 500]      # skip samples taken while idle
    if busy:
        out.update({"sclk_mhz_mean": round(statistics.mean(statistics.mean(x[1]) for x in busy), 1),
                    "sclk_mhz_xcd_min": min(min(x[1]) for x in busy),
                    "sclk_mhz_xcd_max": max(max(x[1]) for x in busy),
                    "power_w_mean": round(statistics.mean(x[0] for x in busy), 1)})
    else:
        out["sclk_mhz_mean"] = None
    return out


def load_probe():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("%s is missing: run __graft_entry__.build()" % PROBE_LIB)
    P = ctypes.CDLL(PROBE_LIB)
    P.bench_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.bench_probe_mfma.restype = ctypes.c_int
    P.bench_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    P.bench_probe_flops.restype = ctypes.c_double
    return P


PROBE_FMT = {"f16": 0, "bf16": 1, "e4m3": 2}


def probe_launcher(torch, fmt: str, iters: int):
    """A launch function for the MFMA-only loop on `fmt` operand data (drawn
    like the workloads' inputs: fp16 U[-1,1), bf16 and E4M3 N(0,1)), one
    workgroup per CU, and its FLOPs per launch."""
    from dense_half_precision_tiled_amd import inputs
    P = load_probe()
    code = PROBE_FMT[fmt]
    n = 32 * 64 * 16 if fmt == "e4m3" else 16 * 64 * 8
    bits = {"f16": lambda: inputs.uniform((n,), 7, inputs.F16), "bf16": lambda: inputs.normal((n,), 7, inputs.BF16),
            "e4m3": lambda: inputs.normal((n,), 7, inputs.E4M3)}[fmt]()
    ops = upload(bits, torch)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * 4 * N_CU, dtype=torch.int64, device="cuda")
    nbytes = ops.numel() * ops.element_size()

    def launch(_keep=(ops, sink, clocks)):
        st = P.bench_probe_mfma(code, N_CU, iters, ops.data_ptr(), nbytes, sink.data_ptr(), clocks.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("probe launch failed (%d)" % st)

    def kernel_mhz():
        """Median over the waves of the last launch of shader clocks per microsecond."""
        import numpy as np
        c = clocks.cpu().numpy().reshape(-1, 2).astype(np.float64)
        c = c[c[:, 0] > 0]
        return float(np.median(c[:, 1] / (c[:, 0] * 0.01))) if c.size else None
    launch.kernel_mhz = kernel_mhz
    return launch, P.bench_probe_flops(code, N_CU, iters)


def kernel_clock(name: str, entry: str):
    """The shader clock the GEMM kernel itself runs at: a child process runs
    `bench.py --timeline 2` on the same workload with the profiling build of
    the library, whose waves record s_memtime and s_memrealtime; returns the
    median over workgroups of the last launch, or None (no profiling build,
    or the child failed).  amd-smi's clock samples are not used for this:
    they read well above the in-kernel clock on short kernels."""
    import subprocess
    from dense_half_precision_tiled_amd import build as B
    if not os.path.exists(B.TIMELINE_LIB):
        return None
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--timeline", "2", "--workload", name,
                            "--entry", entry, "--warmup", "3"], capture_output=True, text=True, timeout=180)
        d = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
        last = d["launches"][-1]
        return {"mhz_median": last["wg_mhz_median"],
                "xcd_mhz": [v["median_mhz"] for v in last["per_xcd"].values()]}
    except Exception:
        return None


def observed(torch, res, seconds: float) -> dict:
    """The clock-based denominators for one measured workload: FLOP/clk/CU at
    the shader clock the kernel runs at (in-kernel counters of the profiling
    build), the fraction of the spec peak at that clock, and the fraction of
    the MFMA-only loop's rate on the same kind of data (its own window, its
    own in-kernel clock); plus socket power and amd-smi's clock readings
    during both windows."""
    w = res["w"]
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    g = clock_window(torch, res["launch"], flops, seconds)
    fmt = "e4m3" if w["fmt"] in EIGHT_BIT else w["fmt"]
    plaunch, pflops = probe_launcher(torch, fmt, 4000 if fmt == "e4m3" else 8000)
    p = clock_window(torch, plaunch, pflops, seconds)
    p["kernel_mhz"] = plaunch.kernel_mhz()
    nominal = FLOP_PER_CLK_CU8 if fmt == "e4m3" else FLOP_PER_CLK_CU
    kc = None if res["entry"] == "gemm_run_splitk" else kernel_clock(
        res["name"], "ws" if res["entry"] == "gemm_run_ws" else "run")
    out = {"gemm_window": g, "probe_window": p, "gemm_kernel_clock": kc,
           "probe": "bench_probe.hip MFMA-only loop, %s operand data, one workgroup per CU" % fmt,
           "frac_of_probe_peak": round(res["tflops"] / p["tflops"], 4),
           "flop_per_clk_per_cu_nominal": nominal,
           "ridge_at_kernel_clock_flop_per_byte": None}
    if kc is not None and kc.get("mhz_median"):
        fpc = res["tflops"] * 1e12 / (N_CU * kc["mhz_median"] * 1e6)
        out["flop_per_clk_per_cu"] = round(fpc, 1)
        out["frac_of_peak_at_kernel_clock"] = round(fpc / nominal, 4)
        out["ridge_at_kernel_clock_flop_per_byte"] = round(
            N_CU * nominal * kc["mhz_median"] * 1e6 / (HBM_GBPS * 1e9), 1)
    if p.get("kernel_mhz"):
        out["probe_flop_per_clk_per_cu"] = round(p["tflops"] * 1e12 / (N_CU * p["kernel_mhz"] * 1e6), 1)
    return out


TIMELINE_WAVES = 65536      # room for 8192 workgroups of 8 waves


def timeline_summary(rec, tiles_of=None):
    """Summary of one launch's timeline records (rows of 8 int64 words:
    start and end on the 100 MHz real-time counter, start and end on the
    shader-clock counter, XCC id << 32 | HW_ID, workgroup id; unused rows are
    zero)."""
    import statistics
    import numpy as np
    rec = np.asarray(rec, dtype=np.int64).reshape(-1, 8)
    rec = rec[rec[:, 1] > 0]
    base = int(rec[:, 0].min())
    tick_us = 0.01                                         # s_memrealtime: 100 MHz
    xcc = (rec[:, 4] >> 32) & 0xF
    hw = rec[:, 4] & 0xFFFFFFFF
    # a CU: XCC, shader engine, shader array and CU index of HW_ID
    cu_key = xcc * 4096 + (((hw >> 13) & 7) << 8) + (((hw >> 12) & 1) << 4) + ((hw >> 8) & 0xF)
    wgs = {}                                               # workgroup: (start, end, xcc, cu, MHz)
    tiles = {}                                             # workgroup: output tiles it computed
    for i in range(rec.shape[0]):
        g = int(rec[i, 5])
        real = int(rec[i, 1] - rec[i, 0])
        mhz = (rec[i, 3] - rec[i, 2]) / (real * tick_us) if real > 0 else 0.0
        a, b, _, _, f = wgs.get(g, (1 << 62, 0, 0, 0, 0.0))
        wgs[g] = (min(a, int(rec[i, 0])), max(b, int(rec[i, 1])), int(xcc[i]), int(cu_key[i]), max(f, mhz))
        tiles[g] = int(rec[i, 6])
    span = (max(v[1] for v in wgs.values()) - base) * tick_us
    per_xcd, cu_busy = {}, {}
    for (a, b, x, c, f) in wgs.values():
        per_xcd.setdefault(x, []).append(((a - base) * tick_us, (b - base) * tick_us, f))
        cu_busy[c] = cu_busy.get(c, 0.0) + (b - a) * tick_us
    durs = [(b - a) * tick_us for (a, b, _, _, _) in wgs.values()]
    # the slowest workgroups, with the output tile each computed (one-tile
    # launches: workgroup id -> (tile row, tile column) from the visit order)
    slow = sorted(wgs.items(), key=lambda kv: kv[1][0] - kv[1][1])[:12]
    slowest = [{"wg": g, "us": round((b - a) * tick_us, 2), "xcd": x,
                "tile": (list(tiles_of[g]) if tiles_of is not None and g < len(tiles_of) else None)}
               for g, (a, b, x, _, _) in slow]
    return {"span_us": round(span, 2), "workgroups": len(wgs), "cus": len(cu_busy), "slowest": slowest,
            "wg_us_min": round(min(durs), 2), "wg_us_median": round(statistics.median(durs), 2),
            "wg_us_max": round(max(durs), 2),
            "wg_mhz_median": round(statistics.median(v[4] for v in wgs.values()), 1),
            "last_start_us": round(max((a - base) * tick_us for (a, _, _, _, _) in wgs.values()), 2),
            "cu_idle_frac": round(1.0 - sum(cu_busy.values()) / (len(cu_busy) * span), 4),
            "per_xcd": {str(x): {"wgs": len(v), "first_end_us": round(min(e for _, e, _ in v), 2),
                                 "median_end_us": round(statistics.median(e for _, e, _ in v), 2),
                                 "last_end_us": round(max(e for _, e, _ in v), 2),
                                 "median_wg_us": round(statistics.median(e - s0 for s0, e, _ in v), 2),
                                 "median_mhz": round(statistics.median(f for _, _, f in v), 1),
                                 "tiles": sum(tiles[g] for g, w in wgs.items() if w[2] == x)}
                        for x, v in sorted(per_xcd.items())}}


def timeline(G, torch, name: str, launches: int, warmup: int, settle_ms: float, entry: str = "run",
             instance=None, relu: int = 0) -> int:
    """Per-workgroup timeline of `launches` launches of one workload, from the
    profiling build of the library (libdhpt_gemm_timeline.so, which records
    for every wave its start and end on the 100 MHz real-time counter and on
    the shader clock, and the XCC and CU it ran on).  Prints, per launch, the kernel span, the end times
    of each XCD's first and last workgroups, workgroup durations, and the
    share of CU time spent outside workgroups."""
    res = measure(G, torch, name, 1, warmup, instance, None, settle_ms, entry, relu)
    w = res["w"]
    inst_id = [i for i in range(G.gemm_num_instances()) if G.gemm_instance_name(i) == res["instance"]][0]
    tm, tn = G.gemm_tile_order(inst_id, w["M"], w["N"])
    tiles_of = list(zip(tm.tolist(), tn.tolist()))
    buf = torch.zeros(TIMELINE_WAVES * 8, dtype=torch.int64, device="cuda")
    lib = G.load()
    lib.gemm_timeline_set(ctypes.c_void_p(buf.data_ptr()), TIMELINE_WAVES)
    out = []
    for it in range(launches):
        buf.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        res["launch"]()
        e1.record()
        torch.cuda.synchronize()
        summ = timeline_summary(buf.cpu().numpy(), tiles_of)
        summ.update({"launch": it, "event_ms": round(e0.elapsed_time(e1), 4)})
        out.append(summ)
    lib.gemm_timeline_set(None, 0)
    print(json.dumps({"timeline": name, "kernel": res["instance"], "launches": out}), flush=True)
    return 0


def _counter_rows(path: str, counter: str):
    """(kernel name, grid size, value) per dispatch of one rocprofv3 counter
    CSV (p_counter_collection.csv), in dispatch order."""
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"].startswith(counter):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"].split("(")[0].replace("void ", ""),
                         int(r["Grid_Size"]), float(r["Counter_Value"])))
    rows.sort()
    return [(k, g, v) for _, k, g, v in rows]


def traffic_summary(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                    workloads, instances, copy_bytes: int) -> int:
    """Write profiles/hbm_traffic.json from two rocprofv3 --pmc runs of
    `bench.py --steps 3 --warmup 1 --settle-ms 0 ...` (FETCH_SIZE, then
    WRITE_SIZE) and two of `--copy-calibration` (the plain copy that scales
    the counters).  The library's dispatches of each run come in the bench's
    workload order, one run of identical dispatches (kernel, grid) per
    workload; each workload's figures are the mean over its dispatches."""
    import statistics

    def runs(path, counter):
        out = []
        for k, g, v in _counter_rows(path, counter):
            if "dhpt::" not in k:
                continue
            if out and out[-1][0] == (k, g):
                out[-1][1].append(v)
            else:
                out.append(((k, g), [v]))
        return out

    def copy_kib(path, counter):
        vals = [v for k, g, v in _counter_rows(path, counter) if "copyBuffer" in k or "Copy" in k]
        return statistics.mean(vals[1:] if len(vals) > 1 else vals)

    fetch_scale = copy_bytes / 1024.0 / copy_kib(copy_fetch_csv, "FETCH_SIZE")
    write_scale = copy_bytes / 1024.0 / copy_kib(copy_write_csv, "WRITE_SIZE")
    fr, wr = runs(fetch_csv, "FETCH_SIZE"), runs(write_csv, "WRITE_SIZE")
    if len(fr) != len(workloads) or len(wr) != len(workloads):
        raise RuntimeError("expected %d workloads, found %d / %d kernel runs" % (len(workloads), len(fr), len(wr)))
    from dense_half_precision_tiled_amd import inputs
    out = {"note": "rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch (KiB), scaled by a %d MiB device copy; "
                   "source_hash: the sources of the kernel's family when the counters were taken" % (copy_bytes >> 20),
           "fetch_scale": fetch_scale, "write_scale": write_scale, "workloads": {}}
    for name, inst, (fk, fv), (wk, wv) in zip(workloads, instances, fr, wr):
        if fk != wk:
            raise RuntimeError("fetch and write runs differ for %s: %s / %s" % (name, fk, wk))
        w = inputs.WORKLOADS[name]
        esz = 1 if w["fmt"] in EIGHT_BIT else 2
        alg = esz * (w["M"] * w["K"] + w["K"] * w["N"]) + (4 if w["out"] == "f32" else 2) * w["M"] * w["N"]
        f, wv_ = statistics.mean(fv), statistics.mean(wv)
        family = inst.split("_")[0]
        out["workloads"][name] = {
            "kernel": fk[0], "instance": inst,
            "source_hash": kernel_source_hash(family) if family in FAMILY_SOURCES else None,
            "fetch_kib_raw": round(f, 2), "write_kib_raw": round(wv_, 2), "dispatches": [len(fv), len(wv)],
            "hbm_bytes_per_launch": int(round((f * fetch_scale + wv_ * write_scale) * 1024)),
            "algorithmic_bytes": alg}
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    for name, e in out["workloads"].items():
        print("| %s | `%s` | %d | %.1f | %.1f | %.1f | %.2fx |" % (
            name, e["kernel"], e["dispatches"][0], e["fetch_kib_raw"], e["fetch_kib_raw"] * fetch_scale / 1024,
            e["write_kib_raw"] * write_scale / 1024, e["hbm_bytes_per_launch"] / e["algorithmic_bytes"]))
    print("fetch_scale %.4f write_scale %.4f" % (fetch_scale, write_scale))
    return 0


def copy_calibration(torch, nbytes: int, steps: int, warmup: int) -> int:
    """Plain device-to-device copy of nbytes: reads nbytes and writes nbytes
    per launch.  Its FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / max(steps, 1)
    print(json.dumps({"copy_bytes": nbytes, "launches": steps + warmup, "ms_per_copy": round(ms, 5),
                      "gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def loop_for(G, torch, name, seconds: float) -> int:
    """Run one workload back to back for `seconds` and print the achieved rate.
    Besides the GEMM workloads, the MFMA-only loop of bench_probe.hip (eight
    independent accumulators per wave, one wave per SIMD on every CU):
    "mfma_probe_bf16_data" / "mfma_probe_f16_data" (32x32x16, operands drawn
    like the bf16 N(0,1) and fp16 U[-1,1) workloads' inputs, rotating so that
    consecutive MFMAs see new values as in a GEMM) and "mfma_probe_e4m3_data"
    (the 8-bit 32x32x64 MFMA on rotating N(0,1) E4M3 operands)."""
    if name in ("mfma_probe_bf16_data", "mfma_probe_f16_data", "mfma_probe_e4m3_data"):
        fmt = name.split("_")[2]
        launch, per = probe_launcher(torch, fmt, 25000 if fmt == "e4m3" else 50000)
        n, ms, t0 = 0, 0.0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ms += e0.elapsed_time(e1)
            n += 1
        flops = n * per
    else:
        import numpy as np
        from dense_half_precision_tiled_amd import inputs
        A, B, w = inputs.workload_inputs(name)
        M, N, K = w["M"], w["N"], w["K"]
        col = w.get("layout", "row") == "col"
        tA, tB = upload(A, torch), upload(np.ascontiguousarray(B.T) if col else B, torch)
        tC = torch.empty((M, N), dtype=torch.float32 if w["out"] == "f32" else torch.int16, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        code = CODES[(w["fmt"], w["out"])]
        args = (M, N, K, code, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N, s)
        if col:
            args = (M, N, K, code, G.GEMM_B_COL_MAJOR, tA.data_ptr(), K, tB.data_ptr(), K, tC.data_ptr(), N,
                    1.0, 0.0, None, 0, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, t0 = 0, time.perf_counter()
        e0.record()
        while time.perf_counter() - t0 < seconds:
            for _ in range(16):
                if (G.gemm_run_ex(*args) if col else G.gemm_run(*args)) != 0:
                    raise RuntimeError("gemm_run failed")
            n += 16
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = n * 2.0 * M * N * K
    print(json.dumps({"loop": name, "launches": n, "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}), flush=True)
    return 0


def power_sample(name: str, seconds: float) -> int:
    """Sample socket power and the eight XCD graphics clocks (amd-smi) while a
    child process runs `bench.py --loop-seconds` on one workload.  This
    process never touches the GPU; the child is started with subprocess (no
    exec)."""
    import statistics
    import subprocess

    def sample():
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=60)
        d = json.loads(r.stdout)["gpu_data"][0]
        clks = [d["clock"][k]["clk"]["value"] for k in d["clock"] if k.startswith("gfx_")]
        return d["power"]["socket_power"]["value"], clks

    idle_p, idle_c = sample()
    child = subprocess.Popen([sys.executable, "-u", os.path.abspath(__file__), "--workload", name,
                              "--loop-seconds", str(seconds)], stdout=subprocess.PIPE, text=True)
    time.sleep(min(2.0, seconds / 4))
    samples = []
    t0 = time.time()
    while child.poll() is None and time.time() - t0 < seconds:
        p, c = sample()
        if statistics.mean(c) > 1000:           # busy: the loop has started
            samples.append((p, c))
        time.sleep(0.3)
    out = child.communicate(timeout=300)[0]
    rate = json.loads([ln for ln in out.splitlines() if ln.startswith("{")][-1])
    res = {"power_sample": name, "seconds": seconds, "loop": rate, "idle_power_w": idle_p,
           "samples": len(samples)}
    if samples:
        res.update({"power_w_mean": round(statistics.mean(s[0] for s in samples), 1),
                    "power_w_min": min(s[0] for s in samples), "power_w_max": max(s[0] for s in samples),
                    "gfx_clk_mhz_mean": round(statistics.mean(statistics.mean(s[1]) for s in samples), 1),
                    "gfx_clk_mhz_xcd_min": min(min(s[1]) for s in samples),
                    "gfx_clk_mhz_xcd_max": max(max(s[1]) for s in samples)})
    print(json.dumps(res), flush=True)
    return child.returncode


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_8192")
    ap.add_argument("--secondary", default="bf16_4096", help="'none' to skip")
    ap.add_argument("--also", default="f16_2048,f16_ragged,f16_256,e4m3_8192",
                    help="comma-separated further workloads reported under other_configs ('none' to skip)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed launches for about this long before the warmups (clock ramp-up)")
    ap.add_argument("--instance", type=int, default=None, help="force a kernel instance id")
    ap.add_argument("--relu", action="store_true",
                    help="apply ReLU in the epilogue (gemm_run_ex: the general-epilogue kernels), e.g. to price "
                         "their cost against the plain ones")
    ap.add_argument("--entry", choices=("run", "ws", "splitk"), default="run",
                    help="call gemm_run / gemm_run_ex (run), gemm_run_ws with a caller-owned workspace (ws), or "
                         "gemm_run_splitk with --splits pieces of K (splitk; 16-bit workloads only)")
    ap.add_argument("--splits", type=int, default=4,
                    help="pieces of K for --entry splitk (0: the library's choice)")
    ap.add_argument("--layout", choices=("row", "col"), default=None,
                    help="storage order of B: row-major (gemm_run) or column-major (gemm_run_ex); "
                         "default: the workload's own (row-major for the 16-bit ones, column-major for 8-bit)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for cpu_baseline (0 to skip)")
    ap.add_argument("--cold", type=int, default=5, metavar="LAUNCHES",
                    help="also time this many single launches of the main workload with cold caches "
                         "(a 512 MiB buffer read before each; 0 to skip)")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="length of each clock-sampling window (main and secondary workload, and the "
                         "MFMA-only probe beside each); 0 to skip")
    ap.add_argument("--loop-seconds", type=float, default=0.0,
                    help="instead of the timed bench, run --workload (or one of the MFMA-only probes "
                         "'mfma_probe_bf16_data', 'mfma_probe_f16_data', 'mfma_probe_e4m3_data') back to back this long")
    ap.add_argument("--power-sample", type=float, default=0.0, metavar="SECONDS",
                    help="run --workload in a child process for SECONDS and sample power and clocks with amd-smi")
    ap.add_argument("--timeline", type=int, default=0, metavar="LAUNCHES",
                    help="instead of the timed bench, record the per-workgroup timeline of this many launches of "
                         "--workload with the profiling build (libdhpt_gemm_timeline.so)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the GEMM, time a plain device copy of BYTES bytes "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="instead of running, write profiles/hbm_traffic.json from rocprofv3 counter CSVs of this "
                         "bench (FETCH_SIZE run, WRITE_SIZE run) and of --copy-calibration (same two counters); "
                         "the workload list is --workload, --secondary, --also")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    if args.power_sample > 0:
        return power_sample(args.workload, args.power_sample)
    if args.traffic_summary:
        names = [args.workload] + ([args.secondary] if args.secondary and args.secondary != "none" else []) + \
            ([x for x in args.also.split(",")] if args.also and args.also != "none" else [])
        from dense_half_precision_tiled_amd import gemm as G0
        insts = []
        for name in names:
            from dense_half_precision_tiled_amd import inputs
            w = inputs.WORKLOADS[name]
            col = w.get("layout", "row") == "col"
            code = CODES[(w["fmt"], w["out"])]
            i = G0.gemm_select_instance_ex(w["M"], w["N"], w["K"], code, 1 if col else 0, 1 << 32, w["K"], 1 << 36,
                                           w["K"] if col else w["N"], 1 << 40, w["N"], 1.0, 0.0, None, 0)
            insts.append(G0.gemm_instance_name(i))
        return traffic_summary(*args.traffic_summary, names, insts, args.copy_calibration or (256 << 20))
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration > 0:
        return copy_calibration(torch, args.copy_calibration, args.steps, args.warmup)

    from dense_half_precision_tiled_amd import gemm as G
    if args.timeline > 0:
        if args.entry == "splitk":
            print("--timeline records the one-kernel entry points (run, ws)", file=sys.stderr)
            return 2
        from dense_half_precision_tiled_amd import build as B
        lib = G.load(B.TIMELINE_LIB)
        lib.gemm_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        return timeline(G, torch, args.workload, args.timeline, args.warmup, args.settle_ms, args.entry,
                        args.instance, int(args.relu))
    G.load()
    if args.loop_seconds > 0:
        return loop_for(G, torch, args.workload, args.loop_seconds)

    main_res = measure(G, torch, args.workload, args.steps, args.warmup, args.instance, args.layout,
                       args.settle_ms, args.entry, int(args.relu), args.splits)

    def summary(r):
        w2 = r["w"]
        return {"workload": describe(w2, r["layout"]), "value": round(r["tflops"], 2), "unit": "TFLOP/s",
                "ms_per_step": round(r["ms"], 5), "frac_of_peak": round(r["tflops"] / peak_for(w2), 4),
                "peak": peak_for(w2),
                "hbm_gbps_algorithmic": round(r["alg_bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
                "kernel": r["instance"], "entry_point": r["entry"], "repeats": repeats(r),
                "traffic": traffic_from_profiles(
                    r["name"] + ("" if r["layout"] == w2.get("layout", "row") else "_" + r["layout"]), r["instance"])}

    main_obs = observed(torch, main_res, args.clock_seconds) if args.clock_seconds > 0 else None
    sec = None
    if args.secondary and args.secondary != "none":
        r2 = measure(G, torch, args.secondary, max(args.steps, 50), args.warmup, args.instance,
                     args.layout, args.settle_ms, args.entry, int(args.relu), args.splits)
        sec = summary(r2)
        if args.clock_seconds > 0:
            sec["observed"] = observed(torch, r2, args.clock_seconds)
        del r2
    others = []
    if args.also and args.also != "none" and args.instance is None:
        from dense_half_precision_tiled_amd import inputs as I3
        for name in args.also.split(","):
            if args.entry == "splitk" and I3.WORKLOADS[name]["fmt"] in EIGHT_BIT:
                continue                     # gemm_run_splitk takes 16-bit inputs only
            r3 = measure(G, torch, name, max(args.steps, 200), args.warmup, None, args.layout,
                         args.settle_ms, args.entry, int(args.relu), args.splits)
            others.append(summary(r3))
            del r3

    w = main_res["w"]
    lay = main_res["layout"]
    traffic = traffic_from_profiles(args.workload + ("" if lay == w.get("layout", "row") else "_" + lay),
                                    main_res["instance"])
    line = {
        "metric": METRIC,
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["fmt"],
        "data": "synthetic",
        "config": {"workload": describe(w, lay),
                   "M": w["M"], "N": w["N"], "K": w["K"], "b_layout": lay,
                   "in": w["fmt"], "out": w["out"], "kernel": main_res["instance"],
                   "entry_point": main_res["entry"], "relu": bool(main_res["relu"]),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(main_res["tflops"], 2), "peak": peak_for(w),
                     "unit": "TFLOP/s", "frac": round(main_res["tflops"] / peak_for(w), 4),
                     "traffic": traffic,
                     "traffic_source": TRAFFIC_SOURCE if traffic is not None else
                     "none: no committed counter summary matches this kernel and its sources",
                     "algorithmic_bytes": main_res["alg_bytes"],
                     "intensity_flop_per_byte": round(2.0 * w["M"] * w["N"] * w["K"] / main_res["alg_bytes"], 1),
                     "ridge_flop_per_byte": round(peak_for(w) * 1e12 / (HBM_GBPS * 1e9), 1),
                     "hbm_gbps_algorithmic": round(main_res["alg_bytes"] / (main_res["ms"] * 1e-3) / 1e9, 1)},
    }
    if main_obs is not None:
        line["roofline"]["observed"] = main_obs
    line["repeats"] = repeats(main_res)
    if args.cold > 0:
        line["cold_l2"] = measure_cold(torch, main_res, args.cold)
    if sec is not None:
        line["secondary"] = sec
    if others:
        line["other_configs"] = others
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(main_res, args.cpu_budget)
    print(json.dumps(line), flush=True)
    if args.cpu_budget > 0 and not line["cpu_baseline"]["parity_on_sample"]["ok"]:
        print("the GPU result differs from the oracle on the sampled rows", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
