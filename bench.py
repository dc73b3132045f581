#!/usr/bin/env python3
"""Benchmark of the LLM.int8() mixed-precision linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one whole call of the hot path on one batch: outlier detection,
token quantization, outlier gathers, the int8 GEMM and its epilogue (the
fp16 outlier product and the fp16 store).  The weight is quantized once
before timing, as it is at load time.  Inputs are seeded synthetic tensors
(workloads/), resident in HBM before the timed region starts.

The K timed steps are K calls of llm_int8_linear captured in one HIP graph
(checked against an eager call), replayed between two synchronizations:
host launch cost does not pace the short few-token calls.  Untimed replays
of the same graph come first, for --settle-ms of GPU time, so that the
timed ones run at the steady-state shader clock.  Two cache states are
measured: warm (one buffer set, reused by every call) and cold (rotating
copies of every buffer, more than twice the 256 MB Infinity Cache per
cycle); `value` is the warm one unless --cold.

Prints one JSON line.  `value` is the effective throughput 2*T*N*K / time
of a step, in TOPS.  `roofline` is for the dominant kernel: the tiled GEMM
against the int8 MFMA peak, or for few tokens the single fused kernel
against HBM bandwidth; it is timed with HIP events on the stream the
library launches on.  `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same call.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA, published
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, published
DEFAULT_WORKLOAD = "prefill_7b_ffn_up_t4096"
METRIC = "effective TOPS (2*T*N*K/s) of llm_int8_linear"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--variant", choices=["int8w", "fp16w", "sq", "cached"], default="int8w",
                    help="outlier columns times the dequantized codes (default) or the fp16 "
                         "weight; sq: the SmoothQuant-style W8A8 call (smoothquant_linear, "
                         "alpha 0.5, calibrated on the first 512 rows of X); cached: "
                         "llm_int8_linear_cached with an outlier-column cache (every call "
                         "after the first reuses the gathered weight columns)")
    ap.add_argument("--cold", action="store_true",
                    help="make `value` the cold-cache measurement (copies of the call's buffers "
                         "rotated, more than 2 x 256 MB per cycle, so that no call finds its "
                         "operands in the Infinity Cache); both are measured either way")
    ap.add_argument("--shape", default=None, metavar="T,K,N",
                    help="the named workload's input recipe at another shape (for counter "
                         "attribution runs; the line then names the shape)")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed replays of the captured graph for this long before the "
                         "timed replay, so that it runs at the steady-state clock (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables it)")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip timing the vendor int8 GEMM (torch._int_mm) for reference")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device copy of known size (for HBM counter scaling)")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="after the measurements, replay graphs of the whole call and of the "
                         "GEMM alone for this long each while `amd-smi metric --power --clock` "
                         "is sampled, and report socket power and XCD clocks (0: skip)")
    return ap.parse_args()


# The headers every kernel source includes: a change in them changes the
# kernels as much as one in the source itself.
KERNEL_HEADERS = ["int8_matmul_amd/csrc/quant_math.h", "int8_matmul_amd/csrc/li8_internal.h"]


def sources_sha256(paths) -> str:
    """SHA-256 over the named files, in order (paths relative to the root)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(hashlib.sha256(fh.read()).digest())
    return h.hexdigest()


def profile_record(name: str, path_src: str, workload: str, shape):
    """The committed counter summary profiles/<name>.json, if it was taken
    on the current kernel source and headers and on this workload and shape
    [T, K, N]; else None."""
    f = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        rec = json.load(fh)
    files = rec.get("sources")
    if not files or rec.get("sources_sha256") != sources_sha256(files):
        return None
    if os.path.relpath(path_src, ROOT) not in files or rec.get("workload_name") != workload:
        return None
    if rec.get("shape") != list(shape):
        return None
    return rec


def kernel_traffic(kernel: str, path_src: str, workload: str, shape):
    """HBM-side bytes per launch of the dominant kernel (FETCH_SIZE +
    WRITE_SIZE scaled by a copy of known size) from
    profiles/<kernel>_<workload>_hbm_traffic.json."""
    rec = profile_record(f"{kernel}_{workload}_hbm_traffic", path_src, workload, shape)
    return rec.get("bytes_per_launch") if rec else None


def clock_adjusted(path_src: str, workload: str, shape, achieved: float):
    """The int8 peak at the shader clock the GEMM ran at in the committed
    counter run (SQ_BUSY_CYCLES per shader engine over the launch time,
    profiles/k_gemm_<workload>_sclk.json), and the fraction of it achieved
    here."""
    name = f"k_gemm_{workload}_sclk"
    rec = profile_record(name, path_src, workload, shape)
    if not rec:
        return None
    ghz = float(rec["sclk_ghz"])
    peak = PEAK_INT8_TOPS * ghz / 2.4
    return {"sclk_ghz": ghz, "peak": round(peak, 1), "frac": round(achieved / peak, 4),
            "sclk_from": f"profiles/{name}.json: SQ_BUSY_CYCLES per shader engine over the "
                         "profiled k_gemm launches (the 5.0 POP/s peak assumes 2.4 GHz)"}


def power_samples(g, seconds: float) -> dict:
    """Replays graph g back to back for `seconds` while a thread samples
    `amd-smi metric --power --clock --json` every 0.25 s; returns the medians
    (over the samples after the first second) of the socket power and of the
    GFX clock averaged over the XCDs."""
    import statistics
    import subprocess
    import threading

    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.perf_counter()
            try:
                r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"],
                                   capture_output=True, text=True, timeout=5)
                d = json.loads(r.stdout)
                gd = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                clk = [v["clk"]["value"] for k, v in gd["clock"].items() if k.startswith("gfx_")]
                samples.append((t, float(gd["power"]["socket_power"]["value"]),
                                sum(clk) / len(clk)))
            except Exception as e:   # amd-smi missing or its format differs
                samples.append((t, None, repr(e)[:120]))
            time.sleep(0.25)

    th = threading.Thread(target=sampler)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        g.replay()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    good = [x for x in samples if x[1] is not None and x[0] - t0 > 1.0]
    if not good:
        return {"error": samples[-1][2] if samples else "no sample"}
    return {"socket_power_w": statistics.median(x[1] for x in good),
            "gfx_clock_mhz": round(statistics.median(x[2] for x in good), 1),
            "samples": len(good)}


def cpu_baseline(X, W, w, target_s: float, variant: str, thr: float):
    """The oracle on a bounded sample, R rows sized so the run takes about
    target_s.  LLM.int8(): detection over all of X (the outlier set needs
    every row), then quantization, the int8 product and the output for the
    first R rows.  sq: the smoothed token quantization, int8 product and
    output for the first R rows (the factors and the weight are offline)."""
    import numpy as np

    import oracle
    cores = oracle.num_threads()
    if variant == "sq":
        s = oracle.sq_factors(oracle.column_absmax(X[:512]), oracle.column_absmax(W), 0.5)
        Wq, sW = oracle.sq_quantize_weight(W, s)

        def run(rows):
            oracle.sq_linear(X[:rows], s, Wq, sW)
        what = "smoothed quantization, int8 product and output for the first {r} of {T} rows"
    else:
        Wq, sW = oracle.quantize_weight(W)
        W16 = W if variant == "fp16w" else None

        def run(rows):
            oracle.linear_rows(X, Wq, sW, thr, np.arange(rows), W16=W16)
        what = ("detection over all {T} rows of X, then quantization, int8 product and "
                "output for the first {r} of {T} rows")
    # grow the sample until one run takes a noticeable time, then size the
    # final sample for about target_s (the per-row cost dominates by then)
    rows, dt = 4, 0.0
    while rows < w.T:
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 8:
            break
        rows = min(w.T, rows * 4)
    rows = int(min(w.T, max(4, rows * target_s / max(dt, 1e-3))))
    # when the whole call is shorter than target_s, it is repeated (up to 3
    # runs while the total stays near target_s) and the fastest run counts
    dts = []
    while True:
        t0 = time.perf_counter()
        run(rows)
        dts.append(time.perf_counter() - t0)
        if len(dts) >= 3 or sum(dts) + dts[-1] > target_s:
            break
    dt = min(dts)
    ops = 2.0 * rows * w.N * w.K
    # the oracle's quantize stage on the whole of X, timed on its own:
    # detection and token quantization (sq: the smoothed token quantization),
    # against the same algorithmic bytes as the GPU's stage minus the
    # outlier gathers
    T, K = X.shape
    t0 = time.perf_counter()
    if variant == "sq":
        oracle.sq_quantize_rows(X, s)
        qbytes = 2 * T * K + 4 * K + T * K + 4 * T
        qwhat = "smoothed token quantization of all of X"
    else:
        flags, _ = oracle.detect_outliers(X, thr)
        oracle.quantize_rows(X, flags)
        qbytes = 2 * T * K + 2 * T * K + T * K + 4 * T
        qwhat = "detection and token quantization of all of X (no outlier gathers)"
    qdt = time.perf_counter() - t0
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(ops / dt / 1e12, 6),
        "unit": "TOPS",
        "cores": cores,
        "cpu_model": model,
        "kind": "oracle",
        "sample": what.format(r=rows, T=w.T) + f" ({rows}x{w.K}x{w.N}); "
                  + (f"fastest of {len(dts)} runs, {dt:.1f} s" if len(dts) > 1 else f"{dt:.1f} s"),
        "quant_gbps": round(qbytes / qdt / 1e9, 3),
        "quant_sample": f"{qwhat} ({T}x{K}); {qdt * 1e3:.1f} ms",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer "
              "runs on a single MI355X. Across GPUs it would be split by output features "
              "(each GPU its share of Wq and sW, X replicated), which is not built here.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import int8_matmul_amd as li8
    import workloads

    w = workloads.WORKLOADS[args.workload]
    shape = {}
    if args.shape:
        shape = dict(zip("TKN", (int(v) for v in args.shape.split(","))))
        w = dataclasses.replace(w, **shape)
    thr = w.threshold if args.threshold is None else args.threshold
    T, K, N = w.T, w.K, w.N
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X_np, W_np, _ = workloads.make(args.workload, **shape)
    X0 = torch.from_numpy(X_np).to(dev)
    W0 = torch.from_numpy(W_np).to(dev)
    s_inv = None
    if args.variant == "sq":
        # offline, once per layer: factors from a calibration batch (the first
        # 512 token rows) and the weight's column maxima; smoothed weight codes
        ax = li8.smoothquant_column_absmax(X0[:512])
        s_f, s_inv = li8.smoothquant_factors(ax, li8.smoothquant_column_absmax(W0), 0.5)
        Wq0, sW0 = li8.smoothquant_quantize_weight(W0, s_f)
    else:
        Wq0, sW0 = li8.quantize_weight(W0)

    # Buffer sets.  Warm: one set, so the call's operands stay in the caches
    # between calls.  Cold: enough copies that the calls of a cycle touch
    # more than twice the 256 MB Infinity Cache, so every call reads its
    # weight and activations from HBM.  Both are measured; `value` is the
    # warm one unless --cold.
    touched = 2 * T * K + N * K + 2 * T * N + T * K + 4 * (T + N)
    ncold = max(2, -(-2 * 256 * 2**20 // touched))
    nsets = ncold if args.cold else 1      # the sets of the primary measurement

    def new_set(first):
        st_ = dict(X=X0 if first else X0.clone(), Wq=Wq0 if first else Wq0.clone(),
                   sW=sW0 if first else sW0.clone(),
                   ws=li8.new_workspace(T, K, N, dev),
                   Y=torch.empty((T, N), dtype=torch.float16, device=dev))
        if args.variant == "fp16w":
            st_["W"] = W0 if first else W0.clone()
        if args.variant == "cached":
            st_["cache"] = li8.new_cache(K, N, dev)
        return st_

    sets = [new_set(i == 0) for i in range(ncold)]
    X, W, Wq, sW, ws, Y = X0, W0, Wq0, sW0, sets[0]["ws"], sets[0]["Y"]
    torch.cuda.synchronize()

    if args.variant == "sq":
        def call(b):
            li8.smoothquant_linear(b["X"], s_inv, b["Wq"], b["sW"], out=b["Y"], workspace=b["ws"])

        def prep(b):
            li8.smoothquant_prepare(b["X"], s_inv, N, b["ws"])

        def gemm(b):
            li8.gemm(b["Wq"], b["sW"], T, b["ws"], out=b["Y"])
    elif args.variant == "cached":
        def call(b):
            li8.linear_cached(b["X"], b["Wq"], b["sW"], b["cache"], thr, out=b["Y"],
                              workspace=b["ws"])

        def prep(b):
            li8.prepare_cached(b["X"], b["Wq"], thr, b["ws"], b["cache"])

        def gemm(b):
            li8.gemm_cached(b["Wq"], b["sW"], T, b["ws"], b["cache"], out=b["Y"])
    elif args.variant == "fp16w":
        def call(b):
            li8.linear_fp16w(b["X"], b["Wq"], b["sW"], b["W"], thr, out=b["Y"], workspace=b["ws"])

        def prep(b):
            li8.prepare_fp16w(b["X"], b["W"], thr, b["ws"])

        def gemm(b):
            li8.gemm_fp16w(b["Wq"], b["sW"], b["W"], T, b["ws"], out=b["Y"])
    else:
        def call(b):
            li8.linear(b["X"], b["Wq"], b["sW"], thr, out=b["Y"], workspace=b["ws"])

        def prep(b):
            li8.prepare(b["X"], b["Wq"], thr, b["ws"])

        def gemm(b):
            li8.gemm(b["Wq"], b["sW"], T, b["ws"], out=b["Y"])

    for i in range(max(args.warmup, ncold)):
        call(sets[i % ncold])
    torch.cuda.synchronize()
    y_eager = Y.clone()

    def capture(fn, reps, nuse):
        """A HIP graph of `reps` back-to-back calls of fn, cycling over the
        first `nuse` buffer sets (no allocation inside)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(sets[0])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                fn(sets[r % nuse])
        torch.cuda.synchronize()
        return g

    def same_as_eager(what, nuse):
        for b in sets[:nuse]:
            if not torch.equal(b["Y"].view(torch.int16), y_eager.view(torch.int16)):
                raise RuntimeError(f"{what}: graph replay differs from the eager call")

    def timed_calls(nuse):
        """Wall-clock and HIP-event ms per call of one graph of `steps` calls
        over `nuse` buffer sets.  The K timed steps are one HIP graph of K
        calls of the product entry point, so that the host's per-call launch
        cost (Python, ctypes) does not pace a short call; the graph's output
        is checked against the eager call before and after timing."""
        g = capture(call, args.steps, nuse)
        for b in sets[:nuse]:
            b["Y"].zero_()
        g.replay()
        torch.cuda.synchronize()
        if args.steps >= nuse:
            same_as_eager("linear", nuse)
        # untimed replays until the GPU has run the graph for settle_ms: the
        # shader clock ramps over the first ~15 ms of sustained load (a call
        # at 4096x4096x11008 goes 214 -> 202 -> 190 -> 184 us over the first
        # four 20-call replays, then stays), and the timed steps are meant
        # to run at the steady clock, as in a model's forward pass
        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < args.settle_ms:
            g.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if args.steps >= nuse:
            same_as_eager("linear (timed)", nuse)
        del g
        return (t1 - t0) * 1e3 / args.steps, e0.elapsed_time(e1) / args.steps

    ms_step, gpu_ms_step = timed_calls(nsets)
    other_n = 1 if args.cold else ncold
    other_ms, other_gpu_ms = timed_calls(other_n)

    # Per-stage times for the roofline, with HIP events on torch's current
    # stream, which is the stream the library launches on.  The tiled GEMM
    # is timed inside R prepare -> gemm calls, the sequence of the timed
    # steps: back to back, GEMMs run at a lower (power-limited) clock than
    # after the memory-bound prepare stage.  The prepare stage is timed as
    # a graph of R prepare calls (eager launch gaps would dominate it).
    # For few tokens the GEMM is a ~10 us kernel, which a graph of R
    # gemm-only calls times better than events around eager launches.
    R = min(args.steps, 50)
    pl = li8.plan(T, K, N)
    few = pl["path"] in ("few_tokens", "few_tokens_split")
    split = pl["path"] == "few_tokens_split"

    def graph_ms(g):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / R

    if few:
        for b in sets:   # (the fused call leaves the workspaces unwritten)
            prep(b)
        g_gemm = capture(gemm, R, nsets)
        gemm_ms = graph_ms(g_gemm)
        del g_gemm
    else:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(R)]
        torch.cuda.synchronize()
        for i in range(R):
            prep(sets[i % nsets])
            ev[i][0].record()
            gemm(sets[i % nsets])
            ev[i][1].record()
        torch.cuda.synchronize()
        gemm_ms = sum(a.elapsed_time(b) for a, b in ev) / R
    if R >= nsets:
        same_as_eager("prepare + gemm", nsets)
    g_prep = capture(prep, R, nsets)
    prep_ms = graph_ms(g_prep)
    del g_prep

    power = None
    if args.power_seconds > 0:
        for b in sets:
            prep(b)
        torch.cuda.synchronize()
        power = {"what": "amd-smi metric --power --clock every 0.25 s during back-to-back graph "
                         "replays; medians over the samples after the first second: socket power, "
                         "and the mean over the 8 XCDs of the GFX clock",
                 "call": power_samples(capture(call, R, nsets), args.power_seconds)}
        if not few:
            power["gemm"] = power_samples(capture(gemm, R, nsets), args.power_seconds)

    st = li8.export_stages(ws, T, K, N)
    nO = int(st["n_outliers"].cpu()[0])
    nO16 = (nO + 15) // 16 * 16
    ops = 2.0 * T * N * K
    tops = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    # algorithmic bytes of the prepare stage: detection reads X; quantization
    # reads X, writes Xq, sX and the gathered outlier columns of X; the weight
    # gather reads and writes nO16 bytes per weight row, unless the tiled GEMM
    # copies those columns itself (llm_int8_plan's fold range) or the call
    # runs on a few-token path (its kernels read them by index)
    gathers = not few and not (args.variant == "int8w" and pl["fold_lo"] < nO <= pl["fold_hi"])
    prep_bytes = 2 * T * K + 2 * T * K + T * K + 4 * T + 2 * T * nO16
    if gathers:
        prep_bytes += 2 * N * nO16
    if args.variant == "cached":
        # the weight gather is skipped on a hit (every timed call)
        prep_bytes = 2 * T * K + 2 * T * K + T * K + 4 * T + 2 * T * nO16
    if args.variant == "sq":
        # one pass: reads X and the factors' reciprocals, writes Xq and sX
        prep_bytes = 2 * T * K + 4 * K + T * K + 4 * T
    prep_gbps = prep_bytes / (prep_ms * 1e-3) / 1e9

    reference = None
    if not args.no_reference:
        # context only: the vendor library's plain int8 GEMM (int32 output, no
        # dequantization, no outlier columns) on the same shape and codes
        Xq = st["Xq"]
        WqT = Wq.t()
        try:
            for _ in range(5):
                torch._int_mm(Xq, WqT)
            torch.cuda.synchronize()
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            r0.record()
            for _ in range(50):
                torch._int_mm(Xq, WqT)
            r1.record()
            torch.cuda.synchronize()
            ref_us = r0.elapsed_time(r1) / 50 * 1e3
            reference = {"what": "torch._int_mm (hipBLASLt): int8 x int8 -> int32 only, same T, K, N",
                         "us": round(ref_us, 2), "tops": round(ops / (ref_us * 1e-6) / 1e12, 1)}
        except Exception as ex:  # the reference is optional context
            reference = {"what": "torch._int_mm", "error": str(ex)[:200]}

    if args.copy_calibration:
        # one device-to-device copy of 1 GiB of initialized data (four
        # times the last-level cache), whose true traffic is 1 GiB read +
        # 1 GiB written: the scale for the HBM byte counters
        a = torch.full((1 << 30,), 7, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if few and args.variant == "sq":
        # prepare kernel + the few-token GEMM on its workspace; the GEMM
        # stage streams Wq once
        gemm_bytes = N * K + T * K + 4 * T + 2 * T * N + 4 * N
        gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm",
                    "kernel": "k_decode (few-token GEMM on the workspace, no outliers)",
                    "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None}
    elif split:
        # three kernels are the whole call (scan of X, split-K int8 MFMA
        # product, finish); the product streams Wq once.  Timed as the whole
        # call: the split product's own share is in its kernel trace
        src = os.path.join(ROOT, "int8_matmul_amd", "csrc", "decode_split.hip")
        call_bytes = N * K + 2 * T * K + 2 * T * N + 4 * N
        gbps = call_bytes / (gpu_ms_step * 1e-3) / 1e9
        roofline = {"bound": "hbm",
                    "kernel": "the whole call: k_dscan + k_dsplit + k_dfinish (split-K "
                              "few-token path; k_dsplit streams Wq)",
                    "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "traffic": kernel_traffic("split_call", src, args.workload, (T, K, N)) if args.variant == "int8w" else None}
    elif few:
        # one fused kernel is the whole call; it streams Wq once
        src = os.path.join(ROOT, "int8_matmul_amd", "csrc", "decode.hip")
        call_bytes = N * K + 2 * T * K + 2 * T * N + 4 * N
        gbps = call_bytes / (gpu_ms_step * 1e-3) / 1e9
        roofline = {"bound": "hbm",
                    "kernel": "k_decode (the fused few-token layer: detect, quantize, "
                              "int8 MFMA, outlier MFMA, epilogue)",
                    "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "traffic": kernel_traffic("k_decode", src, args.workload, (T, K, N)) if args.variant == "int8w" else None}
    else:
        src = os.path.join(ROOT, "int8_matmul_amd", "csrc", "gemm.hip")
        roofline = {"bound": "mfma",
                    "kernel": "k_gemm (int8 MFMA GEMM + dequant/outlier epilogue)",
                    "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                    "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                    # counters taken on the LLM.int8() call only
                    "traffic": kernel_traffic("k_gemm", src, args.workload, (T, K, N)) if args.variant == "int8w" else None,
                    "clock_adjusted": (clock_adjusted(src, args.workload, (T, K, N), gemm_tops)
                                       if args.variant == "int8w" else None)}

    warm_desc = "warm: one buffer set, reused by every call"
    cold_desc = (f"cold: {ncold} rotating copies of the call's buffers, "
                 f"{ncold * touched / 1e6:.0f} MB touched per cycle")
    if roofline.get("traffic") is not None:
        roofline["traffic_what"] = ("bytes per launch past the L2 (FETCH_SIZE + WRITE_SIZE, scaled by a "
                                    "1 GiB copy; Infinity Cache hits included, so an upper bound on HBM "
                                    "bytes), from the committed counter run on the current kernel source")
    entry = {"sq": "smoothquant_linear", "cached": "llm_int8_linear_cached",
             "fp16w": "llm_int8_linear_fp16w"}.get(args.variant, "llm_int8_linear")
    out = {
        "metric": METRIC.replace("llm_int8_linear", entry),
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "gpu_ms_per_step": round(gpu_ms_step, 5),
        "timing": f"one HIP graph of `steps` {entry} calls, wall clock between "
                  "synchronizations; output checked against an eager call; before it, "
                  f"untimed replays of the same graph for {args.settle_ms:g} ms (the clock "
                  "ramps over the first ~15 ms of sustained load)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.desc if not shape else f"{w.desc}, at T={T} K={K} N={N}",
                   "name": args.workload, "T": T, "K": K, "N": N,
                   "threshold": None if args.variant == "sq" else thr, "n_outliers": nO,
                   "outlier_weight": ("int8w" if args.variant == "cached" else
                                      args.variant if args.variant != "sq" else None),
                   "outlier_cache": args.variant == "cached",
                   "method": ("SmoothQuant-style W8A8, alpha 0.5" if args.variant == "sq"
                              else "LLM.int8() decomposition"),
                   "parallelism": "single GPU",
                   "cache_state": cold_desc if args.cold else warm_desc},
        "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        ("warm" if args.cold else "cold"): {
            "cache_state": warm_desc if args.cold else cold_desc,
            "value": round(ops / (other_ms * 1e-3) / 1e12, 2),
            "ms_per_step": round(other_ms, 5),
            "gpu_ms_per_step": round(other_gpu_ms, 5),
            "pct_int8_peak": round(100.0 * ops / (other_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2)},
        "path": ("prepare kernel + few-token GEMM" if few and args.variant == "sq" else
                 "few-token split-K kernels" if split else
                 "few-token fused kernel" if few else
                 f"prepare kernels + tiled GEMM ({pl['tile_m']}x{pl['tile_n']} tiles"
                 + ("; the GEMM copies the weight's outlier columns)" if (
                     args.variant == "int8w" and pl["fold_lo"] < nO <= pl["fold_hi"]) else ")")),
        "prepare_us": round(prep_ms * 1e3, 2),
        "gemm_us": round(gemm_ms * 1e3, 2),
        "quant_gbps": round(prep_gbps, 1),
        "quant_pct_hbm_peak": round(100.0 * prep_gbps / PEAK_HBM_GBPS, 2),
        "vendor_int8_gemm": reference,
        "roofline": roofline,
    }
    if power is not None:
        out["power"] = power
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(X_np, W_np, w, args.cpu_seconds, args.variant, thr)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
