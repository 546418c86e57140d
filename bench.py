"""Benchmark: block-scaled FP8 linear-layer training pass on one MI355X.

A step is one linear layer's full FP8 pass at the fused MLP gate+up shape of a ~2B decoder
(X [8192, 2048] bf16 = 2 x 4096 tokens, W [12288, 2048], dY [8192, 12288]):
  quantise X along K and along the tokens (one read) and W by 128x128 tiles (+ transposed codes)
  in one launch, fprop Y = X W^T, quantise dY along N and along the tokens (one read), dgrad
  dX = dY W, wgrad dW = dY^T X.  (--unfused: one quantiser pass per orientation, eight launches.)
Inputs are seeded synthetic tensors resident in HBM before timing starts. Before the --warmup
steps, whole steps run for 60 ms of GPU time so that the timed steps do not fall inside the clock
dip that follows the host's input phase.

Printed (one JSON line): value = the three GEMMs' 2*M*N*K flops per step / step GPU time
(quantisers included), the fprop GEMM kernel against the FP8 MFMA roofline, per-kernel event
timings, hipBLASLt's FP8 / BF16 GEMMs on the fprop shape as context, and the CPU oracle timed on
a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--variant auto|mx|promote] [--unfused]
                    [--no-cpu-baseline] [--no-configs] [--no-comparators]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s and % of MI355X FP8 MFMA peak, 1 GPU"
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (AMD published figure, no sparsity)
PEAK_HBM_GBS = 8000.0
WORKLOAD = "mlp_gateup_layer_step"
# launch order of one step (LinearStep.launches)
KERNELS_FUSED = ["quant_x_dual_w_tiles", "fprop_gemm", "quant_dy_dual", "dgrad_gemm", "wgrad_gemm"]
KERNELS_UNFUSED = ["quant_x_rows", "quant_w_tiles", "fprop_gemm", "quant_dy_rows", "dgrad_gemm", "quant_dy_cols",
                   "quant_x_cols", "wgrad_gemm"]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--variant", choices=["auto", "mx", "promote"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="one quantiser pass per orientation (eight launches)")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the per-configuration GEMMs")
    ap.add_argument("--no-comparators", action="store_true", help="skip timing hipBLASLt on the fprop shape")
    ap.add_argument("--only", choices=["fprop_gemm", "hipblaslt_fp8", "quant_dy_dual", "copy"], default=None,
                    help="profiling modes: run only the headline fprop GEMM, hipBLASLt's FP8 GEMM on the same "
                         "E4M3 codes (per-tensor unit scales, for counter comparisons), only the dual-orientation "
                         "dY quantiser, or only a 1 GiB device copy (the calibration kernel for the FETCH_SIZE / "
                         "WRITE_SIZE counters), --steps times")
    ap.add_argument("--summarize-prof", nargs="+", metavar="DIR", default=None,
                    help="print a text summary of rocprofv3 csv output directories and exit (with --steps: "
                         "the number of timed steps at the end of a traced run of layer steps)")
    return ap.parse_args()


def _dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _alg_bytes(name, m, n, k):
    """Algorithmic HBM bytes of one kernel launch (reads + writes, each byte once)."""
    g = 128
    if name in ("quant_x_rows", "quant_x_cols"):
        rows, cols = m, k
        return rows * cols * 2 + rows * cols + (rows * cols // g) * 4
    if name in ("quant_dy_rows", "quant_dy_cols"):
        return m * n * 2 + m * n + (m * n // g) * 4
    if name == "quant_x_dual":  # one read, both code sets and scale sets written
        return m * k * 2 + 2 * (m * k + (m * k // g) * 4)
    if name == "quant_x_dual_w_tiles":
        return _alg_bytes("quant_x_dual", m, n, k) + _alg_bytes("quant_w_tiles", m, n, k)
    if name == "quant_dy_dual":
        return m * n * 2 + 2 * (m * n + (m * n // g) * 4)
    if name == "quant_w_tiles":
        return n * k * 2 + 2 * n * k + (n * k // (g * g)) * 4
    if name == "fprop_gemm":
        return m * k + n * k + m * n * 2 + (k // g) * m * 4 + (n // g) * (k // g) * 4
    if name == "dgrad_gemm":
        return m * n + k * n + m * k * 2 + (n // g) * m * 4 + (n // g) * (k // g) * 4
    if name == "wgrad_gemm":
        return n * m + k * m + n * k * 2 + (m // g) * n * 4 + (m // g) * k * 4
    raise KeyError(name)


def run_step_timed(step, steps, torch):
    """Run `steps` steps with an event after every kernel launch (all on the current stream)."""
    import fp8_block_scaled_pf8_amd._lib as L

    st = torch.cuda.current_stream()
    launches = step.launches()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(steps)]
    for i in range(steps):
        e = evs[i]
        e[0].record(st)
        for j, (name, fn) in enumerate(launches):
            L.check(fn(), name)
            e[j + 1].record(st)
    return [name for name, _ in launches], evs


SETTLE_MS = 60.0


def settle(torch, fn, warm_ms):
    """Run fn back to back, in groups of 10 launches, until at least warm_ms of GPU time has
    passed since the first one. Returns (launches run, GPU ms)."""
    st = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    start.record(st)
    runs, ms = 0, 0.0
    for _ in range(200):
        for _ in range(10):
            fn()
        runs += 10
        end = torch.cuda.Event(enable_timing=True)
        end.record(st)
        end.synchronize()
        ms = start.elapsed_time(end)
        if ms >= warm_ms:
            break
    return runs, ms


def time_steady(torch, fn, reps=50, warm_ms=SETTLE_MS, group=10):
    """Per-launch times (us) of fn once the chip has settled: fn runs back to back for at least
    warm_ms of GPU time first (after an idle host phase the clocks dip for some tens of ms), then
    `reps` launches run in groups of `group` back-to-back launches with an event between groups
    (an event between every two launches would add its marker's gap, some microseconds, to each).
    Returns the median, p10 and p90 over the groups of their mean time per launch, and the host's
    time per launch to enqueue them (a GPU time close to it would be the host's launch rate)."""
    st = torch.cuda.current_stream()
    settle(torch, fn, warm_ms)
    ngroups = max(reps // group, 1)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(ngroups + 1)]
    t0 = time.perf_counter()
    evs[0].record(st)
    for g in range(ngroups):
        for _ in range(group):
            fn()
        evs[g + 1].record(st)
    host_us = (time.perf_counter() - t0) * 1e6 / (ngroups * group)
    torch.cuda.synchronize()
    us = np.array([evs[g].elapsed_time(evs[g + 1]) * 1e3 / group for g in range(ngroups)])
    return float(np.median(us)), float(np.percentile(us, 10)), float(np.percentile(us, 90)), host_us


def time_comparators(torch, pf8, m, n, k, reps=100):
    """On the fprop shape, as context: this library's plain BF16 GEMM (same pipeline, BF16
    operands), and hipBLASLt through torch: FP8 E4M3 with one scale per tensor and per row /
    column (not block scales), and BF16."""
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    a = (torch.randn(m, k, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    b = (torch.randn(n, k, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    sa, sb = torch.ones((m, 1), device=dev), torch.ones((1, n), device=dev)
    ab, bb = a.to(torch.bfloat16), b.to(torch.bfloat16).contiguous()
    y16 = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    cases = {
        "libpf8_bf16": lambda: pf8.gemm_bf16(ab, bb, out=y16),
        "hipblaslt_fp8_tensorwise": lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one,
                                                             out_dtype=torch.bfloat16),
        "hipblaslt_fp8_rowwise": lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16),
        "hipblaslt_bf16": lambda: torch.mm(ab, bb.t()),
    }
    out = {}
    for name, fn in cases.items():
        try:
            us, p10, p90, host_us = time_steady(torch, fn, reps)
            out[name] = {"us": round(us, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                         "host_us_per_launch": round(host_us, 1),
                         "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)}
        except Exception as ex:  # a comparator that torch cannot run is reported, not fatal
            out[name] = {"error": repr(ex)[:200]}
    del a, b, ab, bb, y16
    torch.cuda.empty_cache()
    return {"shape": [m, n, k], "note": "library GEMMs without block scales; context only; per-launch median, p10 "
                                        "and p90 after at least 60 ms of back-to-back launches", **out}


def device_peak_fp8():
    """Dense FP8 MFMA peak from the device itself: compute units x max engine clock x 8192 FLOP per
    clock and CU (rocminfo's GPU agent), beside the published figure. None if rocminfo is unavailable."""
    import re
    import subprocess

    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:  # pragma: no cover - depends on the host
        return None
    for agent in re.split(r"\n(?=\*+\s*\n\s*Agent \d+)", out):
        name = re.search(r"^\s*Name:\s*(\S+)", agent, re.M)
        cus = re.search(r"Compute Unit:\s*(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", agent)
        if name and name.group(1).startswith("gfx") and cus and mhz:
            tflops = int(cus.group(1)) * int(mhz.group(1)) * 1e6 * 8192 / 1e12
            return {"arch": name.group(1), "cus": int(cus.group(1)), "max_clock_mhz": int(mhz.group(1)),
                    "tflops": round(tflops, 1), "source": "rocminfo: CUs x max clock x 8192 FLOP/clk/CU"}
    return None


def time_cold_warm(torch, fn, reps=20, flush_bytes=512 << 20):
    """One kernel launch timed with events, cold (reading a flush_bytes buffer evicts L2 and the 256 MB
    Infinity Cache before every launch, outside the events; a read leaves no dirty lines whose
    write-back would be charged to the kernel) and warm (back to back)."""
    import fp8_block_scaled_pf8_amd._lib as L

    scratch = torch.ones(flush_bytes, dtype=torch.uint8, device="cuda:0")
    st = torch.cuda.current_stream()
    pairs = {"cold": [], "warm": []}
    for _ in range(reps):
        scratch.max()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        L.check(fn(), "cold launch")
        e1.record(st)
        pairs["cold"].append((e0, e1))
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        L.check(fn(), "warm launch")
        e1.record(st)
        pairs["warm"].append((e0, e1))
    torch.cuda.synchronize()
    del scratch
    out = {}
    for kind, evs in pairs.items():
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        out[f"{kind}_us_median"] = round(float(np.median(us)), 2)
        out[f"{kind}_us_p10"] = round(float(np.percentile(us, 10)), 2)
        out[f"{kind}_us_p90"] = round(float(np.percentile(us, 90)), 2)
    return out


def time_config_gemms(pf8, torch, reps=100):
    """Kernel time of each configured GEMM (inputs quantised on the GPU first): median, p10 and p90
    over groups of 10 back-to-back launches of the mean time per launch, `reps` launches in all,
    after at least 60 ms of back-to-back launches (the inputs are built on the host, so the GPU
    comes out of an idle phase before every configuration)."""
    from workloads import WORKLOADS, generate

    out = {}
    for key in ["attn_fprop", "mlp_gateup_fprop", "mlp_down_fprop_dgrad", "wgrad"]:
        wl = WORKLOADS[key]
        t = generate(wl)
        dev = {name: _dev_bf16(b, torch) for name, b in t.items()}
        for layout, m, n, k in wl.gemms:
            if layout == "fprop":
                qx, sx = pf8.quant_act_1x128(dev["X"], "cols")
                qw, _, sw = pf8.quant_w_128x128(dev["W"], transposed=False)
                fn = lambda qx=qx, sx=sx, qw=qw, sw=sw: pf8.fprop(qx, sx, qw, sw, out=y)  # noqa: E731
            elif layout == "dgrad":
                qdy, sdy = pf8.quant_act_1x128(dev["dY"], "cols")
                _, qwt, sw = pf8.quant_w_128x128(dev["W"])
                fn = lambda qdy=qdy, sdy=sdy, qwt=qwt, sw=sw: pf8.dgrad(qdy, sdy, qwt, sw, out=y)  # noqa: E731
            else:
                qdyt, sdyt = pf8.quant_act_1x128(dev["dY"], "rows")
                qxt, sxt = pf8.quant_act_1x128(dev["X"], "rows")
                fn = lambda a=qdyt, sa=sdyt, b=qxt, sb=sxt: pf8.wgrad(a, sa, b, sb, out=y)  # noqa: E731
            y = pf8.ops.result_buffer(m, n, torch.bfloat16, "cuda:0")
            us, p10, p90, host_us = time_steady(torch, fn, reps)
            tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
            out[f"{key}:{layout}"] = {"m": m, "n": n, "k": k, "us": round(us, 2), "us_p10": round(p10, 2),
                                      "us_p90": round(p90, 2), "host_us_per_launch": round(host_us, 1),
                                      "tflops": round(tf, 1),
                                      "frac_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del dev
        torch.cuda.empty_cache()
    return out


def cpu_baseline(sample_tokens=8192):
    """The oracle as it stands, on the first `sample_tokens` tokens of the same layer pass."""
    import oracle
    from workloads import generate

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t = generate(WORKLOAD)
    x, w, dy = t["X"][:sample_tokens], t["W"], t["dY"][:sample_tokens]
    m, k = x.shape
    n = w.shape[0]
    t0 = time.perf_counter()
    qx, sx = oracle.quant_act_1x128(x, "cols")
    qw, qwt, sw = oracle.quant_w_128x128(w)
    oracle.gemm_fprop(qx, sx, qw, sw)
    qdy, sdy = oracle.quant_act_1x128(dy, "cols")
    oracle.gemm_dgrad(qdy, sdy, qwt, sw)
    qdyt, sdyt = oracle.quant_act_1x128(dy, "rows")
    qxt, sxt = oracle.quant_act_1x128(x, "rows")
    oracle.gemm_wgrad(qdyt, sdyt, qxt, sxt)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * m * n * k
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover - not Linux
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2), "cpu_model": cpu_model,
            "sample": f"the same layer pass (quantisers and the three GEMMs, float64 oracle) on {m} of the 8192 tokens: "
                      f"X [{m},{k}], W [{n},{k}], dY [{m},{n}]; host cpus={os.cpu_count()} "
                      f"affinity={len(os.sched_getaffinity(0))}"}


GEMM_SRC = os.path.join(ROOT, "fp8_block_scaled_pf8_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fprop_gemm_8192x12288x2048_traffic.txt")


def gemm_source_hash() -> str:
    import hashlib

    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per fprop launch from the committed counter summary, if it matches this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines() if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("gemm_source_sha256_16", "").strip() != gemm_source_hash():
        return None  # the kernel changed since the counters were taken
    return int(float(kv["hbm_bytes_per_launch"]))


def only_mode(args, torch, pf8):
    """Minimal launch loops for rocprofv3 (no timing output beyond one line)."""
    from workloads import generate

    if args.only == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": args.steps}), flush=True)
        return
    if args.only == "quant_dy_dual":
        dy = _dev_bf16(generate(WORKLOAD, only=["dY"])["dY"], torch)
        for _ in range(args.steps):
            pf8.quant_act_dual(dy)
        torch.cuda.synchronize()
        print(json.dumps({"only": "quant_dy_dual", "rows": dy.shape[0], "cols": dy.shape[1],
                          "launches": args.steps}), flush=True)
        return
    t = generate(WORKLOAD, only=["X", "W"])
    qx, sx = pf8.quant_act_1x128(_dev_bf16(t["X"], torch), "cols")
    qw, _, sw = pf8.quant_w_128x128(_dev_bf16(t["W"], torch), transposed=False)
    y = pf8.ops.result_buffer(qx.shape[0], qw.shape[0], torch.bfloat16, "cuda:0")  # the step's layout
    if args.only == "hipblaslt_fp8":
        # context for counter comparisons: hipBLASLt's FP8 GEMM (one unit scale per tensor) on the
        # very same E4M3 codes
        a8, b8 = qx.view(torch.float8_e4m3fn), qw.view(torch.float8_e4m3fn)
        one = torch.ones((), device="cuda:0")
        for _ in range(args.steps):
            torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    else:
        for _ in range(args.steps):
            pf8.fprop(qx, sx, qw, sw, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "m": qx.shape[0], "n": qw.shape[0], "k": qx.shape[1],
                      "launches": args.steps, "gemm_source_sha256_16": gemm_source_hash()}), flush=True)


def _counter_step_positions(path, timed_steps):
    """Per launch position of the layer step, the counters of the timed steps (the run of whole
    steps ends with the timed steps, then as many event-timed ones), and for the GEMMs the MFMA
    busy cycles per SIMD (1024 SIMDs) over the GPU-active cycles per XCD (8 XCDs)."""
    import csv
    from collections import OrderedDict

    disp = OrderedDict()
    for r in csv.DictReader(open(path)):
        rec = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                      "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        rec[r["Counter_Name"]] = float(r["Counter_Value"])
    pf8_rows = [disp[i] for i in sorted(disp) if "pf8::" in disp[i]["name"]]
    names = [r["name"] for r in pf8_rows]
    kernels = KERNELS_FUSED if any("quant_fwd" in n for n in names) else KERNELS_UNFUSED
    nk = len(kernels)
    nsteps = 0
    while (nsteps + 1) * nk <= len(names) and names[nsteps * nk:(nsteps + 1) * nk] == names[:nk]:
        nsteps += 1
    if nsteps < 2 * timed_steps:
        return
    lo, hi = nsteps - 2 * timed_steps, nsteps - timed_steps
    for j, kname in enumerate(kernels):
        v = [pf8_rows[i * nk + j] for i in range(lo, hi)]
        counters = sorted(c for c in v[0] if c not in ("name", "ns"))
        avg = {c: sum(x[c] for x in v) / len(v) for c in counters}
        ns = sum(x["ns"] for x in v) / len(v)
        line = " ".join(f"{c}={avg[c]:.6g}" for c in counters)
        print(f"timed step position {kname}: dispatches={len(v)} avg_ns={ns:.0f} {line}")
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) > 0 and avg.get("GRBM_GUI_ACTIVE", 0) > 0:
            busy, act = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024, avg["GRBM_GUI_ACTIVE"] / 8
            print(f"timed step position {kname}: mfma_busy_cycles_per_simd={busy:.0f} "
                  f"active_cycles_per_xcd={act:.0f} mfma_busy_frac={busy / act:.3f}")


def summarize_prof(dirs, timed_steps=50):
    """Text summary of rocprofv3 csv directories: kernel stats and per-dispatch counter averages.
    For a kernel trace of the layer step, also the per-launch-position averages over every step
    after the first two, over the timed steps and over the event-timed steps that follow them
    (`timed_steps` each, at the end of the run of steps), with the mean gap between launches."""
    import csv
    import glob
    from collections import defaultdict

    for d in dirs:
        print(f"## {d}")
        for f in sorted(glob.glob(os.path.join(d, "*kernel_stats.csv"))):
            for r in csv.DictReader(open(f)):
                print(f"kernel {r['Name'][:90]}: calls={r['Calls']} avg_ns={float(r['AverageNs']):.0f} "
                      f"min_ns={r['MinNs']} max_ns={r['MaxNs']} pct={float(r['Percentage']):.2f}")
        for f in sorted(glob.glob(os.path.join(d, "*kernel_trace.csv"))):
            # per-position view of the layer step: the libpf8 launches repeat in LinearStep order
            rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
            pf8_rows = [r for r in rows if "pf8::" in r["Kernel_Name"]]
            seq = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in pf8_rows]
            dual = any("quant_fwd" in r["Kernel_Name"] for r in pf8_rows)
            kernels = KERNELS_FUSED if dual else KERNELS_UNFUSED
            # the step's launches come first; later launches (the FP32-accumulate timing) end the run
            names = [r["Kernel_Name"] for r in pf8_rows]
            nsteps = 0
            while (nsteps + 1) * len(kernels) <= len(names) and \
                    names[nsteps * len(kernels):(nsteps + 1) * len(kernels)] == names[:len(kernels)]:
                nsteps += 1
            nk = len(kernels)

            def positions(label, lo, hi):
                for j, name in enumerate(kernels):
                    v = [seq[i * nk + j] for i in range(lo, hi)]
                    print(f"{label} {name}: dispatches={len(v)} avg_ns={sum(v) / len(v):.0f} "
                          f"min_ns={min(v)} max_ns={max(v)}")
                gaps = [int(pf8_rows[i * nk + j + 1]["Start_Timestamp"]) - int(pf8_rows[i * nk + j]["End_Timestamp"])
                        for i in range(lo, hi) for j in range(nk - 1)]
                print(f"{label} gap between launches: avg_ns={sum(gaps) / len(gaps):.0f}")

            if nsteps >= 3:
                positions("step position", 2, nsteps)  # every step but the first two
            if nsteps >= 2 * timed_steps:
                # bench.py ends its run of steps with the timed steps (no event between launches),
                # then as many steps with an event after every launch (the per-launch breakdown)
                positions("timed step position", nsteps - 2 * timed_steps, nsteps - timed_steps)
                positions("event-timed step position", nsteps - timed_steps, nsteps)
        for f in sorted(glob.glob(os.path.join(d, "*counter_collection.csv"))):
            agg = defaultdict(list)
            for r in csv.DictReader(open(f)):
                agg[(r["Kernel_Name"][:90], r["Counter_Name"])].append(float(r["Counter_Value"]))
            for (kname, cname), v in sorted(agg.items()):
                print(f"counter {cname} kernel {kname}: dispatches={len(v)} avg={sum(v) / len(v):.6g}")
            _counter_step_positions(f, timed_steps)


def main():
    args = parse_args()
    if args.summarize_prof:
        summarize_prof(args.summarize_prof, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the path has no multi-GPU "
              "mode: each GPU would run this same per-layer pass on its own micro-batch", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_block_scaled_pf8_amd as pf8
    from workloads import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.only:
        only_mode(args, torch, pf8)
        return
    variant = {"auto": pf8.PF8_GEMM_AUTO, "mx": pf8.PF8_GEMM_MX_SCALED, "promote": pf8.PF8_GEMM_PROMOTE}[args.variant]
    wl = WORKLOADS[WORKLOAD]
    t = generate(wl)
    x, w, dy = (_dev_bf16(t[nm], torch) for nm in ("X", "W", "dY"))
    del t
    step = pf8.LinearStep(x, w, dy, variant=variant, fused=not args.unfused)
    m, n, k = step.m, step.n, step.k
    print(f"# workload {WORKLOAD}: M={m} N={n} K={k}, variant={args.variant}, "
          f"{'unfused' if args.unfused else 'dual-orientation'} quantisers", file=sys.stderr, flush=True)

    # Settle: after the host phase that builds the inputs the GPU has idled for seconds, and its
    # power management then runs the first ~25 ms of work through a clock dip and recovery. A
    # training loop runs steps back to back, so the steady state is the one to time: whole steps
    # run until 60 ms of GPU time have passed (the same floor as the per-configuration timings
    # below), then the --warmup steps, then exactly --steps timed steps. Reported as settle_steps.
    settle_steps, settle_ms = settle(torch, step.run, SETTLE_MS)
    for _ in range(args.warmup):
        step.run()
    st = torch.cuda.current_stream()
    # The timed steps: exactly --steps steps with one event before and one after them, as a
    # training loop runs them (no event between launches).
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(st)
    for _ in range(args.steps):
        step.run()
    ev_end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step_wall = wall * 1e3 / args.steps
    ms_step = ev_start.elapsed_time(ev_end) / args.steps
    # The per-launch breakdown: as many steps again, with an event after every launch (on the
    # launch stream). Each event costs the step a few microseconds, so these steps run longer.
    names, evs = run_step_timed(step, args.steps, torch)
    torch.cuda.synchronize()
    per = {name: 0.0 for name in names}
    per_all = {name: [] for name in names}
    gpu_ms = 0.0
    for e in evs:
        for j, name in enumerate(names):
            dt = e[j].elapsed_time(e[j + 1])
            per[name] += dt
            per_all[name].append(dt * 1e3)
        gpu_ms += e[0].elapsed_time(e[-1])
    per = {kname: v / args.steps for kname, v in per.items()}
    ms_step_instr = gpu_ms / args.steps
    flops = step.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    kernels = {}
    for name in names:
        ms = per[name]
        entry = {"us": round(ms * 1e3, 2), "us_median": round(float(np.median(per_all[name])), 2),
                 "us_p10": round(float(np.percentile(per_all[name], 10)), 2),
                 "us_p90": round(float(np.percentile(per_all[name], 90)), 2)}
        if name.endswith("gemm"):
            tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            entry.update(tflops=round(tf, 1), frac_peak=round(tf / PEAK_FP8_TFLOPS, 4))
        else:
            gbs = _alg_bytes(name, m, n, k) / (ms * 1e-3) / 1e9
            entry.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        kernels[name] = entry
    # the FP32 weight gradient accumulated into a main gradient (pf8_block_gemm_f32, accumulate=1), on
    # the step's own codes, timed the same way: reported beside the step, not part of it
    main_grad = torch.zeros((n, k), dtype=torch.float32, device="cuda:0")
    settle(torch, lambda: pf8.wgrad_f32(step.qdyt, step.sdyt, step.qxt, step.sxt, out=main_grad, accumulate=True),
           SETTLE_MS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(20):
        pf8.wgrad_f32(step.qdyt, step.sdyt, step.qxt, step.sxt, out=main_grad, accumulate=True)
    e1.record(st)
    torch.cuda.synchronize()
    f32_us = e0.elapsed_time(e1) * 1e3 / 20
    del main_grad
    # a later micro-batch of the same optimizer step: W's codes (made by the steps above) reused
    settle(torch, lambda: step.run(weight_codes=False), SETTLE_MS)  # after a change of load, too, the clocks move
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        step.run(weight_codes=False)
    e1.record(st)
    torch.cuda.synchronize()
    mb_ms = e0.elapsed_time(e1) / args.steps
    # cold-cache (L2 and Infinity Cache evicted before every launch) against warm timing of the
    # headline GEMM and of the dY quantiser, on the step's own buffers
    thunks = dict(step.launches())
    cache = {"flush_bytes": 512 << 20}
    for name in ("fprop_gemm", "quant_dy_dual"):
        if name in thunks:
            cache[name] = time_cold_warm(torch, thunks[name])
    fp_ms = per["fprop_gemm"]
    achieved = 2.0 * m * n * k / (fp_ms * 1e-3) / 1e12
    traffic = measured_traffic() if args.variant == "auto" else None
    roofline = {"bound": "mfma", "kernel": "fprop_gemm", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM, calibrated FETCH_SIZE + WRITE_SIZE)",
                "algorithmic_bytes_per_launch": _alg_bytes("fprop_gemm", m, n, k),
                "algorithmic_flops_per_launch": 2 * m * n * k, "avg_launch_us": round(fp_ms * 1e3, 2)}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": settle_steps, "settle_gpu_ms": round(settle_ms, 1),
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": WORKLOAD, "m_tokens": m, "n": n, "k": k, "gemms": ["fprop", "dgrad", "wgrad"],
                   "variant": args.variant, "quantisers": "single" if args.unfused else "dual",
                   "launches_per_step": len(names), "title": wl.title},
        "pct_of_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "wall_ms_per_step": round(ms_step_wall, 4),
        "instrumented_ms_per_step": round(ms_step_instr, 4),
        # every step of the per-launch breakdown and its fprop GEMM, in order (a step inside a clock
        # transient would show here)
        "step_us_each": [round(e[0].elapsed_time(e[-1]) * 1e3, 1) for e in evs],
        "fprop_us_each": [round(v, 1) for v in per_all["fprop_gemm"]],
        "roofline": roofline,
        "kernels": kernels,
        "wgrad_f32_accumulate": {"us": round(f32_us, 2), "tflops": round(2.0 * m * n * k / (f32_us * 1e-6) / 1e12, 1),
                                 "note": "dW in FP32 added to a main gradient (not part of the step)"},
        "micro_batch_step": {"ms_per_step": round(mb_ms, 4), "tflops": round(flops / (mb_ms * 1e-3) / 1e12, 1),
                             "launches": len(step.launches(weight_codes=False)),
                             "note": "the step of a later micro-batch of one optimizer step: W's codes reused, "
                                     "X's dual quantiser alone (not the headline value)"},
        "cache": cache,
        "peak_device": device_peak_fp8(),
    }
    del step, x, w, dy
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["config_gemms"] = time_config_gemms(pf8, torch)
    if not args.no_comparators:
        result["comparators"] = time_comparators(torch, pf8, m, n, k)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
