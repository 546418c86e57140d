"""Host logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte counts behind the
roofline figures, the device-peak parser and the per-launch-position profile summary."""
import csv
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_algorithmic_bytes():
    b = _bench()
    m, n, k, g = 8192, 12288, 2048, 128
    # GEMM: both code operands once, the BF16 result, the activation scales (one per row and K block)
    # and the weight tile scales
    assert b._alg_bytes("fprop_gemm", m, n, k) == m * k + n * k + 2 * m * n + (k // g) * m * 4 + (n // g) * (k // g) * 4
    assert b._alg_bytes("fprop_gemm", m, n, k) == 243_800_064  # 243.8 MB, the headline GEMM's figure
    # dual quantiser: one BF16 read, two code sets and two scale sets written
    assert b._alg_bytes("quant_dy_dual", m, n, k) == 2 * m * n + 2 * (m * n + (m * n // g) * 4)
    # weight tiles: BF16 read, codes and transposed codes, one scale per 128x128 tile
    assert b._alg_bytes("quant_w_tiles", m, n, k) == 2 * n * k + 2 * n * k + (n * k // (g * g)) * 4
    # the fused forward quantiser moves exactly what its two parts move
    assert b._alg_bytes("quant_x_dual_w_tiles", m, n, k) == (b._alg_bytes("quant_x_dual", m, n, k)
                                                             + b._alg_bytes("quant_w_tiles", m, n, k))


_ROCMINFO = """*******
Agent 1
*******
  Name:                    AMD EPYC 9575F 64-Core Processor
  Marketing Name:          AMD EPYC 9575F 64-Core Processor
  Compute Unit:            128
  Max Clock Freq. (MHz):   3300
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Compute Unit:            256
  Max Clock Freq. (MHz):   2400
  ISA Info:
    ISA 1
      Name:                    amdgcn-amd-amdhsa--gfx950:sramecc+:xnack-
"""


def test_device_peak_from_rocminfo(monkeypatch):
    b = _bench()

    class Out:
        stdout = _ROCMINFO

    monkeypatch.setattr(subprocess, "run", lambda *a, **kw: Out())
    peak = b.device_peak_fp8()
    assert peak["arch"] == "gfx950" and peak["cus"] == 256 and peak["max_clock_mhz"] == 2400
    assert peak["tflops"] == 5033.2  # 256 CUs x 2.4 GHz x 8192 FLOP per clock and CU

    def missing(*a, **kw):
        raise FileNotFoundError("rocminfo")

    monkeypatch.setattr(subprocess, "run", missing)
    assert b.device_peak_fp8() is None


def test_profile_summary_step_positions(tmp_path, capsys):
    """The per-position view takes the leading run of whole steps and stops at other launches. It
    averages every step but the first two, then the timed steps and the event-timed steps that end
    the run (timed_steps each), with the mean gap between a step's launches."""
    b = _bench()
    step = ["pf8::quant_fwd_kernel(pf8::FwdQuantArgs)",
            "void pf8::gemm_mx_kernel<256, 256, false, false, 5, false, false>(pf8::GemmArgs, int, int)",
            "pf8::quant_dual_kernel(unsigned short const*)",
            "void pf8::gemm_mx_kernel<256, 256, false, false, 5, false, false>(pf8::GemmArgs, int, int)",
            "void pf8::gemm_mx_kernel<192, 256, true, false, 5, false, false>(pf8::GemmArgs, int, int)"]
    rows, t = [], 0
    for i in range(9):  # steps 0-2: settle and warm-up, 3-5: timed, 6-8: event-timed (wider gaps)
        gap = 500 if i >= 6 else 10
        for j, name in enumerate(step):
            dur = 1000 * (j + 1) + i
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + gap
    for _ in range(2):  # FP32-accumulate launches after the step, not part of it
        rows.append({"Kernel_Name": "void pf8::gemm_mx_kernel<192, 256, true, true, 5, true, false>(...)",
                     "Start_Timestamp": t, "End_Timestamp": t + 99999})
        t += 100009
    with open(tmp_path / "step_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)
    b.summarize_prof([str(tmp_path)], timed_steps=3)
    out = capsys.readouterr().out.splitlines()
    for label, steps, mean_i, gap in (("step position", 7, 5, (16 * 10 + 12 * 500) / 28),
                                      ("timed step position", 3, 4, 10), ("event-timed step position", 3, 7, 500)):
        lines = [ln for ln in out if ln.startswith(label + " ") and "gap between" not in ln]
        assert [ln.split(":")[0].split()[-1] for ln in lines] == b.KERNELS_FUSED
        for j, ln in enumerate(lines):
            assert f"dispatches={steps} avg_ns={1000 * (j + 1) + mean_i} " in ln
        assert f"{label} gap between launches: avg_ns={gap:.0f}" in out


def test_profile_summary_counter_step_positions(tmp_path, capsys):
    """Counter view of the layer step: per launch position, the timed steps' counter averages (the
    run of steps ends with timed_steps timed and as many event-timed steps), and for a GEMM the MFMA
    busy cycles per SIMD over the active cycles per XCD."""
    b = _bench()
    step = ["pf8::quant_fwd_kernel(pf8::FwdQuantArgs)",
            "void pf8::gemm_mx_persistent_kernel<256, false>(pf8::GemmArgs, int, int)",
            "pf8::quant_dual_kernel(unsigned short const*)",
            "void pf8::gemm_mx_kernel<256, 256, false, false, 5, false, false>(pf8::GemmArgs, int, int)",
            "void pf8::gemm_mx_persistent_kernel<192, true>(pf8::GemmArgs, int, int)"]
    rows, disp, t = [], 0, 0
    for i in range(7):  # steps 0: warm-up, 1-3: timed, 4-6: event-timed
        for j, name in enumerate(step):
            disp += 1
            active = 8000.0 * (j + 1) + (0 if 1 <= i <= 3 else 1e6)  # only the timed steps give the expected mean
            busy = 1024.0 * 600 * (j % 2)  # the GEMM positions (1, 3) are busy 600 cycles per SIMD
            for cname, val in (("GRBM_GUI_ACTIVE", active), ("SQ_VALU_MFMA_BUSY_CYCLES", busy)):
                rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": cname, "Counter_Value": val,
                             "Start_Timestamp": t, "End_Timestamp": t + 100 * (j + 1)})
            t += 1000
    rows.append({"Dispatch_Id": disp + 1, "Kernel_Name": "void pf8::gemm_mx_kernel<192, 256, true, true, 5, true, false>",
                 "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1.0, "Start_Timestamp": t, "End_Timestamp": t + 1})
    path = tmp_path / "pmc_counter_collection.csv"
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        wr.writerows(rows)
    b._counter_step_positions(str(path), 3)
    out = capsys.readouterr().out.splitlines()
    for j, name in enumerate(b.KERNELS_FUSED):
        assert f"timed step position {name}: dispatches=3 avg_ns={100 * (j + 1)} GRBM_GUI_ACTIVE={8000 * (j + 1)} " in \
            next(ln for ln in out if ln.startswith(f"timed step position {name}: dispatches"))
    busy = [ln for ln in out if "mfma_busy_frac" in ln]
    assert busy == ["timed step position fprop_gemm: mfma_busy_cycles_per_simd=600 active_cycles_per_xcd=2000 "
                    "mfma_busy_frac=0.300",
                    "timed step position dgrad_gemm: mfma_busy_cycles_per_simd=600 active_cycles_per_xcd=4000 "
                    "mfma_busy_frac=0.150"]
