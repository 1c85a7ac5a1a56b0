"""Host-only checks of the measurement code: bench.py's one-GPU contract and
roofline arithmetic, the algorithmic FLOP and byte counts against the sizes of
the tensors a layer is built from, and the arithmetic of profiling.py's
rocprofv3 summaries on small hand-made CSV files."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_picks_the_bound_by_the_ridge():
    import bench
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)   # FLOP per byte
    # above the ridge: MFMA-bound, achieved in TFLOP/s
    r = bench.roofline_of(2.0 * ridge * 1e9, 1e9, 1e-3, True)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2.0 * ridge)
    assert r["frac"] == pytest.approx(2.0 * ridge / bench.PEAK_BF16_TFLOPS)
    # below it: HBM-bound, achieved in GB/s
    r = bench.roofline_of(0.5 * ridge * 1e9, 1e9, 1e-3, True)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(1000.0 / bench.PEAK_HBM_GBS)
    # fp32 layers are priced against the fp32 peak
    r = bench.roofline_of(1e15, 1e9, 1.0, False)
    assert r["peak"] == bench.PEAK_FP32_TFLOPS


@pytest.mark.parametrize("dtype,n_shared", [("bf16", 0), ("bf16", 2), ("fp32", 1)])
def test_algorithmic_counts_match_the_layer_tensors(dtype, n_shared):
    """FLOPs and bytes from the shapes of the tensors a layer is made of: each
    kept row multiplies through one expert's three matrices, every token
    through the router and the shared experts; the active experts' weights,
    the shared weights, the router, x and the fp32 y move once."""
    from dynamic_task_scheduling_amd import configs
    from dynamic_task_scheduling_amd.synth import make_layer
    s = configs.LayerShape(T=40, d=64, E=8, k=2, f=96, dtype=dtype, n_shared=n_shared,
                           f_shared=32 if n_shared else 0)
    t = make_layer(s, "count", 0, 0, "cpu")
    counts = [11, 0, 7, 0, 30, 1, 0, 31]          # any routing with these per-expert rows
    R, active = sum(counts), sum(c > 0 for c in counts)
    per_row = 2 * (t["w_gate"][0].numel() + t["w_up"][0].numel() + t["w_down"][0].numel())
    shared = 0
    if n_shared:
        shared = 2 * sum(t[n].numel() for n in ("ws_gate", "ws_up", "ws_down"))
    flops = 2 * s.T * t["w_router"].numel() + R * per_row + s.T * shared
    assert configs.flops(s, R) == pytest.approx(flops)
    def nbytes(x):
        return x.numel() * x.element_size()
    w_one = nbytes(t["w_gate"][0]) + nbytes(t["w_up"][0]) + nbytes(t["w_down"][0])
    b = active * w_one + nbytes(t["w_router"]) + nbytes(t["x"]) + 4 * s.T * s.d
    if n_shared:
        b += sum(nbytes(t[n]) for n in ("ws_gate", "ws_up", "ws_down"))
    assert configs.algo_bytes(s, active) == pytest.approx(b)


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    from dynamic_task_scheduling_amd import profiling
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # two dispatches of the kernel, each reported in two parts (summed per dispatch)
    fetch = _write_csv(tmp_path / "f.csv", hdr, [
        [1, "moe::k_dynamic<bf16>", "FETCH_SIZE", 300], [1, "moe::k_dynamic<bf16>", "FETCH_SIZE", 100],
        [2, "moe::k_dynamic<bf16>", "FETCH_SIZE", 500], [2, "moe::k_dynamic<bf16>", "FETCH_SIZE", 300],
        [3, "other", "FETCH_SIZE", 1e9]])
    write = _write_csv(tmp_path / "w.csv", hdr, [
        [1, "moe::k_dynamic<bf16>", "WRITE_SIZE", 64], [2, "moe::k_dynamic<bf16>", "WRITE_SIZE", 192]])
    # a 1-MiB copy that the counters report as 512 KiB read and 1024 KiB written
    cf = _write_csv(tmp_path / "cf.csv", hdr, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512]])
    cw = _write_csv(tmp_path / "cw.csv", hdr, [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024]])
    out = tmp_path / "t.json"
    profiling.traffic(argparse.Namespace(fetch=fetch, write=write, copy_fetch=cf, copy_write=cw, copy_mib=1,
                                         workload="w", kernel="k_dynamic<", algo_bytes=1.0,
                                         command=["c"], out=str(out)))
    d = json.load(open(out))
    assert d["fetch_kib_per_dispatch"] == pytest.approx(600.0)      # (400 + 800) / 2
    assert d["write_kib_per_dispatch"] == pytest.approx(128.0)
    assert d["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert d["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert d["traffic_bytes_per_launch"] == pytest.approx((600.0 * 2.0 + 128.0) * 1024.0)


def test_counter_summary_derives_clock_and_mfma_busy(tmp_path):
    from dynamic_task_scheduling_amd import profiling
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    cycles = 1.0e6                                   # per XCD
    rows = [[1, "moe::k_dynamic<bf16>", "GRBM_GUI_ACTIVE", 8 * cycles],
            [1, "moe::k_dynamic<bf16>", "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * cycles],
            [1, "moe::k_dynamic<bf16>", "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * cycles],
            [1, "moe::k_dynamic<bf16>", "SQ_WAVE_CYCLES", 1024 * cycles / 4],
            [1, "moe::k_dynamic<bf16>", "SQ_LDS_BANK_CONFLICT", 10],
            [1, "moe::k_dynamic<bf16>", "SQ_LDS_IDX_ACTIVE", 1000],
            [2, "not_this_kernel", "GRBM_GUI_ACTIVE", 1.0]]
    c = _write_csv(tmp_path / "sq.csv", hdr, rows)
    out = tmp_path / "c.md"
    profiling.counters(argparse.Namespace(csv=c, workload="w", kernel="k_dynamic<", command="c",
                                          duration_us=500.0, note="", out=str(out)))
    text = open(out).read()
    assert "shader clock = cycles / kernel duration (500.0 us) = 2.00 GHz" in text
    assert "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) = 50.0%" in text
    assert "SQ_WAVE_CYCLES = 100.0% of wave-cycles" in text
    assert "LDS bank-conflict cycles / LDS active cycles = 1.0%" in text


def test_kernel_stats_lists_matching_kernels_and_timed_median(tmp_path):
    from dynamic_task_scheduling_amd import profiling
    stats = _write_csv(tmp_path / "s.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"], [
        ["void moe::k_dynamic<unsigned short, false>(moe::Params)", 5, 5000, 1000, 900, 1200],
        ["Cijk_Ailk_Bljk_MT256x256x64", 2, 4000, 2000, 1900, 2100],
        ["at::native::elementwise", 3, 1000, 333, 300, 400]])
    trace = _write_csv(tmp_path / "t.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], [
        ["void moe::k_dynamic<unsigned short, false>(moe::Params)", 0, 5000],      # warm-up
        ["void moe::k_dynamic<unsigned short, false>(moe::Params)", 0, 1000],
        ["void moe::k_dynamic<unsigned short, false>(moe::Params)", 0, 3000],
        ["void moe::k_dynamic<unsigned short, false>(moe::Params)", 0, 2000]])
    out = tmp_path / "k.md"
    ns = dict(csv=stats, workload="w", kernel="k_dynamic<", command="c", note="", match="moe::,copyBuffer",
              trace=trace, timed=3, out=str(out))
    profiling.kernel_stats(argparse.Namespace(**ns))
    text = open(out).read()
    assert "`moe::k_dynamic<bf16, false>` | 5 | 1.0 | 0.9 | 1.2 | 50.0%" in text
    assert "Cijk_" not in text and "elementwise" not in text
    assert "median 2.0 us, mean 2.0 us, min 1.0 us, max 3.0 us" in text
    ns.update(match="Cijk_", trace="", timed=0)
    profiling.kernel_stats(argparse.Namespace(**ns))
    text = open(out).read()
    assert "Cijk_Ailk_Bljk_MT256x256x64` | 2 | 2.0" in text and "moe::" not in text
