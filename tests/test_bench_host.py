"""Host-side checks of bench.py and of the light/heavy rule mirror; no GPU.

* ``--gpus`` above 1 exits with status 2 before touching a device;
* ``--summarize-mfma`` turns a kernel trace and a counter run into MFMA pipe
  occupancy: busy cycles over (GRBM_GUI_ACTIVE / 8 XCDs) x 256 CUs x 4 SIMDs,
  and the clock over the dispatch's own start-to-end time;
* ``moe.light_experts`` follows the library's default rule;
* the composite layer bound adds the router's and the FFN's binding rooflines.
"""
import csv
import importlib.util
import json
import os
import subprocess
import sys
import types

import numpy as np

from expert_ffn_layer_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_mfma_normalisation(tmp_path):
    bench = load_bench()
    gu = "void moe::(anonymous namespace)::ffn_heavy_kernel<(moe::Mode)0, 0, 1>(moe::FfnArgs)"
    dn = "void moe::(anonymous namespace)::ffn_heavy_kernel<(moe::Mode)1, 1, 1>(moe::FfnArgs)"
    kt, pmc = tmp_path / "kt", tmp_path / "pmc"
    kt.mkdir()
    pmc.mkdir()
    # two gate|up launches of 1000 us, one down launch of 500 us
    _write_csv(kt / "bench_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs"],
               [[gu, 2, 2_000_000], [dn, 1, 500_000]])
    cus, simds, xcds = 256, 4, 8
    rows = []
    # gate|up: 2.0 GHz over 1 ms -> 2e6 cycles per XCD, reported x8; 50% busy
    for d in (1, 2):
        cyc = 2_000_000
        rows.append([d, gu, "GRBM_GUI_ACTIVE", cyc * xcds, 0, 1_000_000])
        rows.append([d, gu, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * cus * simds, 0, 1_000_000])
    # down: 1.5 GHz over 0.5 ms, 25% busy, busy counts split over two rows
    cyc = 750_000
    rows.append([3, dn, "GRBM_GUI_ACTIVE", cyc * xcds, 10, 500_010])
    for _ in range(2):
        rows.append([3, dn, "SQ_VALU_MFMA_BUSY_CYCLES", 0.125 * cyc * cus * simds, 10, 500_010])
    _write_csv(pmc / "bench_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"], rows)
    log = tmp_path / "run.log"
    log.write_text(json.dumps({"value": 1.0, "ms_per_step": 2.0, "roofline": {
        "kernel": "gateup_heavy", "flops": 1.0e12, "kernel_us": 1000.0}}) + "\n")
    bench.PROFILES = str(tmp_path)
    args = types.SimpleNamespace(summarize_mfma=(str(kt), str(pmc), str(log)), config="prefill",
                                 weights="bf16")
    bench.summarize_mfma(args)
    out = [p for p in os.listdir(tmp_path) if p.startswith("mfma_busy__")]
    assert out == ["mfma_busy__prefill_T8192_H4096_E512_k10_I1024.md"]
    text = (tmp_path / out[0]).read_text()
    assert "| gateup_heavy | 2 | 1000.0 | 50.0% | 2000 |" in text
    assert "| down_heavy | 1 | 500.0 | 25.0% | 1500 |" in text
    assert "1000.0 TFLOP/s" in text and "40.0%" in text


def test_light_rule_mirror():
    counts = np.array([0, 1, 8, 9, 16, 64, 65, 200])
    # T <= 64: every expert light (no expert can get more than T rows)
    s = moe.make_shape(64, 256, 8, 2, 64)
    assert np.array_equal(moe.light_experts(counts, s), (counts >= 1) & (counts <= 64))
    # T*k > 8E: the cold tail only (1..8 rows)
    s = moe.make_shape(1000, 256, 8, 2, 64)
    assert np.array_equal(moe.light_experts(counts, s), (counts >= 1) & (counts <= 8))
    # decided from the routing: mean of the touched experts vs 8
    s = moe.make_shape(100, 256, 512, 2, 64)
    low = np.array([0, 3, 5, 8, 12])      # mean 7 -> up to 64 rows light
    high = np.array([0, 3, 5, 8, 40])     # mean 14 -> the cold tail only
    assert np.array_equal(moe.light_experts(low, s), low >= 1)
    assert np.array_equal(moe.light_experts(high, s), (high >= 1) & (high <= 8))
    # a fixed threshold is taken as given
    s = moe.make_shape(100, 256, 512, 2, 64, light_max_rows=16)
    assert np.array_equal(moe.light_experts(counts, s), (counts >= 1) & (counts <= 16))


def test_composite_lower_bound():
    """The composite bound adds the router's and the FFN's binding rooflines:
    decode-shaped numbers worked by hand (HBM 8 TB/s, fp32 157.3 TFLOP/s,
    bf16 2.5 PFLOP/s)."""
    b = load_bench()
    # router: 512 KiB of x + 8 MiB of W_g (1.11 us at 8 TB/s) against
    # 268 MFLOP at 157.3 TFLOP/s (1.71 us): the fp32 FLOPs bind
    rb, rf = 64 * 4096 * 2 + 4096 * 512 * 4, 2 * 64 * 4096 * 512
    t_router = max(rb / 8e12, rf / 157.3e12)
    assert abs(t_router - rf / 157.3e12) < 1e-15  # 1.706 us, the FLOPs bind
    # FFN: 368 touched experts x 24 MiB + out (HBM-bound)
    fb, ff = 368 * 3 * 4096 * 1024 * 2 + 64 * 4096 * 4, 6 * 640 * 4096 * 1024
    t_ffn = fb / 8e12
    assert ff / 2.5e15 < t_ffn
    assert abs(b.composite_lower_bound(rb, rf, fb, ff) - (t_router + t_ffn)) < 1e-12
    # an FFN past the ridge takes its FLOPs term
    assert abs(b.composite_lower_bound(0, 0, 1e6, 1e15) - 1e15 / 2.5e15) < 1e-12
