"""The bench's byte model and the test tolerances, pinned to figures the pages print
(tests/golden/page_figures.json names the page and section of each)."""
import json
import os

import pytest

import bench
from parity import TOL, row_sum_bound

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_one_pass_model_reproduces_logical_bandwidth():
    f = FIG["fused_fp16_1024x1024_warm"]
    gbps = bench.byte_model(f["M"], f["N"], f["elem_bytes"]) / (f["us"] * 1e-6) / 1e9
    assert round(gbps / 10) * 10 == f["printed_GBps"]  # 1639.7 -> "about 1,640"


def test_one_pass_model_reproduces_traffic_and_roof_fraction():
    f = FIG["fused_bf16_8192x4096"]
    bf16 = bench.byte_model(f["M"], f["N"], 2)
    fp32 = bench.byte_model(f["M"], f["N"], 4)
    assert round(bf16 / 1e6) == f["printed_MB_bf16"]
    assert round(fp32 / 1e6) == f["printed_MB_fp32"]
    frac = bf16 / (f["us"] * 1e-6) / 1e9 / f["roof_GBps"]
    lo, hi = f["printed_fraction_range"]
    assert lo <= frac <= hi


def test_wide_model_is_three_passes_over_the_matrix():
    f = FIG["warpline_k2_online_4x32768"]
    ops = f["useful_TOPs"] * 1e12 * f["ms"] * 1e-3
    requested = ops / f["ops_per_requested_byte"]
    wide = bench.byte_model(f["M"], f["N"], f["elem_bytes"], wide=True)
    one_pass = bench.byte_model(f["M"], f["N"], f["elem_bytes"])
    assert abs(requested / wide - 1) < 0.005          # 786,584 vs 786,432
    assert abs(requested / one_pass - 1) > 0.4        # the 2MN model does not fit
    # the memory branch is the ceiling times the same intensity
    assert f["ops_per_requested_byte"] * f["ceiling_GBps"] / 1e3 == pytest.approx(
        f["memory_branch_TOPs"], rel=1e-3)


def test_tolerances_follow_the_pages():
    t = FIG["softmax_tolerance_bf16"]
    assert TOL["bf16"] == (t["atol"], t["rtol"])
    assert TOL["f16"] == (t["atol"], t["rtol"])   # the same tolerance applied to FP16
    r = FIG["row_sum_tolerance_fp32"]
    assert row_sum_bound("f32") == r["tolerance"]
    assert r["failing_row_sum"] - 1 > row_sum_bound("f32")


def test_stats_and_summaries():
    st = bench.stats_us([0.001, 0.002, 0.003, 0.004])
    assert st["median_us"] == 2.5 and st["min_us"] == 1.0 and st["max_us"] == 4.0
    assert st["mean_us"] == 2.5 and st["n"] == 4


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (5, 3), (3, 5), (64, 64), (130, 70), (2048, 2048)])
def test_attention_pair_count(Sq, Sk):
    """The attention FLOP model counts the (query, key) pairs the bottom-right causal
    mask leaves visible: brute force over the mask, and S(S+1)/2 when Sq == Sk."""
    import numpy as np
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    assert bench.attention_pairs(Sq, Sk, True) == int((j <= i + Sk - Sq).sum())
    assert bench.attention_pairs(Sq, Sk, False) == Sq * Sk
    if Sq == Sk:
        assert bench.attention_pairs(Sq, Sk, True) == Sq * (Sq + 1) // 2


def test_gpu_sampler_is_a_diagnostic_only():
    """The clock/power sampler returns None, not an error, when no device can be queried
    (no GPU or no amdsmi here); with readings it summarises the per-XCD clocks and
    ignores unavailable fields."""
    import torch
    s = bench.GpuSampler()
    if not torch.cuda.is_available():
        assert s.start(torch).stop() is None
    fake = bench.GpuSampler()
    fake._thread = type("T", (), {"join": lambda self: None})()
    fake._stop = type("E", (), {"set": lambda self: None})()
    fake.samples = [{"current_gfxclks": [2100, 2000, "N/A"], "current_socket_power": 900,
                     "temperature_hotspot": 60, "temperature_mem": "N/A", "current_uclk": 2000},
                    {"current_gfxclks": [2200, 65535], "current_socket_power": "N/A"}]
    st = fake.stop()
    assert st["samples"] == 2
    assert (st["gfx_clk_mhz_min"], st["gfx_clk_mhz_max"], st["gfx_clk_mhz_mean"]) == (2000, 2200, 2100.0)
    assert st["socket_power_w_max"] == 900 and st["hotspot_c_max"] == 60 and st["mem_temp_c_max"] is None


def test_rotating_timing_interleaves_the_calls(monkeypatch):
    """Round i times every call once, starting from call i mod n, each after a cache
    sweep; warm-up calls carry no events; every call gets exactly `steps` samples."""
    log = []

    class FakeEvents:
        def __init__(self, n):
            self.n, self.used = n, 0

        def next_pair(self):
            self.used += 1
            return ("start", "stop")

        def samples_ms(self, torch):
            return [0.001 * (1 + i) for i in range(self.used)]

        def close(self):
            pass

    monkeypatch.setattr(bench, "DispatchEvents", FakeEvents)

    def make(k):
        def call(events=(None, None)):
            log.append((k, events != (None, None)))
        return call

    flushes = []
    st = bench.time_rotating(None, [make(0), make(1), make(2)], lambda: flushes.append(1), 4, 2)
    warm, timed = log[:6], log[6:]
    assert all(not t for _, t in warm) and all(t for _, t in timed)
    assert [k for k, _ in timed] == [0, 1, 2, 1, 2, 0, 2, 0, 1, 0, 1, 2]
    assert len(flushes) == len(log) == 18
    assert [s["n"] for s in st] == [4, 4, 4]
    assert st[0]["mean_us"] == pytest.approx(2.5)


def _counter_csv(path, dispatches, counter):
    """A rocprofv3 --pmc CSV with the columns the bench reads: (kernel, value) per dispatch."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(dispatches, 1):
            w.writerow([i, k, counter, v])


def test_traffic_table_groups_calls_at_cache_sweeps(tmp_path):
    """The cache-sweep dispatches cut the library's kernels into calls; other kernels are
    ignored; the copy of known size scales each counter; launch counts are checked."""
    sweep, copy = "void smx::k_sweep_read16(uint4 const*, long)", "void smx::k_copy16<false>(x)"
    fwd, wide_a, wide_b = "void smx::k_softmax_rows<2>(a)", "void smx::k_wide_stats(b)", "void smx::k_wide_norm(c)"
    mib = 1024.0  # KiB
    man = {"copy_bytes": 64 << 20, "calls": [
        {"op": "copy", "bytes": 64 << 20, "launches": 1},
        {"workload": "w", "op": "forward", "plan": "auto", "resolved": "resident", "G": 256, "V": 2,
         "cpw": 0, "grid": 4096, "model_bytes": 64 << 20, "launches": 1},
        {"op": "setup", "workload": "w", "launches": None},
        {"workload": "w", "op": "backward", "plan": "wide", "resolved": "wide", "G": 0, "V": 0,
         "cpw": 2, "grid": 2048, "model_bytes": 96 << 20, "launches": 2}]}
    # FETCH_SIZE reads half on the copy, as on the hardware; torch kernels in between
    fetch = [(sweep, 1e6), (copy, 16 * mib), ("void at::native::fill(x)", 5.0), (sweep, 1e6),
             (fwd, 16.5 * mib), (sweep, 1e6), (fwd, 3.0), (sweep, 1e6), (sweep, 1e6),
             (wide_a, 16 * mib), (wide_b, 16 * mib)]
    write = [(sweep, 0), (copy, 32 * mib), (sweep, 0), (fwd, 32 * mib), (sweep, 0), (fwd, 1.0),
             (sweep, 0), (wide_a, 0.0), (wide_b, 32 * mib)]
    for name, rows, ctr in (("f.csv", fetch, "FETCH_SIZE"), ("w.csv", write, "WRITE_SIZE")):
        _counter_csv(tmp_path / name, rows, ctr)
    with open(tmp_path / "m.json", "w") as f:
        json.dump(man, f)
    t = bench.traffic_table(str(tmp_path / "m.json"), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rows = [r for r in t.splitlines() if r.startswith("| w ")]
    assert len(rows) == 2
    fwd_cells = [c.strip() for c in rows[0].strip("|").split("|")]
    bwd_cells = [c.strip() for c in rows[1].strip("|").split("|")]
    assert fwd_cells[1:3] == ["forward", "auto"] and bwd_cells[1:3] == ["backward", "wide"]
    # forward: 33 MiB fetched (x2 scale) + 32 MiB written over 64 MiB algorithmic
    assert float(fwd_cells[8]) == pytest.approx(65 / 64, abs=1e-3)
    # backward: 2 x 32 MiB fetched + 32 MiB written = the 96 MiB model
    assert float(bwd_cells[8]) == pytest.approx(1.0, abs=1e-3)
    assert "FETCH_SIZE x 2.00000" in t
    # a call whose kernel count differs from its plan's launch count is refused
    man["calls"][3]["launches"] = 1
    with open(tmp_path / "m.json", "w") as f:
        json.dump(man, f)
    with pytest.raises(RuntimeError, match="dispatches"):
        bench.traffic_table(str(tmp_path / "m.json"), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))


def test_sweep_table_from_a_log(tmp_path):
    """The per-config table: the automatic plan's time against the same-run copy of the
    same bytes, and the MALL flag from the model bytes."""
    log = tmp_path / "sweep.log"
    rows = [
        {"workload": "normal_bf16_4096x4096", "op": "forward", "copy_ceiling_bytes": 67108864,
         "copy_us": 10.9, "copy_shape": "grid 1024", "copy_GBps": 6156.8},
        {"workload": "normal_bf16_4096x4096", "plan": "auto", "resolved": "persistent", "G": 256,
         "V": 2, "cpw": 0, "grid": 2048, "model_bytes": 67108864, "mean_us": 11.8, "median_us": 11.7,
         "GBps": 5687.2, "pct_peak": 71.09, "frac_of_copy": 0.9237, "mall_resident": True},
        {"workload": "normal_bf16_4096x4096", "op": "backward", "plan": "auto", "mean_us": 17.0},
    ]
    log.write_text("".join("[sweep] " + json.dumps(r) + "\n" for r in rows))
    t = bench.sweep_table(str(log))
    line = [ln for ln in t.splitlines() if ln.startswith("| c2 |")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[2] == "persistent" and cells[3] == "67,108,864" and cells[4] == "11.80"
    assert cells[7] == "10.90" and cells[9] == "0.924" and cells[10] == "yes"


def test_bytes_fit_line_and_table():
    """The least-squares line of the bytes fit recovers an exact line, and the table
    reports the fitted intercept and rate."""
    xs = [16 << 20, 32 << 20, 64 << 20, 1 << 30]
    a, b = bench.linfit(xs, [2.5 + x / 6e6 for x in xs])  # 2.5 us + bytes / 6 TB/s (us)
    assert abs(a - 2.5) < 1e-9 and abs(1e-3 / b - 6000) < 1e-6
    d = {"series": [{"dtype": "bf16", "N": 4096, "fit": {
        "softmax_us": {"intercept_us": 3.1, "GBps": 6800.0}, "copy_us": {"intercept_us": 2.5, "GBps": 6900.0}},
        "points": [{"M": 4096, "plan": "persistent", "model_bytes": 67108864, "softmax_us": 11.8,
                    "copy_us": 10.9, "copy_shape": "grid 1024"}]}]}
    t = bench.fit_table(d)
    assert "3.10 us + bytes / 6800 GB/s" in t and "| 4096 | persistent | 67,108,864 | 11.80 | 10.90 | 1.083 |" in t
