"""Bench: cold BF16 4096 x 4096 row softmax on one MI355X through the C ABI.

One step is one cold call of ``sm_softmax_fwd`` over the seeded 4096 x 4096 BF16
matrix (x ~ N(0, 2^2), seed 2026), after a 1 GiB read-only sweep that evicts the
input from L2 and MALL. The sweep runs outside the timed events.

Protocol (the pages' methodology, restated):
  * a correctness gate before any timing (Warpline README, the correctness
    paragraph): output properties on the GPU first, then, in the CPU-baseline leg,
    the FP64 oracle's result on the same input compared element by element with
    the timed call's output (the run fails if they disagree);
  * a burst of calls to bring the clocks up ("Measured optimization case studies",
    section "GPU clocks: the first calls after an idle pause", which uses 200 ms; 1 s
    here, so that the clock/power sampler also sees the SMU's metrics table refresh
    under load);
  * W untimed cold steps, then K timed cold steps, each bracketed by its own pair
    of HIP events on the launch stream; median, p10, p90, MAD, min, max and mean
    are reported (Warpline README, the suite-protocol paragraph);
  * throughput from the byte model 2 * M * N * elem (one read and one write of
    every element: "Fused Softmax on GPU", section "The Bandwidth Formula"), as a
    fraction of the 8 TB/s HBM3E peak and of a measured 16-byte copy moving the
    same bytes cold;
  * the FP64 oracle timed on this host's cores on the same input (a baseline,
    not the target).

The softmax backward (dx = y * (dy - sum(y * dy)), byte model 3 * M * N * elem, or
5 * M * N * elem on the two-pass wide path) is timed the same way on the same shape,
with y the forward's output and a seeded dy, and reported beside the headline.

The fused attention forward (softmax(scale * Q K^T) V with the online softmax, the
fusion "Fused Softmax on GPU" names in its closing section) is timed on the
attention-shaped workload -- 8 x 32 heads, 2048 queries and keys, d = 128, BF16,
causal -- against the MFMA roofline: FLOPs = 4 * heads * d * visible (query, key)
pairs over the dense BF16 peak of 2.5 PFLOP/s; torch's SDPA on the same tensors is
reported beside it as a reference point.

Prints ONE JSON line on stdout. ``--sweep`` also times every workload and plan,
forward and backward, the residual RMSNorm shapes and the attention shapes, and
writes those lines to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import itertools
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E, decimal GB/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16/FP16 MFMA
# attention-shaped workload: 8 x 32 heads, 2048 x 2048, head dim 128, BF16, causal
ATTN_WORKLOAD = {"heads": 8 * 32, "S": 2048, "d": 128, "dtype": "bf16", "causal": True}
FLUSH_BYTES = 1 << 30
WORKLOAD = "normal_bf16_4096x4096"
# device code of the one-pass row kernels: a traffic record stays valid while these
# are unchanged and the plan still launches the recorded instance
KERNEL_SOURCES = ["memory_bound_row_sm_amd/csrc/sm_device.hpp",
                  "memory_bound_row_sm_amd/csrc/sm_kernels.hpp",
                  "memory_bound_row_sm_amd/csrc/sm_rows_inst.inl"]


def byte_model(M: int, N: int, elem_bytes: int, wide: bool = False) -> int:
    """Algorithmic bytes of one call: every element read once and written once
    (2 M N elem), or read twice and written once on the two-pass wide path."""
    return (3 if wide else 2) * M * N * elem_bytes


def stats_us(samples_ms) -> dict:
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    med = float(np.median(a))
    return {"median_us": med, "mean_us": float(a.mean()), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "mad_us": float(np.median(np.abs(a - med))),
            "min_us": float(a.min()), "max_us": float(a.max()), "n": int(a.size)}


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def row_kernel_name(dt_code: int, info: dict) -> str:
    """The demangled name (without arguments) of the row-kernel instance a plan launches."""
    b = lambda v: "true" if v else "false"
    return (f"smx::k_softmax_rows<{dt_code}, {info['lanes_per_row']}, {info['vecs_per_lane']}, "
            f"{b(info['prefetch'])}, {b(info['nt_loads'])}>")


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources and for the instance the plan launches (else
    None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha() or t.get("kernel") != kernel:
        return None
    return t.get("hbm_bytes_per_launch")


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class DispatchEvents:
    """HIP event pairs that the library attaches to its kernel dispatches
    (hipExtLaunchKernel), so each pair spans exactly the call's kernels on the
    launch stream: no host launch latency, no queue gaps. The events are created
    without the system-scope fence that a default event performs when it is
    recorded (that fence, not the kernel, cost about 3 us per cold call). Created
    through the HIP runtime that torch already loaded (the library binds to the
    same one)."""

    def __init__(self, n: int, flags=HIP_EVENT_DISABLE_SYSTEM_FENCE):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            rc = (self.hip.hipEventCreate(ctypes.byref(e)) if flags is None else
                  self.hip.hipEventCreateWithFlags(ctypes.byref(e), flags))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events.append(e)
        self.used = 0

    def next_pair(self):
        a, b = self.events[2 * self.used], self.events[2 * self.used + 1]
        self.used += 1
        return a, b

    def samples_ms(self, torch):
        torch.cuda.synchronize()
        out = []
        for i in range(self.used):
            ms = ctypes.c_float()
            rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * i],
                                              self.events[2 * i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.append(ms.value)
        return out

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def make_flush(torch, sm, s_handle):
    """A cold-cache call: one read-only sweep of a 1 GiB device buffer on the stream."""
    buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")

    def flush():
        rc = sm.sm_bench_flush(buf.data_ptr(), FLUSH_BYTES, s_handle)
        if rc != 0:
            raise sm.SoftmaxError(rc, "sm_bench_flush")
    return flush


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sweep", action="store_true", help="also time every workload and plan (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm diagnostic lane (profiling runs: every softmax call is cold)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 kernel trace of this bench (cold/warm per kernel) and exit")
    ap.add_argument("--summarize-counters", metavar="COUNTER_CSV",
                    help="per-kernel mean of each rocprofv3 --pmc counter (per dispatch) and exit")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle timing on the host")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-attention", action="store_true", help="skip the attention timing")
    ap.add_argument("--plan-grid", metavar="OUT_JSON",
                    help="time every plan on the row-plan grid (18 row counts x 10 widths, "
                         "BF16 forward), write the cell times to OUT_JSON, print the regret "
                         "summary as one JSON line, and exit")
    ap.add_argument("--grid-runs", type=int, default=2, help="repeat runs of the plan grid")
    ap.add_argument("--grid-steps", type=int, default=10, help="timed cold calls per plan and cell")
    ap.add_argument("--grid-op", default="fwd", choices=["fwd", "bwd", "rms"])
    ap.add_argument("--grid-dtype", default="bf16", choices=["bf16", "f16", "f32"])
    ap.add_argument("--score-grid", metavar="GRID_JSON",
                    help="print the regret summary of a plan-grid file and exit")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from the two rocprofv3 --pmc "
                         "CSVs (FETCH_SIZE run, WRITE_SIZE run) of this bench, and exit")
    ap.add_argument("--counter-pass", metavar="MANIFEST_JSON",
                    help="one cold call of every sweep case, each after a cache sweep (run it "
                         "under rocprofv3 --pmc), write the calls in dispatch order, and exit")
    ap.add_argument("--traffic-table", nargs=3, metavar=("MANIFEST_JSON", "FETCH_CSV", "WRITE_CSV"),
                    help="HBM bytes per call of every sweep case from the counter pass's manifest "
                         "and its FETCH_SIZE and WRITE_SIZE runs (markdown on stdout), and exit")
    ap.add_argument("--sq-csv", help="with --traffic-table: an SQ counter run of the same pass")
    ap.add_argument("--bytes-fit", action="store_true",
                    help="cold time against bytes (16 MiB - 1 GiB) for the softmax and the copy, "
                         "with a least-squares fit t = a + bytes / B of each; prints a table")
    ap.add_argument("--fit-table", metavar="FIT_JSON", help="print a --bytes-fit result as markdown")
    ap.add_argument("--sweep-table", metavar="SWEEP_LOG",
                    help="print the per-config table (time, %% of 8 TB/s, copy ceiling) of a "
                         "--sweep log and exit")
    ap.add_argument("--sweep-log", help="with --traffic-table: a --sweep log, for times and GB/s")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return 0
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic), indent=1))
        return 0
    if args.traffic_table:
        print(traffic_table(*args.traffic_table, sq_csv=args.sq_csv, sweep_log=args.sweep_log))
        return 0
    if args.sweep_table:
        print(sweep_table(args.sweep_table))
        return 0
    if args.fit_table:
        with open(args.fit_table) as f:
            print(fit_table(json.loads(f.read().strip().splitlines()[-1])))
        return 0
    if args.score_grid:
        with open(args.score_grid) as f:
            print(json.dumps(score_grid(json.load(f))))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no communication: each GPU would run the same "
              "kernel on its own block of rows).", file=sys.stderr)
        return 2

    import torch
    import memory_bound_row_sm_amd as sm
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    sm.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    s_handle = stream.cuda_stream

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if args.plan_grid:
        return plan_grid(torch, sm, s_handle, log, args)
    if args.bytes_fit:
        return bytes_fit(torch, sm, s_handle, make_flush(torch, sm, s_handle), log, args)
    if args.counter_pass:
        return counter_pass(torch, sm, workloads, make_flush(torch, sm, s_handle), s_handle,
                            args.counter_pass, 64 << 20, log)

    # ---------------------------------------------------------------- input
    x_cpu = workloads.generate(WORKLOAD)
    sha = workloads.sha256(x_cpu)
    x = x_cpu.to(dev)
    out = torch.full_like(x, float("nan"))
    M, N = x.shape
    es = x.element_size()
    info = sm.plan_for(x, out)
    model_bytes = byte_model(M, N, es, wide=info["plan_name"] == "wide")
    assert model_bytes == info["model_bytes"]
    log(f"[bench] {WORKLOAD}: {M}x{N} bf16, sha256 {sha[:16]}, plan {info['plan_name']} "
        f"G={info['lanes_per_row']} V={info['vecs_per_lane']} grid={info['grid']}")

    dt_code = {torch.float32: sm.SM_F32, torch.float16: sm.SM_F16, torch.bfloat16: sm.SM_BF16}[x.dtype]
    opts = sm.SmOpts()  # all zero: the automatic plan, as sm_softmax_fwd

    def call(events=None):
        opts.start_event, opts.stop_event = events if events else (None, None)
        rc = sm.sm_softmax_fwd_ex(x.data_ptr(), out.data_ptr(), M, N, x.stride(0), out.stride(0),
                                  dt_code, opts, 0, 0, s_handle)
        if rc != 0:
            raise sm.SoftmaxError(rc, "sm_softmax_fwd_ex")

    # ---------------------------------------------------------------- correctness gate
    # Properties every correct output has (finite, in [0, 1], rows summing to 1
    # within the BF16 rounding bound); the element-wise oracle comparison runs in
    # the CPU-baseline leg below, on the same input.
    rc = sm.sm_softmax_fwd(x.data_ptr(), out.data_ptr(), M, N, x.stride(0), out.stride(0),
                           dt_code, s_handle)
    if rc != 0:
        raise sm.SoftmaxError(rc, "sm_softmax_fwd")
    torch.cuda.synchronize()
    sums = out.sum(dim=1, dtype=torch.float64)
    gate_ok = bool(torch.isfinite(out).all()) and bool(((out >= 0) & (out <= 1)).all()) and \
        float((sums - 1).abs().max()) <= 2.0 ** -8 + 1e-5
    if not gate_ok:
        log("[bench] property gate FAILED")
        return 1
    log("[bench] property gate passed")

    flush = make_flush(torch, sm, s_handle)

    # ---------------------------------------------------------------- clocks up
    # 1 s of cache sweeps keep the GPU busy without calling the timed kernel, so a
    # profiler's per-kernel average covers only the calls below, and long enough for the
    # SMU's metrics table (refreshed every few hundred ms) to show the loaded clocks
    sampler = GpuSampler().start(torch)  # through the burst and the cold lane
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        for _ in range(20):
            flush()
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- cold lane
    for _ in range(args.warmup):
        flush()
        call()
    ev = DispatchEvents(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        flush()
        call(ev.next_pair())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state = {"during_softmax_cold_lane": sampler.stop()}
    cold = stats_us(ev.samples_ms(torch))
    ev.close()
    log(f"[bench] timed {args.steps} cold steps in {wall:.3f} s wall (flush sweeps included)")

    # ---------------------------------------------------------------- warm lane (diagnostic)
    warm = None
    if not args.no_warm:
        ev = DispatchEvents(args.steps)
        for _ in range(args.steps):
            call(ev.next_pair())
        warm = stats_us(ev.samples_ms(torch))
        ev.close()

    # ---------------------------------------------------------------- copy ceiling, same bytes, cold
    src = torch.empty(model_bytes // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)

    def copy(grid, scope, events=(None, None)):
        rc = sm.sm_bench_copy(src.data_ptr(), dst.data_ptr(), src.numel(), grid, scope, s_handle,
                              *events)
        if rc != 0:
            raise sm.SoftmaxError(rc, "sm_bench_copy")

    # the ceiling is the best of a few launch shapes under either store policy, timed in
    # rotating order
    shapes = [(grid, scope) for scope in (0, 1)
              for grid in (512, 1024, 2048, 4096, 8192)]  # 8192: one vector per thread at 32 MiB
    sts = time_rotating(torch, [lambda events=(None, None), g=g, s=s: copy(g, s, events)
                                for g, s in shapes], flush, args.steps, args.warmup)
    k = min(range(len(shapes)), key=lambda i: sts[i]["mean_us"])
    copy_cold, (copy_grid, copy_scope) = sts[k], shapes[k]
    del src, dst

    gbps = model_bytes / (cold["mean_us"] * 1e-6) / 1e9
    gbps_median = model_bytes / (cold["median_us"] * 1e-6) / 1e9
    copy_gbps = model_bytes / (copy_cold["mean_us"] * 1e-6) / 1e9
    log(f"[bench] cold mean {cold['mean_us']:.2f} us median {cold['median_us']:.2f} us -> "
        f"{gbps:.0f} GB/s ({100 * gbps / PEAK_GBPS:.1f}% of 8 TB/s); copy ceiling {copy_gbps:.0f} GB/s"
        + (f"; warm median {warm['median_us']:.2f} us" if warm else ""))

    # ---------------------------------------------------------------- backward, same shape, cold
    bwd = None
    if not args.no_backward:
        bwd = bench_backward(torch, sm, workloads, out, flush, s_handle, args.steps, args.warmup, log)

    # ---------------------------------------------------------------- attention forward
    attn = None
    if not args.no_attention:
        sampler = GpuSampler().start(torch)
        attn = bench_attention(torch, sm, s_handle, args.steps, args.warmup, log)
        state["during_attention"] = sampler.stop()

    # ---------------------------------------------------------------- sweep (stderr)
    if args.sweep:
        sweep(torch, sm, workloads, flush, s_handle, log, args)
        sweep_attention(torch, sm, s_handle, log, max(20, args.steps // 10))

    # ---------------------------------------------------------------- CPU baseline
    cpu, parity = None, {"passed": None, "note": "oracle leg skipped (--no-cpu-baseline)"}
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(x_cpu, out, model_bytes, args.cpu_seconds, log)
        if not parity.get("passed"):
            log(f"[bench] oracle parity FAILED: {parity}")

    traffic = load_traffic(WORKLOAD, row_kernel_name(dt_code, info))
    result = {
        "metric": "achieved HBM GB/s (and % of MI355X peak) for cold BF16 softmax, 4096x4096",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold["mean_us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": M, "N": N, "cold": True,
                   "plan": info["plan_name"], "lanes_per_row": info["lanes_per_row"],
                   "vecs_per_lane": info["vecs_per_lane"], "grid": info["grid"],
                   "input_sha256": sha},
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "value_median_GBps": round(gbps_median, 1),
        "cold_us": {k: round(v, 3) if isinstance(v, float) else v for k, v in cold.items()},
        "warm_us": ({k: round(v, 3) if isinstance(v, float) else v for k, v in warm.items()}
                    if warm else None),
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "copy_ceiling_us": round(copy_cold["mean_us"], 3),
        "copy_ceiling_grid": copy_grid,
        "copy_ceiling_stores": "device_scope" if copy_scope else "plain",
        "frac_of_copy_ceiling": round(gbps / copy_gbps, 4),
        "timed_region_wall_s": round(wall, 4),
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_GBPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "backward": bwd,
        "attention": attn,
        "gpu_state": state,
    }
    print(json.dumps(result), flush=True)
    return 0 if parity.get("passed") is not False else 1


def summarize_trace(path: str) -> str:
    """Per kernel: dispatch count and mean/median/min duration of the dispatches that
    follow a cache sweep (cold) and of the others (warm), from a rocprofv3
    kernel-trace CSV. Only this library's kernels are listed."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    groups = {}
    prev = ""
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        lane = "cold" if "sweep" in prev else "warm"
        prev = name
        if "smx::" not in name:  # torch's own set-up kernels
            continue
        key = (name.split("(")[0].replace("void ", ""), r["Grid_Size_X"], r["Workgroup_Size_X"], lane)
        groups.setdefault(key, []).append(dur)
    lines = [f"{'kernel':48s} {'grid(items)':>11s} {'wg':>5s} {'lane':5s} {'calls':>6s} "
             f"{'mean_us':>9s} {'median_us':>9s} {'min_us':>8s}"]
    for (k, g, w, lane), v in sorted(groups.items()):
        lines.append(f"{k[:48]:48s} {g:>11s} {w:>5s} {lane:5s} {len(v):6d} "
                     f"{statistics.mean(v):9.3f} {statistics.median(v):9.3f} {min(v):8.3f}")
    return "\n".join(lines)


def summarize_counters(path: str) -> dict:
    """{kernel: {counter: mean value per dispatch, "dispatches": n}} from a rocprofv3
    --pmc counter-collection CSV (FETCH_SIZE / WRITE_SIZE are KiB per dispatch)."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        k = r["Kernel_Name"].split("(")[0].replace("void ", "")
        d = acc.setdefault(k, {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {}
    for k, d in acc.items():
        out[k] = {c: round(statistics.mean(v), 3) for c, v in d.items()}
        out[k]["dispatches"] = max(len(v) for v in d.values())
    return out


def record_traffic(fetch_csv: str, write_csv: str) -> dict:
    """Build the HBM-traffic record of the headline kernel from the FETCH_SIZE and
    WRITE_SIZE counter runs of this bench. The 16-byte copy kernel in the same runs
    moves a known number of bytes; its counts give the scale of each counter."""
    f, w = summarize_counters(fetch_csv), summarize_counters(write_csv)
    soft = [k for k in f if "k_softmax_rows" in k]
    cp = "smx::k_copy16<false>"  # plain stores: the calibration copy
    if len(soft) != 1 or cp not in f or cp not in w:
        raise RuntimeError(f"expected one softmax row kernel and the copy kernel, found {sorted(f)}")
    k = soft[0]
    M, N, es = 4096, 4096, 2
    copy_bytes = M * N * es  # the copy moves the model's bytes: half read, half written
    ff = (copy_bytes / 1024) / f[cp]["FETCH_SIZE"]
    wf = (copy_bytes / 1024) / w[cp]["WRITE_SIZE"]
    fetch = f[k]["FETCH_SIZE"] * ff * 1024
    write = w[k]["WRITE_SIZE"] * wf * 1024
    alg = byte_model(M, N, es)
    rec = {"workload": WORKLOAD, "kernel": k, "kernel_source_sha": kernel_source_sha(),
           "algorithmic_bytes_per_launch": alg,
           "fetch_size_kib_raw": f[k]["FETCH_SIZE"], "write_size_kib_raw": w[k]["WRITE_SIZE"],
           "dispatches": {"fetch": f[k]["dispatches"], "write": w[k]["dispatches"]},
           "calibration": {"copy_kernel": f"{cp} moving {copy_bytes >> 20} MiB in and "
                                          f"{copy_bytes >> 20} MiB out",
                           "copy_fetch_size_kib_raw": f[cp]["FETCH_SIZE"],
                           "copy_write_size_kib_raw": w[cp]["WRITE_SIZE"],
                           "fetch_factor": round(ff, 5), "write_factor": round(wf, 5)},
           "hbm_fetch_bytes_per_launch": int(round(fetch)),
           "hbm_write_bytes_per_launch": int(round(write)),
           "hbm_bytes_per_launch": int(round(fetch + write)),
           "traffic_over_algorithmic": round((fetch + write) / alg, 5),
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {os.path.dirname(fetch_csv)} -o fetch -- "
               "python3 -u bench.py --steps 20 --warmup 2 --no-warm --no-cpu-baseline --no-backward",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {os.path.dirname(write_csv)} -o write -- "
               "python3 -u bench.py --steps 20 --warmup 2 --no-warm --no-cpu-baseline --no-backward",
               f"python bench.py --record-traffic {fetch_csv} {write_csv}"]}
    path = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def counter_groups(path: str) -> list:
    """The library's dispatches in a rocprofv3 --pmc CSV, in dispatch order, cut into
    groups at each cache-sweep dispatch (empty groups dropped): one group per call of
    the counter pass, each a list of (kernel, {counter: value})."""
    import csv
    rows = {}
    for r in csv.DictReader(open(path)):
        k = r["Kernel_Name"].split("(")[0].replace("void ", "")
        d = rows.setdefault(int(r["Dispatch_Id"]), (k, {}))[1]
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    groups, cur = [], []
    for i in sorted(rows):
        k, c = rows[i]
        if not k.startswith("smx::"):
            continue
        if k.startswith("smx::k_sweep_read16"):
            if cur:
                groups.append(cur)
            cur = []
        else:
            cur.append((k, c))
    if cur:
        groups.append(cur)
    return groups


def traffic_table(manifest_path: str, fetch_csv: str, write_csv: str, sq_csv=None,
                  sweep_log=None) -> str:
    """Markdown table of the HBM bytes of one cold call per sweep case (FETCH_SIZE and
    WRITE_SIZE summed over the call's kernels, each scaled by what it reads for the
    calibration copy of known size), against the plan's algorithmic bytes; with sq_csv,
    VALU busy and LDS bank conflicts; with sweep_log, the sweep's mean time and the
    physical GB/s."""
    with open(manifest_path) as f:
        man = json.load(f)
    calls = man["calls"]
    runs = {"FETCH_SIZE": counter_groups(fetch_csv), "WRITE_SIZE": counter_groups(write_csv)}
    if sq_csv:
        runs["SQ"] = counter_groups(sq_csv)
    for name, g in runs.items():
        if len(g) != len(calls):
            raise RuntimeError(f"{name} run: {len(g)} call groups, manifest has {len(calls)}")
        for c, grp in zip(calls, g):
            if c["launches"] is not None and c["launches"] != len(grp):
                raise RuntimeError(f"{name} run: {c} has {len(grp)} dispatches: "
                                   f"{[k for k, _ in grp]}")

    def total(grp, counter):
        return sum(v.get(counter, 0.0) for _, v in grp)

    cb = man["copy_bytes"]
    if not runs["FETCH_SIZE"][0][0][0].startswith("smx::k_copy16"):
        raise RuntimeError("the first call is not the calibration copy")
    ff = (cb / 2 / 1024) / total(runs["FETCH_SIZE"][0], "FETCH_SIZE")
    wf = (cb / 2 / 1024) / total(runs["WRITE_SIZE"][0], "WRITE_SIZE")
    times = {}
    if sweep_log:
        for line in open(sweep_log):
            if line.startswith("[sweep] "):
                d = json.loads(line[len("[sweep] "):])
                if "plan" in d:  # row kernels only (the attention lines carry no plan)
                    times[(d["workload"], d.get("op", "forward"), d["plan"])] = d.get("mean_us")
    head = ["workload", "op", "plan", "resolved (G, V, cpw, grid)", "kernels", "algorithmic MB",
            "fetched MB", "written MB", "HBM / algorithmic"]
    if times:
        head += ["mean µs", "physical GB/s"]
    if sq_csv:
        head += ["VALU busy", "LDS bank conflicts / LDS instr."]
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for i, c in enumerate(calls):
        if c["op"] in ("copy", "setup"):
            continue
        fetch = total(runs["FETCH_SIZE"][i], "FETCH_SIZE") * ff * 1024
        write = total(runs["WRITE_SIZE"][i], "WRITE_SIZE") * wf * 1024
        cells = [c["workload"], c["op"], c["plan"],
                 f"{c['resolved']} ({c['G']}, {c['V']}, {c['cpw']}, {c['grid']})",
                 str(c["launches"]), f"{c['model_bytes'] / 1e6:.3f}", f"{fetch / 1e6:.3f}",
                 f"{write / 1e6:.3f}", f"{(fetch + write) / c['model_bytes']:.3f}"]
        if times:
            t = times.get((c["workload"], c["op"], c["plan"]))
            cells += [f"{t:.3f}", f"{(fetch + write) / (t * 1e-6) / 1e9:.0f}"] if t else ["", ""]
        if sq_csv:
            g = runs["SQ"][i]
            busy = total(g, "SQ_ACTIVE_INST_VALU") / max(total(g, "SQ_BUSY_CU_CYCLES"), 1.0)
            lds = total(g, "SQ_INSTS_LDS")
            conf = total(g, "SQ_LDS_BANK_CONFLICT") / lds if lds else 0.0
            cells += [f"{100 * busy:.0f}%", f"{conf:.3f}"]
        out.append("| " + " | ".join(cells) + " |")
    out.append("")
    out.append(f"Calibration: the 16-byte copy of {cb >> 20} MiB ({cb >> 21} MiB in, {cb >> 21} MiB out) "
               f"gives FETCH_SIZE x {ff:.5f}, WRITE_SIZE x {wf:.5f}.")
    return "\n".join(out)


def cpu_model() -> str | None:
    """The host CPU's model name (from /proc/cpuinfo), None where unavailable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x_cpu, gpu_out, model_bytes: int, budget_s: float, log):
    """The FP64 oracle, as it stands, on this host's cores: repetitions of the whole
    4096 x 4096 input until the budget is spent (median per repetition), and one
    single-thread run for reference. The oracle's result on this input is also
    compared element by element with the GPU output of the timed call."""
    import oracle
    import workloads
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare, rel_thr_bound
    s = workloads.storage_numpy(x_cpu)
    threads = oracle.max_threads()
    oracle.softmax_f64(s, "bf16", threads=threads)  # warm-up
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t = time.perf_counter()
        oracle.softmax_f64(s, "bf16", threads=threads)
        times.append(time.perf_counter() - t)
    med = statistics.median(times)
    t = time.perf_counter()
    oracle.softmax_f64(s, "bf16", threads=1)
    t1 = time.perf_counter() - t
    res = {"value": round(model_bytes / med / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"the whole 4096x4096 BF16 input, {len(times)} repetitions in "
                     f"{sum(times):.1f} s, median per repetition {med * 1e3:.1f} ms",
           "value_1_thread": round(model_bytes / t1 / 1e9, 3), "cpu_model": cpu_model(),
           "host_cpus_available": len(os.sched_getaffinity(0))}
    log(f"[bench] cpu oracle: {res}")
    try:
        parity = {"passed": True, **compare(gpu_out, x_cpu, what="bench output")}
        # the thresholded relative error (|y| > 1e-3) is gated as well: one rounding
        # plus the one-ulp neighbour, 2^-6 relative in BF16
        parity["max_rel_thr_bound"] = rel_thr_bound("bf16")
        if parity["max_rel_thr"] > parity["max_rel_thr_bound"]:
            parity["passed"] = False
    except AssertionError as e:
        parity = {"passed": False, "error": str(e)[:500]}
    log(f"[bench] oracle parity: {parity}")
    return res, parity


# ------------------------------------------------------------------ row-plan grid
# The grid of "Measured optimization case studies", section "Choosing the plans from
# a grid": every plan timed at 18 row counts and 10 widths from 12288 to 1,048,576,
# and a rule scored by its regret, the rule's time over the best plan's time in the
# same cell, minus 1 (mean, 90th percentile, cells more than 10% off). The page
# names some of its row counts and widths; the others are filled in here.
GRID_ROWS = (1, 2, 4, 8, 16, 24, 32, 48, 64, 80, 96, 128, 192, 256, 384, 512, 768, 1024)
GRID_WIDTHS = (12288, 16384, 32768, 32769, 50257, 65536, 131072, 262144, 524288, 1048576)
GRID_PLANS = {  # forced plans; "auto" is the library's own rule
    "auto": {}, "split": {"plan": 4}, "wide": {"plan": 3}, "resident": {"plan": 1},
    "persistent": {"plan": 2},
    **{f"split_v{v}": {"plan": 4, "vecs_per_lane": v} for v in (1, 2, 4, 8)},
    **{f"wide_c{c}": {"plan": 3, "chunks_per_wave": c} for c in (1, 2, 4, 8)},
}


def _signature(info) -> str:
    d = info.as_dict()
    return (f"{d['plan_name']}:G{d['lanes_per_row']}:V{d['vecs_per_lane']}:c{d['chunks_per_wave']}"
            f":p{d['waves_per_row']}:g{d['grid']}:pf{d['prefetch']}:nt{d['nt_loads']}")


def plan_grid(torch, sm, s_handle, log, args) -> int:
    """Time every plan of every grid cell (cold calls, dispatch events), write the cell
    times, print the regret summary."""
    dev = torch.device("cuda")
    flush = make_flush(torch, sm, s_handle)

    bwd = args.grid_op == "bwd"
    rms = args.grid_op == "rms"
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[args.grid_dtype]
    code = {"bf16": sm.SM_BF16, "f16": sm.SM_F16, "f32": sm.SM_F32}[args.grid_dtype]
    runs = []
    for run in range(args.grid_runs):
        cells = []
        gen = torch.Generator(device="cuda").manual_seed(2026)
        for N in GRID_WIDTHS:
            for M in GRID_ROWS:
                x = (torch.randn(M, N, device=dev, generator=gen) * 3).to(tdt)
                out = torch.empty_like(x)
                dy = w = None
                if bwd:
                    sm.softmax(x, out=x)  # y
                    dy = torch.randn(M, N, device=dev, generator=gen).to(tdt)
                if rms:  # residual and weight
                    dy = torch.randn(M, N, device=dev, generator=gen).to(tdt)
                    w = (1 + 0.5 * torch.randn(N, device=dev, generator=gen)).to(tdt)
                keys, calls = {}, {}
                for key, o in GRID_PLANS.items():
                    opts = sm._opts(o)
                    if bwd:
                        rc, info = sm.sm_softmax_bwd_plan_query(
                            x.data_ptr(), dy.data_ptr(), out.data_ptr(), M, N, N, N, N, code,
                            opts, 0)
                    elif rms:
                        rc, info = sm.sm_rmsnorm_plan_query(
                            x.data_ptr(), dy.data_ptr(), w.data_ptr(), out.data_ptr(), 0, M, N, N, N,
                            N, 0, 1e-6, code, opts, 0)
                    else:
                        rc, info = sm.sm_softmax_plan_query(x.data_ptr(), out.data_ptr(), M, N, N, N,
                                                            code, opts, 0)
                    if rc != 0:
                        continue
                    sig = _signature(info)
                    keys[key] = sig
                    if sig in calls:
                        continue

                    def call(events=(None, None), opts=opts):
                        opts.start_event, opts.stop_event = events
                        if bwd:
                            r = sm.sm_softmax_bwd_ex(x.data_ptr(), dy.data_ptr(), out.data_ptr(), M, N,
                                                     N, N, N, code, opts, 0, 0, s_handle)
                        elif rms:
                            r = sm.sm_rmsnorm_fwd_ex(x.data_ptr(), dy.data_ptr(), w.data_ptr(),
                                                     out.data_ptr(), 0, M, N, N, N, N, 0, 1e-6,
                                                     code, opts, 0, 0, s_handle)
                        else:
                            r = sm.sm_softmax_fwd_ex(x.data_ptr(), out.data_ptr(), M, N, N, N,
                                                     code, opts, 0, 0, s_handle)
                        if r != 0:
                            raise sm.SoftmaxError(r)

                    calls[sig] = call
                # the distinct plans of a cell in rotating order, sample by sample
                st = time_rotating(torch, list(calls.values()), flush, args.grid_steps, 2)
                times = {sig: round(s["mean_us"], 3) for sig, s in zip(calls, st)}
                cells.append({"M": M, "N": N, "keys": keys, "us": times})
                del x, out, dy, w
            torch.cuda.empty_cache()
            log(f"[grid] run {run + 1}: width {N} done ({len(cells)} cells)")
        runs.append(cells)
    if sm.sync_failures() != 0:
        raise RuntimeError("SPLIT waits timed out during the grid")
    data = {"op": args.grid_op, "dtype": args.grid_dtype, "rows": GRID_ROWS, "widths": GRID_WIDTHS,
            "steps": args.grid_steps, "runs": runs}
    with open(args.plan_grid, "w") as f:
        json.dump(data, f, separators=(",", ":"))
    print(json.dumps(score_grid(data)), flush=True)
    return 0


def score_grid(data: dict) -> dict:
    """Regret of the library's rule and of simple alternatives on a plan grid:
    per cell, (time of the rule's plan) / (best forced plan's time) - 1."""
    def rules(c):
        k = c["keys"]
        r = {"library": k.get("auto"), "always_split": k.get("split") or k.get("wide"),
             "always_wide": k.get("wide")}
        r["one_pass_when_it_fits"] = k.get("resident") or k.get("auto")
        return r

    out = {"op": data["op"], "cells": None, "rules": {}}
    per_run = []
    for cells in data["runs"]:
        regrets = {}
        for c in cells:
            best = min(c["us"][sig] for key, sig in c["keys"].items() if key != "auto")
            for name, sig in rules(c).items():
                if sig is None or sig not in c["us"]:
                    continue
                regrets.setdefault(name, []).append(c["us"][sig] / best - 1.0)
        per_run.append(regrets)
        out["cells"] = len(cells)
    for name in per_run[0]:
        rs = [np.asarray(r[name]) for r in per_run]
        out["rules"][name] = {
            "mean_regret_pct": [round(100 * float(a.mean()), 2) for a in rs],
            "p90_regret_pct": round(100 * float(np.percentile(rs[0], 90)), 2),
            "cells_over_10pct": int((rs[0] > 0.10).sum()), "cells": int(rs[0].size)}
    if len(data["runs"]) > 1:  # run-to-run noise of the same plan in the same cell
        d = []
        for c1, c2 in zip(data["runs"][0], data["runs"][1]):
            for sig, t in c1["us"].items():
                if sig in c2["us"]:
                    d.append(abs(c2["us"][sig] / t - 1.0))
        out["repeat_diff_pct"] = {"median": round(100 * float(np.median(d)), 2),
                                  "p90": round(100 * float(np.percentile(d, 90)), 2)}
    return out


def time_rotating(torch, calls, flush, steps, warmup):
    """Cold timing of several calls of one workload, interleaved: round i times every
    call once, after a cache sweep each, starting from call i mod len(calls), so slow
    drifts of clock and temperature spread over all calls alike instead of landing on
    whichever call happened to run last. ``warmup`` untimed rounds come first. Returns
    one stats_us() dict per call, in the order given."""
    n = len(calls)
    for i in range(warmup):
        for j in range(n):
            flush()
            calls[(i + j) % n]()
    evs = [DispatchEvents(steps) for _ in calls]
    for i in range(steps):
        for j in range(n):
            k = (i + j) % n
            flush()
            calls[k](evs[k].next_pair())
    out = []
    for e in evs:
        out.append(stats_us(e.samples_ms(torch)))
        e.close()
    return out


SWEEP_PLANS = {"auto": 0, "resident": 1, "persistent": 2, "wide": 3, "split": 4}

# residual RMSNorm shapes: the FP16 shapes of "Measured optimization case studies"
# (residual RMSNorm section) and the BF16 batch x hidden shapes of the Warpline README
RMS_SHAPES = [("f16", 32, 127), ("f16", 1024, 1024), ("f16", 512, 4097), ("f16", 16384, 4096),
              ("f16", 4, 32769), ("f16", 64, 131072), ("bf16", 1, 1024), ("bf16", 8, 1024),
              ("bf16", 16, 2048), ("bf16", 32, 4096), ("bf16", 64, 4096), ("bf16", 64, 8192)]


def plan_fields(info: dict, op: str) -> dict:
    """The plan columns of a sweep line."""
    return {"resolved": info["plan_name"], "G": info["lanes_per_row"], "V": info["vecs_per_lane"],
            "cpw": info["waves_per_row"] if op == "rmsnorm" else info["chunks_per_wave"],
            "grid": info["grid"], "model_bytes": info["model_bytes"]}


def rmsnorm_groups(torch, sm, s_handle):
    """The residual RMSNorm cases (y only), one shape at a time: yields (workload, op,
    setup, runs) as softmax_groups does."""
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    code = {"f16": sm.SM_F16, "bf16": sm.SM_BF16}
    gen = torch.Generator(device="cuda").manual_seed(2026)
    for dt, M, N in RMS_SHAPES:
        x = (torch.randn(M, N, device="cuda", generator=gen) * 2).to(tdt[dt])
        r = torch.randn(M, N, device="cuda", generator=gen).to(tdt[dt])
        w = (1 + 0.5 * torch.randn(N, device="cuda", generator=gen)).to(tdt[dt])
        y = torch.empty_like(x)
        runs = []
        for pname, p in SWEEP_PLANS.items():
            o = sm.SmOpts()
            o.plan = p
            rc, info = sm.sm_rmsnorm_plan_query(x.data_ptr(), r.data_ptr(), w.data_ptr(), y.data_ptr(),
                                                0, M, N, N, N, N, 0, 1e-6, code[dt], o, 0)
            if rc != 0:
                continue

            def call(events=(None, None), o=o):
                o.start_event, o.stop_event = events
                rc = sm.sm_rmsnorm_fwd_ex(x.data_ptr(), r.data_ptr(), w.data_ptr(), y.data_ptr(), 0, M,
                                          N, N, N, N, 0, 1e-6, code[dt], o, 0, 0, s_handle)
                if rc != 0:
                    raise sm.SoftmaxError(rc)
            runs.append((pname, info.as_dict(), call, None))
        yield f"rmsnorm_{dt}_{M}x{N}", "rmsnorm", None, runs
        del runs, x, r, w, y
    torch.cuda.empty_cache()


def softmax_groups(torch, sm, workloads, s_handle, clocks_up=None):
    """The softmax cases of the sweep, one workload at a time: yields (workload, op,
    setup, runs) for op "forward", then "backward", with runs = [(plan name, plan info,
    call, check)]: call(events) runs one call under that plan, check() (or None) returns
    fields that describe its output, and setup() (or None) must run before the group's
    calls (the backward's y is the forward's output). A workload's tensors live until
    the generator moves on; clocks_up() runs after each input reaches the device."""
    names = ["normal_f32_128x781", "normal_bf16_4096x4096",
             *[f"spiky_f16_8192x{n}" for n in workloads.SPIKE_WIDTHS],
             "offset_bf16_64x131072", "causal_bf16_524288x2048"]
    for name in names:
        x = workloads.generate(name).to("cuda")
        if clocks_up is not None:
            clocks_up()
        out = torch.empty_like(x)
        M, N = x.shape
        dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[x.dtype]
        plans = {k: p for k, p in SWEEP_PLANS.items() if not (p in (1, 2) and N > 8192)}
        runs = []
        for pname, p in plans.items():
            o = sm.SmOpts()
            o.plan = p

            def call(events=(None, None), o=o):
                o.start_event, o.stop_event = events
                rc = sm.sm_softmax_fwd_ex(x.data_ptr(), out.data_ptr(), M, N, N, N, dt, o, 0, 0,
                                          s_handle)
                if rc != 0:
                    raise sm.SoftmaxError(rc)
            runs.append((pname, sm.plan_for(x, out, {"plan": p}), call, None))
        yield name, "forward", None, runs
        dy = workloads.upstream_grad(x.shape, workloads.dtype_name(x), device="cuda")
        runs = []
        for pname, p in plans.items():
            info, call, dx = backward_call(torch, sm, out, dy, p, s_handle)
            # property of every correct dx: each row sums to about 0
            runs.append((pname, info, call, lambda dx=dx: {
                "max_abs_row_sum": round(dx.float().sum(dim=1).abs().max().item(), 6)}))
        yield name, "backward", lambda: sm.softmax(x, out), runs
        del runs, x, out, dy
        torch.cuda.empty_cache()


# MI355X's last-level cache (MALL / Infinity Cache): a workload of at most this many
# bytes can be served partly from it even after the 1 GiB sweep, on its write-backs
MALL_BYTES = 256 << 20
# copy-ceiling launch shapes: (workgroups, store policy) -- device-scope (sc1) stores are
# the row kernels' own policy; workgroups 0: one 16-byte vector per thread (a grid that
# covers the copy once, like the resident row plans)
COPY_SHAPES = [(1024, 1), (4096, 1), (16384, 1), (0, 1), (1024, 0), (4096, 0), (16384, 0), (0, 0)]


def copy_calls(torch, sm, s_handle, model_bytes: int):
    """[(shape, call)] for a 16-byte copy of model_bytes / 2 bytes (read) into as many
    (written), under each of COPY_SHAPES."""
    n = max(16, (model_bytes // 2) // 16 * 16)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out = []
    for grid, scope in COPY_SHAPES:
        grid = grid or -(-(n // 16) // 256)
        def call(events=(None, None), grid=grid, scope=scope):
            rc = sm.sm_bench_copy(src.data_ptr(), dst.data_ptr(), n, grid, scope, s_handle, *events)
            if rc != 0:
                raise sm.SoftmaxError(rc, "sm_bench_copy")
        out.append((f"grid {grid}, {'device-scope' if scope else 'plain'} stores", call))
    return out


def sweep(torch, sm, workloads, flush, s_handle, log, args):
    """Cold timing of every workload under every plan that can take it (residual
    RMSNorm, then softmax forward and backward), the plans of a workload in rotating
    order."""
    steps = max(100, args.steps // 2)  # at least 100 timed samples per (workload, plan)

    def clocks_up():  # the GPU idled while the input was built on the host
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(20):
                flush()
            torch.cuda.synchronize()

    groups = itertools.chain(rmsnorm_groups(torch, sm, s_handle),
                             softmax_groups(torch, sm, workloads, s_handle, clocks_up))
    for name, op, setup, runs in groups:
        if setup is not None:
            setup()
        # the copy ceiling of this workload: a cold 16-byte copy moving the automatic
        # plan's model bytes (half read, half written), timed in the same rotation
        model = runs[0][1]["model_bytes"]
        copies = copy_calls(torch, sm, s_handle, model)
        stats = time_rotating(torch, [r[2] for r in runs] + [c[1] for c in copies], flush, steps, 10)
        cst = stats[len(runs):]
        k = min(range(len(copies)), key=lambda i: cst[i]["mean_us"])
        copy_us, copy_shape = cst[k]["mean_us"], copies[k][0]
        log("[sweep] " + json.dumps({"workload": name, "op": op, "copy_ceiling_bytes": model,
                                     "copy_us": round(copy_us, 3), "copy_shape": copy_shape,
                                     "copy_GBps": round(model / (copy_us * 1e-6) / 1e9, 1)}))
        for (pname, info, _, check), st in zip(runs, stats):
            gb = info["model_bytes"] / (st["mean_us"] * 1e-6) / 1e9
            line = {"workload": name, "plan": pname, **plan_fields(info, op),
                    "mean_us": round(st["mean_us"], 3), "median_us": round(st["median_us"], 3),
                    "GBps": round(gb, 1), "pct_peak": round(100 * gb / PEAK_GBPS, 2),
                    # the copy moves the automatic plan's model bytes: a plan with more
                    # model bytes (WIDE) is compared on the time the copy took
                    "frac_of_copy": round(copy_us / st["mean_us"], 4),
                    "mall_resident": model <= MALL_BYTES}
            if op != "forward":
                line = {"workload": name, "op": op, **{k: v for k, v in line.items() if k != "workload"}}
            if check is not None:
                line.update(check())
            log("[sweep] " + json.dumps(line))
        del copies


# series of the bytes fit: (dtype, row width, row counts) -- BF16 rows of 4096 (the
# headline's rows) and FP16 rows of 2048, 16 MiB to 1 GiB of model bytes
FIT_SERIES = [("bf16", 4096, (1024, 2048, 4096, 8192, 16384, 32768, 65536)),
              ("f16", 2048, (2048, 4096, 8192, 16384, 32768, 65536, 131072))]


def linfit(xs, ys):
    """Least-squares line y = a + b x: (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx
    return my - b * mx, b


def bytes_fit(torch, sm, s_handle, flush, log, args) -> int:
    """Cold time of the automatic softmax plan and of the best copy shape moving the same
    bytes, at sizes from 16 MiB to 1 GiB, each series fitted as t = a + bytes / B: the
    intercept a is the fixed cost of a call (launch, ramp, tail), B its streaming rate.
    The headline's gap to the copy splits into the difference of intercepts and of
    slopes."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}
    code = {"bf16": sm.SM_BF16, "f16": sm.SM_F16}
    steps = max(50, args.steps // 2)
    out = {"series": []}
    for dt, N, rows in FIT_SERIES:
        pts = []
        for M in rows:
            x = torch.randn(M, N, device="cuda").to(tdt[dt])
            y = torch.empty_like(x)
            o = sm.SmOpts()

            def call(events=(None, None), x=x, y=y, M=M, o=o):
                o.start_event, o.stop_event = events
                rc = sm.sm_softmax_fwd_ex(x.data_ptr(), y.data_ptr(), M, N, N, N, code[dt], o, 0, 0,
                                          s_handle)
                if rc != 0:
                    raise sm.SoftmaxError(rc)
            info = sm.plan_for(x, y)
            model = info["model_bytes"]
            copies = copy_calls(torch, sm, s_handle, model)
            st = time_rotating(torch, [call] + [c[1] for c in copies], flush, steps, 5)
            k = 1 + min(range(len(copies)), key=lambda i: st[1 + i]["mean_us"])
            pt = {"M": M, "N": N, "dtype": dt, "plan": info["plan_name"], "model_bytes": model,
                  "softmax_us": round(st[0]["mean_us"], 3), "copy_us": round(st[k]["mean_us"], 3),
                  "copy_shape": copies[k - 1][0]}
            log("[fit] " + json.dumps(pt))
            pts.append(pt)
            del x, y, copies
            torch.cuda.empty_cache()
        xs = [p["model_bytes"] for p in pts]
        fits = {}
        for key in ("softmax_us", "copy_us"):
            a, b = linfit(xs, [p[key] for p in pts])
            fits[key] = {"intercept_us": round(a, 3), "GBps": round(1e-3 / b, 1)}
        out["series"].append({"dtype": dt, "N": N, "points": pts, "fit": fits})
    print(json.dumps(out), flush=True)
    return 0


def fit_table(d: dict) -> str:
    """Markdown of a --bytes-fit result."""
    lines = []
    for ser in d["series"]:
        f = ser["fit"]
        lines += [f"{ser['dtype'].upper()} rows of {ser['N']}: softmax t = "
                  f"{f['softmax_us']['intercept_us']:.2f} us + bytes / {f['softmax_us']['GBps']:.0f} GB/s; "
                  f"copy t = {f['copy_us']['intercept_us']:.2f} us + bytes / {f['copy_us']['GBps']:.0f} GB/s",
                  "", "| M | plan | model bytes | softmax µs | copy µs | softmax / copy time | copy shape |",
                  "|---:|---|---:|---:|---:|---:|---|"]
        for p in ser["points"]:
            lines.append(f"| {p['M']} | {p['plan']} | {p['model_bytes']:,} | {p['softmax_us']:.2f} | "
                         f"{p['copy_us']:.2f} | {p['softmax_us'] / p['copy_us']:.3f} | {p['copy_shape']} |")
        lines.append("")
    return "\n".join(lines)


# the configurations of the forward softmax hot path, in the order they are tabled
CONFIG_ROWS = [("c1", "normal_f32_128x781"), ("c2", "normal_bf16_4096x4096"),
               *[(f"c3 N={n}", f"spiky_f16_8192x{n}") for n in (127, 256, 1000, 2048, 4096, 8192)],
               ("c4", "offset_bf16_64x131072"), ("c5", "causal_bf16_524288x2048")]


def sweep_table(path: str) -> str:
    """Markdown tables of a --sweep log: per config, the automatic forward plan's cold
    time, GB/s on the byte model, % of 8 TB/s, and the same-run cold copy of the same
    bytes (its time and the plan's fraction of it); then every plan of every config."""
    lines = []
    with open(path) as f:
        for ln in f:
            if "[sweep] " in ln:
                lines.append(json.loads(ln.split("[sweep] ", 1)[1]))
    copies = {(d["workload"], d["op"]): d for d in lines if "copy_us" in d}
    fwd = {(d["workload"], d["plan"]): d for d in lines if "plan" in d and "op" not in d}
    out = ["| config | workload | plan | model bytes | µs | GB/s | % of 8 TB/s | copy µs | "
           "copy GB/s | fraction of copy | ≤ 256 MiB (MALL) |",
           "|---|---|---|---:|---:|---:|---:|---:|---:|---:|---|"]
    for cfg, name in CONFIG_ROWS:
        d, c = fwd.get((name, "auto")), copies.get((name, "forward"))
        if d is None or c is None:
            continue
        out.append(f"| {cfg} | {name} | {d['resolved']} | {d['model_bytes']:,} | {d['mean_us']:.2f} | "
                   f"{d['GBps']:.0f} | {d['pct_peak']:.1f} | {c['copy_us']:.2f} | "
                   f"{c['copy_GBps']:.0f} | {d['frac_of_copy']:.3f} | "
                   f"{'yes' if d['mall_resident'] else 'no'} |")
    out += ["", "Every plan (forward):", "",
            "| workload | plan | resolved | µs | GB/s | % of 8 TB/s | fraction of copy |",
            "|---|---|---|---:|---:|---:|---:|"]
    for cfg, name in CONFIG_ROWS:
        for (w, pl), d in fwd.items():
            if w == name:
                out.append(f"| {name} | {pl} | {d['resolved']} | {d['mean_us']:.2f} | {d['GBps']:.0f} | "
                           f"{d['pct_peak']:.1f} | {d['frac_of_copy']:.3f} |")
    return "\n".join(out)


def counter_pass(torch, sm, workloads, flush, s_handle, manifest_path, copy_bytes, log) -> int:
    """One cold call of every sweep case (residual RMSNorm, softmax forward and
    backward, every plan), each right after a cache sweep, for rocprofv3 --pmc runs of
    their own; first a 16-byte copy of copy_bytes, the calibration of the byte counters.
    Writes the calls in dispatch order to manifest_path: the cache-sweep kernel's
    dispatches cut the counter rows of the library's kernels into these calls."""
    src = torch.ones(copy_bytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    flush()
    rc = sm.sm_bench_copy(src.data_ptr(), dst.data_ptr(), src.numel(), 0, 0, s_handle, None, None)
    if rc != 0:
        raise sm.SoftmaxError(rc, "sm_bench_copy")
    del src, dst
    calls = [{"op": "copy", "bytes": copy_bytes, "launches": 1}]
    failures = sm.sync_failures()
    groups = itertools.chain(rmsnorm_groups(torch, sm, s_handle),
                             softmax_groups(torch, sm, workloads, s_handle))
    for name, op, setup, runs in groups:
        if setup is not None:
            flush()
            setup()
            calls.append({"op": "setup", "workload": name, "launches": None})
        for pname, info, call, _ in runs:
            flush()
            call()
            calls.append({"workload": name, "op": op, "plan": pname, **plan_fields(info, op),
                          "launches": info["launches"]})
    torch.cuda.synchronize()
    if sm.sync_failures() != failures:
        raise RuntimeError("SPLIT waits timed out during the counter pass")
    with open(manifest_path, "w") as f:
        json.dump({"copy_bytes": copy_bytes, "calls": calls}, f, indent=0)
    log(f"[counters] {len(calls)} calls written to {manifest_path}")
    return 0


def backward_call(torch, sm, y, dy, plan, s_handle):
    """(plan info, call, dx) for sm_softmax_bwd_ex under ``plan``, dx in a buffer of its
    own; call(events) runs one backward with the dispatch events given."""
    dx = torch.empty_like(y)
    M, N = y.shape
    o = sm.SmOpts()
    o.plan = plan
    info = sm.plan_for_backward(y, dy, dx, {"plan": plan})
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[y.dtype]

    def call(events=(None, None)):
        o.start_event, o.stop_event = events
        rc = sm.sm_softmax_bwd_ex(y.data_ptr(), dy.data_ptr(), dx.data_ptr(), M, N, y.stride(0),
                                  dy.stride(0), dx.stride(0), dt, o, 0, 0, s_handle)
        if rc != 0:
            raise sm.SoftmaxError(rc, "sm_softmax_bwd_ex")
    return info, call, dx


def time_backward(torch, sm, y, dy, plan, flush, s_handle, steps, warmup):
    """Cold timing of sm_softmax_bwd_ex (dx in a buffer of its own) under ``plan``."""
    info, call, dx = backward_call(torch, sm, y, dy, plan, s_handle)
    st, = time_rotating(torch, [call], flush, steps, warmup)
    # property of every correct dx: each row sums to d * (1 - sum(y)), about 0
    rs = dx.float().sum(dim=1).abs().max().item()
    info["max_abs_row_sum"] = rs
    return st, info


def bench_backward(torch, sm, workloads, y, flush, s_handle, steps, warmup, log):
    dy = workloads.upstream_grad(y.shape, workloads.dtype_name(y), device="cuda")
    st, info = time_backward(torch, sm, y, dy, 0, flush, s_handle, steps, warmup)
    gb = info["model_bytes"] / (st["mean_us"] * 1e-6) / 1e9
    res = {"op": "softmax backward dx = y*(dy - sum(y*dy))", "plan": info["plan_name"],
           "lanes_per_row": info["lanes_per_row"], "vecs_per_lane": info["vecs_per_lane"],
           "grid": info["grid"], "model_bytes": info["model_bytes"],
           "cold_mean_us": round(st["mean_us"], 3), "cold_median_us": round(st["median_us"], 3),
           "GBps": round(gb, 1), "pct_of_peak": round(100 * gb / PEAK_GBPS, 2),
           "max_abs_row_sum": info["max_abs_row_sum"]}
    log(f"[bench] backward: {res}")
    if not info["max_abs_row_sum"] < 0.05:
        raise RuntimeError(f"backward rows do not sum to about 0: {info['max_abs_row_sum']}")
    return res


class GpuSampler:
    """Clock, power and temperature of the GPU while a lane runs: a thread of this
    process polls amdsmi's GPU metrics in-process (no child process) every `period`
    seconds between start() and stop(). stop() returns the mean and range of the
    XCDs' graphics clocks, the memory clock, socket power and the hottest readings, or
    None where amdsmi is missing or fails: the readings are a diagnostic and never
    fail the bench."""
    _handle = None

    def __init__(self, period: float = 0.025):
        self.period = period
        self.samples = []
        self._thread = None
        self._stop = None

    @classmethod
    def _device(cls, torch):
        if cls._handle is None:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            h = hs[0]
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for cand in hs:  # the handle of torch's device 0, by PCI bus, where known
                try:
                    if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(cand).split(":")[1], 16) == bus:
                        h = cand
                except Exception:
                    pass
            cls._handle = h
        return cls._handle

    def start(self, torch):
        import threading
        try:
            import amdsmi
            h = self._device(torch)
        except Exception:
            return self
        self._stop = threading.Event()

        def poll():
            while not self._stop.is_set():
                try:
                    self.samples.append(amdsmi.amdsmi_get_gpu_metrics_info(h))
                except Exception:
                    pass
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=poll, daemon=True)
        self._thread.start()
        return self

    def stop(self) -> dict | None:
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        # unavailable fields read "N/A" or an all-ones 16-bit value (65535): keep numbers
        # in a plausible range only (MHz, W, degrees C)
        def vals(key, hi, many=False):
            out = []
            for m in self.samples:
                xs = (m.get(key) or []) if many else [m.get(key)]
                out += [x for x in xs if isinstance(x, (int, float)) and 0 < x < hi]
            return out

        clocks = vals("current_gfxclks", 10000, many=True)
        power = vals("current_socket_power", 10000)
        hot = vals("temperature_hotspot", 200)
        memt = vals("temperature_mem", 200)
        uclk = vals("current_uclk", 10000)
        if not self.samples:
            return None
        distinct = len({tuple(m.get("current_gfxclks") or []) for m in self.samples})
        return {"samples": len(self.samples), "distinct_readings": distinct,
                "gfx_clk_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None,
                "gfx_clk_mhz_min": min(clocks) if clocks else None,
                "gfx_clk_mhz_max": max(clocks) if clocks else None,
                "mem_clk_mhz": max(uclk) if uclk else None,
                "socket_power_w_mean": round(sum(power) / len(power), 1) if power else None,
                "socket_power_w_max": max(power) if power else None,
                "hotspot_c_max": max(hot) if hot else None,
                "mem_temp_c_max": max(memt) if memt else None}


def attention_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """Visible (query, key) pairs of one head; the causal mask is aligned to the bottom
    right (query i sees keys j <= i + Sk - Sq)."""
    if not causal:
        return Sq * Sk
    off = Sk - Sq
    return sum(max(0, min(Sk, i + off + 1)) for i in range(Sq))


def time_attention(torch, sm, q, k, v, o, causal, s_handle, steps, warmup):
    """sm_attention_fwd_ex on [BH][S][d] tensors, each call bracketed by its own events."""
    BH, Sq, d = q.shape
    Sk = k.shape[1]
    dt = {torch.float16: sm.SM_F16, torch.bfloat16: sm.SM_BF16}[q.dtype]
    st_ = (q.stride(1), q.stride(0), k.stride(1), k.stride(0), v.stride(1), v.stride(0),
           o.stride(1), o.stride(0))
    opts = sm.SmOpts()

    def call(events=(None, None)):
        opts.start_event, opts.stop_event = events
        rc = sm.sm_attention_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, BH, Sq,
                                    Sk, d, st_, 1.0 / float(d) ** 0.5, int(causal), dt, opts, s_handle)
        if rc != 0:
            raise sm.SoftmaxError(rc, "sm_attention_fwd_ex")

    for _ in range(warmup):
        call()
    t = DispatchEvents(steps)
    for _ in range(steps):
        call(t.next_pair())
    st = stats_us(t.samples_ms(torch))
    t.close()
    return st


def time_torch_sdpa(torch, q, k, v, causal, steps):
    """torch's scaled_dot_product_attention on the same tensors (a reference point; it
    aligns the causal mask top-left, the same as bottom-right when Sq == Sk)."""
    F = torch.nn.functional
    qq, kk, vv = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
    for _ in range(3):
        F.scaled_dot_product_attention(qq, kk, vv, is_causal=causal)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        F.scaled_dot_product_attention(qq, kk, vv, is_causal=causal)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def attention_inputs(torch, BH, S, d, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return [torch.randn(BH, S, d, device="cuda", generator=g).to(tdt) for _ in range(3)]


def bench_attention(torch, sm, s_handle, steps, warmup, log):
    w = ATTN_WORKLOAD
    BH, S, d, causal = w["heads"], w["S"], w["d"], w["causal"]
    q, k, v = attention_inputs(torch, BH, S, d, w["dtype"], 2026)
    o = torch.full_like(q, float("nan"))
    st = time_attention(torch, sm, q, k, v, o, causal, s_handle, min(steps, 50), min(warmup, 5))
    torch.cuda.synchronize()
    # exact properties of a correct output: finite, and the first query of every head
    # sees only key 0, so its output row is v_0 itself
    if not bool(torch.isfinite(o).all()) or not torch.equal(o[:, 0].view(torch.int16),
                                                            v[:, 0].view(torch.int16)):
        raise RuntimeError("attention property gate failed")
    flops = 4 * BH * d * attention_pairs(S, S, causal)
    tflops = flops / (st["mean_us"] * 1e-6) / 1e12
    ref_us = time_torch_sdpa(torch, q, k, v, causal, 10)
    res = {"op": "fused attention forward (online softmax)", "workload": "attention_bf16_256x2048x2048_d128",
           "heads": BH, "Sq": S, "Sk": S, "d": d, "causal": causal, "dtype": w["dtype"],
           "flops": flops, "mean_us": round(st["mean_us"], 2), "median_us": round(st["median_us"], 2),
           "TFLOPs": round(tflops, 1),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
           "torch_sdpa_us": round(ref_us, 2), "speedup_vs_torch_sdpa": round(ref_us / st["mean_us"], 3)}
    log(f"[bench] attention: {res}")
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


ATTN_SHAPES = [("bf16", 256, 2048, 128, True), ("bf16", 256, 2048, 128, False),
               ("f16", 256, 2048, 128, True), ("bf16", 256, 2048, 64, True),
               ("bf16", 256, 2048, 64, False), ("bf16", 64, 4096, 128, True),
               ("bf16", 32, 8192, 128, True), ("bf16", 1024, 512, 128, True)]


def sweep_attention(torch, sm, s_handle, log, steps):
    """Attention forward at the sweep's shapes, against the MFMA roofline and torch's SDPA."""
    for dt, BH, S, d, causal in ATTN_SHAPES:
        q, k, v = attention_inputs(torch, BH, S, d, dt, 7)
        o = torch.empty_like(q)
        st = time_attention(torch, sm, q, k, v, o, causal, s_handle, steps, 3)
        tflops = 4 * BH * d * attention_pairs(S, S, causal) / (st["mean_us"] * 1e-6) / 1e12
        ref_us = time_torch_sdpa(torch, q, k, v, causal, 5)
        line = {"workload": f"attention_{dt}_{BH}x{S}x{S}_d{d}", "op": "attention",
                "causal": causal, "mean_us": round(st["mean_us"], 2),
                "median_us": round(st["median_us"], 2), "TFLOPs": round(tflops, 1),
                "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                "torch_sdpa_us": round(ref_us, 2)}
        log("[sweep] " + json.dumps(line))
        del q, k, v, o
    torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
