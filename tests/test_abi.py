"""The C ABI on the host: exported symbols, argument validation (which runs before
any HIP call, so it is testable without a GPU), and the plan rule evaluated for a
256-CU device without touching one."""
import os
import re
import subprocess

import pytest

import memory_bound_row_sm_amd as sm
from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

F32, F16, BF16 = sm.SM_F32, sm.SM_F16, sm.SM_BF16
OK, INVALID, DTYPE, OVERLAP, NO_DEVICE, PLAN = 0, -1, -2, -3, -5, -7
BASE = 1 << 32  # a fake, 256-byte aligned device address: never dereferenced on these paths


def declared_functions():
    names = []
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sm_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(sm.EXPORTED_SYMBOLS), names
    out = subprocess.run(["nm", "-D", "--defined-only", sm.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing
    lib = sm.lib()
    for n in names:
        assert hasattr(lib, n)


def test_version_and_strerror():
    assert sm.sm_softmax_version() == sm.ABI_VERSION == 10200
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert sm.sm_softmax_strerror(code) and sm.sm_softmax_strerror(code) != "unknown status"
    assert sm.sm_softmax_strerror(99) == "unknown status"


@pytest.mark.parametrize("args,want", [
    ((BASE, BASE * 2, 4, 8, 8, 8, 7), DTYPE),           # unknown dtype
    ((BASE, BASE * 2, -1, 8, 8, 8, F32), INVALID),      # negative M
    ((BASE, BASE * 2, 4, -8, 8, 8, F32), INVALID),      # negative N
    ((0, BASE * 2, 4, 8, 8, 8, F32), INVALID),          # null input
    ((BASE, 0, 4, 8, 8, 8, F32), INVALID),              # null output
    ((BASE, BASE * 2, 4, 8, 7, 8, F32), INVALID),       # input stride < N
    ((BASE, BASE * 2, 4, 8, 8, 7, F32), INVALID),       # output stride < N
    ((BASE + 2, BASE * 2, 4, 8, 8, 8, F32), INVALID),   # input not element aligned
    ((BASE, BASE * 2 + 1, 4, 8, 8, 8, BF16), INVALID),  # output not element aligned
    ((BASE, BASE * 2, 4, 1 << 31, 1 << 31, 1 << 31, F16), INVALID),  # N > 2^31 - 1
    ((BASE, BASE * 2, 1 << 62, 8, 1 << 40, 8, F32), INVALID),        # byte span overflows
    ((BASE, BASE + 16, 4, 8, 8, 8, F32), OVERLAP),      # shifted by 4 elements
    ((BASE, BASE, 4, 8, 8, 16, F32), OVERLAP),          # same base, different strides
    ((BASE, BASE, 0, 8, 8, 8, F32), OK),                # M == 0: nothing to do
    ((0, 0, 4, 0, 0, 0, F32), OK),                      # N == 0: nothing to do, pointers unused
])
def test_argument_validation(args, want):
    got = sm.sm_softmax_fwd(*args, 0)
    assert got == want, (args, got, sm.sm_softmax_strerror(got))
    # the extended entry point validates the same way
    assert sm.sm_softmax_fwd_ex(*args, None, 0, 0, 0) == want


def test_interleaved_rows_overlap_rule():
    # common stride 16 (elements, f32): out shifted by D elements
    for D, want in [(8, OK), (4, OVERLAP), (-8, OK), (-9, OVERLAP), (16, OVERLAP), (24, OK)]:
        rc = sm.sm_softmax_fwd(BASE, BASE + 4 * D if D >= 0 else BASE, 4, 8, 16, 16, F32, 0) \
            if D >= 0 else sm.sm_softmax_fwd(BASE - 4 * D, BASE, 4, 8, 16, 16, F32, 0)
        if rc == NO_DEVICE:
            rc = OK  # validation passed; no device on this host
        assert rc == want, (D, rc)


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_no_device():
    rc = sm.sm_softmax_fwd(BASE, BASE * 2, 4, 8, 8, 8, F32, 0)
    assert rc == NO_DEVICE


def plan(M, N, dtype, opts=None, in_ptr=BASE, out_ptr=BASE * 2, si=None, so=None):
    rc, info = sm.sm_softmax_plan_query(in_ptr, out_ptr, M, N, si or N, so or N, dtype, opts, 256)
    return rc, info.as_dict()


def test_plan_rule_one_pass_shapes():
    # (M, N, dtype) -> (lanes per row, vectors per lane, plan); the host-only query
    # assumes 2048 threads per CU, i.e. 2048 / block workgroups per CU, 256 CUs
    cases = {
        (8192, 127, F16): (32, 1, "persistent"),      # 254-byte rows: 17 windows when misaligned
        (8192, 256, F16): (32, 1, "persistent"),
        (8192, 1000, F16): (64, 2, "persistent"),
        (4096, 4096, BF16): (256, 2, "persistent"),   # 4096 groups = 2 rounds of 2048
        (8192, 4096, F16): (256, 2, "resident"),      # 8192 groups: 4 rounds
        (8192, 8192, F16): (256, 4, "resident"),
        (524288, 2048, BF16): (256, 1, "resident"),    # 16-bit, 4 GiB: one vector per lane
        (262144, 2048, BF16): (256, 1, "resident"),    # exactly 2 GiB
        (262143, 2048, BF16): (128, 2, "resident"),    # one row short of 2 GiB
        (65536, 2048, BF16): (128, 2, "resident"),
        (262144, 1024, F32): (128, 2, "resident"),     # FP32 keeps 128 x 2 at 2 GiB
        (16384, 1024, F32): (128, 2, "resident"),
        (128, 781, F32): (128, 2, "persistent"),      # 3124-byte rows: 196 windows
        (16, 8192, F32): (512, 4, "persistent"),
    }
    for (M, N, dt), (G, V, name) in cases.items():
        rc, p = plan(M, N, dt)
        assert rc == OK
        assert (p["lanes_per_row"], p["vecs_per_lane"], p["plan_name"]) == (G, V, name), (M, N, dt, p)
        es = 4 if dt == F32 else 2
        assert p["model_bytes"] == 2 * M * N * es
        assert p["lanes_per_row"] * p["vecs_per_lane"] * 16 >= N * es
        # streaming loads from 1 GiB of traffic up, on 128- to 1024-lane rows
        assert p["nt_loads"] == (1 if 2 * M * N * es >= 1 << 30 and G >= 128 else 0)
        if name == "persistent":
            assert p["grid"] == min(256 * 2048 // p["block"], -(-M // (p["block"] // G)))
            assert p["prefetch"] == (1 if G <= 64 else 0)


def test_nontemporal_option():
    rc, p = plan(4096, 4096, BF16, {"nontemporal": 1})
    assert rc == OK and p["nt_loads"] == 1
    rc, p = plan(8192, 1000, F16, {"nontemporal": 1})
    assert rc == OK and p["nt_loads"] == 0          # 64-lane rows have no streaming instance
    rc, p = plan(524288, 2048, BF16)
    assert p["nt_loads"] == 1
    rc, p = plan(524288, 2048, BF16, {"nontemporal": -1})
    assert p["nt_loads"] == 0
    rc, p = plan(64, 131072, BF16, {"nontemporal": 1})
    assert p["plan_name"] == "split" and p["nt_loads"] == 1
    rc, p = plan(64, 131072, BF16, {"nontemporal": 1, "plan": sm.SM_PLAN_WIDE})
    assert p["plan_name"] == "wide" and p["nt_loads"] == 1
    for bad in (2, 5, -2):
        rc, p = plan(524288, 2048, BF16, {"nontemporal": bad})
        assert rc == PLAN


def test_plan_rule_wide():
    W = {"plan": sm.SM_PLAN_WIDE}
    rc, p = plan(64, 131072, BF16, W)
    assert rc == OK and p["plan_name"] == "wide"
    assert p["chunks_per_wave"] == 1 and p["waves_per_row"] == 128
    assert p["workspace_bytes"] == 64 * 128 * 8
    assert p["model_bytes"] == 3 * 64 * 131072 * 2
    assert p["launches"] == 2 and p["grid"] == 64 * 128 // 4
    rc, p = plan(1024, 16384, BF16, W)  # 16384 chunks over 8192 wave slots -> 2 per wave
    assert p["chunks_per_wave"] == 2 and p["waves_per_row"] == 8
    rc, p = plan(4, 8193, F32, W)
    assert p["plan_name"] == "wide" and p["waves_per_row"] == 9


def test_plan_rule_split():
    # host path: 256 CUs x 8 workgroups = 2048 slots, half of them usable (1024)
    rc, p = plan(64, 131072, BF16)  # 16384 windows; V=4 -> 16 slices, 1024 items: one round
    assert rc == OK and p["plan_name"] == "split" and p["launches"] == 1
    assert (p["vecs_per_lane"], p["waves_per_row"], p["grid"]) == (4, 16, 1024)
    assert p["workspace_bytes"] == 64 * 16 * 32 and p["model_bytes"] == 2 * 64 * 131072 * 2
    rc, p = plan(4, 8193, BF16)  # just past the one-pass limit: 1025 windows -> 3 slices of 512
    assert p["plan_name"] == "split" and (p["vecs_per_lane"], p["waves_per_row"]) == (2, 3)
    assert p["grid"] == 12 and p["slice_windows"] == 342  # 1025 windows spread over 3 slices
    rc, p = plan(1024, 32769, BF16, {"plan": sm.SM_PLAN_SPLIT, "vecs_per_lane": 8})
    assert (p["waves_per_row"], p["slice_windows"]) == (3, 1366)  # not 2048 + 2048 + 1
    rc, p = plan(1, 1 << 20, BF16)  # V=2 would need 256 slices per row: V=4, 128 slices
    assert (p["vecs_per_lane"], p["waves_per_row"], p["grid"]) == (4, 128, 128)
    rc, p = plan(8, 1 << 18, BF16)  # V=2: 64 slices, 512 workgroups in one round
    assert (p["vecs_per_lane"], p["waves_per_row"], p["grid"]) == (2, 64, 512)
    # 2048 windows and at least 128 rows: one-pass rows (the grid's finding)
    rc, p = plan(1024, 16384, BF16)
    assert p["plan_name"] == "persistent" and (p["lanes_per_row"], p["vecs_per_lane"]) == (512, 4)
    rc, p = plan(8192, 16384, BF16)
    assert p["plan_name"] == "resident" and (p["lanes_per_row"], p["vecs_per_lane"]) == (512, 4)
    rc, p = plan(127, 16384, BF16)  # fewer rows: SPLIT
    assert p["plan_name"] == "split"
    rc, p = plan(1024, 65536, BF16)  # 8192 windows: SPLIT at any row count
    assert p["plan_name"] == "split"
    rc, p = plan(1024, 131072, BF16)  # rounds unavoidable: V=4 while rows need <= 16 slices
    assert (p["vecs_per_lane"], p["waves_per_row"], p["grid"]) == (4, 16, 1024)
    rc, p = plan(1024, 524288, BF16)  # V=4 would need 64 slices: the largest V, 32 slices
    assert (p["vecs_per_lane"], p["waves_per_row"], p["grid"]) == (8, 32, 1024)
    rc, p = plan(1, 1 << 25, BF16)  # 2^22 windows: even V=8 needs 2048 slices > 1024
    assert rc == OK and p["plan_name"] == "wide"
    S = {"plan": sm.SM_PLAN_SPLIT}
    rc, p = plan(1, 1 << 25, BF16, S)
    assert rc == PLAN
    rc, p = plan(64, 131072, BF16, {**S, "vecs_per_lane": 2, "grid": 64})
    assert rc == OK and (p["waves_per_row"], p["grid"]) == (32, 64)   # 2 rows per round
    rc, p = plan(64, 131072, BF16, {**S, "vecs_per_lane": 2, "grid": 48})
    assert rc == PLAN  # not a multiple of the 32 slices per row
    rc, p = plan(64, 131072, BF16, {**S, "vecs_per_lane": 3})
    assert rc == PLAN
    rc, p = plan(100, 3000, BF16, S)  # forced on a narrow row: 375 windows, V=2 -> 1 slice
    assert rc == OK and p["plan_name"] == "split" and (p["vecs_per_lane"], p["waves_per_row"]) == (2, 1)
    rc, p = plan(100, 3000, BF16, {**S, "vecs_per_lane": 1})
    assert rc == OK and p["waves_per_row"] == 2


def test_plan_rule_fp32_forward():
    """FP32 rows (fitted on an FP32 row-plan grid): SPLIT slices of one vector per lane
    while a row's slices fit one round, one-pass rows up to 8192 windows from 128 rows,
    the largest V in rounds, and WIDE with 8 chunks per wave for rows of 2^17 windows or
    more that SPLIT would take 4 or more rounds over; BF16 keeps its own choices there."""
    rc, p = plan(4, 8193, F32)  # 2049 windows -> 9 slices of 256
    assert p["plan_name"] == "split" and (p["vecs_per_lane"], p["waves_per_row"]) == (1, 9)
    assert p["grid"] == 36 and p["slice_windows"] == 228
    rc, p = plan(256, 32768, F32)  # 8192 windows, 256 rows: one-pass 1024 x 8
    assert (p["plan_name"], p["lanes_per_row"], p["vecs_per_lane"]) == ("persistent", 1024, 8)
    rc, p = plan(127, 32768, F32)  # fewer rows: SPLIT
    assert p["plan_name"] == "split"
    rc, p = plan(256, 65536, F32)  # 16384 windows in rounds: the largest V
    assert p["plan_name"] == "split" and (p["vecs_per_lane"], p["waves_per_row"]) == (8, 8)
    rc, p = plan(256, 1 << 20, F32)  # 2^18 windows, 128 slices per row, 32 rounds: WIDE
    assert (p["plan_name"], p["chunks_per_wave"], p["launches"]) == ("wide", 8, 2)
    rc, p = plan(4, 1 << 20, F32)  # one round of 512 slices: SPLIT
    assert p["plan_name"] == "split" and p["vecs_per_lane"] == 8
    rc, p = plan(256, 1 << 20, F32, {"plan": sm.SM_PLAN_SPLIT})  # forced: SPLIT in rounds
    assert rc == OK and p["plan_name"] == "split"
    rc, p = plan(256, 1 << 20, F32, {"grid": 1024})  # a fixed (valid) SPLIT grid keeps SPLIT
    assert rc == OK and p["plan_name"] == "split"
    for M, N, want in [(256, 65536, ("split", 8)), (4, 16386, ("split", 2)), (256, 1 << 21, ("split", 8))]:
        rc, p = plan(M, N, BF16)
        assert (p["plan_name"], p["vecs_per_lane"]) == want, (M, N, p)


def test_plan_at_the_width_limit():
    """N = 2^31 - 1, the widest row the ABI takes, in each dtype and alignment: the plan
    (SPLIT cannot hold a row's slices at once, so WIDE) has window and chunk counts that
    cover the row exactly, the same count the kernels form in 64 bits (the 32-bit sum
    head + N + E - 1 would overflow here); 2^31 is rejected."""
    N = (1 << 31) - 1
    for dt, es in ((F32, 4), (F16, 2), (BF16, 2)):
        E = 16 // es
        for base in (BASE, BASE + es):  # aligned, and one element past a 16-byte boundary
            head = (base % 16) // es
            rc, p = sm.sm_softmax_plan_query(base, BASE * 4, 1, N, N, N, dt, None, 256)
            assert rc == OK and p.as_dict()["plan_name"] == "wide", (dt, base, rc)
            nwin = (head + N + E - 1) // E
            assert head + N + E - 1 > (1 << 31) - 1 or dt == F32
            wpc = 1024 // E
            nchunks = (nwin + wpc - 1) // wpc
            d = p.as_dict()
            assert d["waves_per_row"] == (nchunks + d["chunks_per_wave"] - 1) // d["chunks_per_wave"]
            assert d["model_bytes"] == 3 * N * es
        rc, _ = sm.sm_softmax_plan_query(BASE, BASE * 4, 1, N + 1, N + 1, N + 1, dt, None, 256)
        assert rc == INVALID


def test_plan_forcing_and_limits():
    rc, p = plan(100, 5000, BF16, {"plan": sm.SM_PLAN_RESIDENT})
    assert rc == OK and p["plan_name"] == "resident" and p["grid"] == 100 and p["prefetch"] == 0
    rc, p = plan(100, 5000, BF16, {"plan": sm.SM_PLAN_WIDE})
    assert rc == OK and p["plan_name"] == "wide"
    rc, p = plan(100, 5000, BF16, {"plan": sm.SM_PLAN_PERSISTENT, "lanes_per_row": 64,
                                   "vecs_per_lane": 1})
    assert rc == PLAN  # 64 windows hold 512 elements, not 5000
    rc, p = plan(100, 40000, BF16, {"plan": sm.SM_PLAN_RESIDENT})
    assert rc == OK and (p["lanes_per_row"], p["vecs_per_lane"]) == (1024, 8)
    rc, p = plan(100, 2000, BF16, {"plan": sm.SM_PLAN_RESIDENT})
    assert (p["lanes_per_row"], p["vecs_per_lane"]) == (128, 2)   # one table for both plans
    rc, p = plan(100, 2000, BF16, {"plan": sm.SM_PLAN_PERSISTENT})
    assert (p["lanes_per_row"], p["vecs_per_lane"]) == (128, 2)
    # the 16-bit long-call shape applies to automatic shapes only
    rc, p = plan(524288, 2048, BF16, {"lanes_per_row": 128})
    assert rc == OK and (p["lanes_per_row"], p["vecs_per_lane"]) == (128, 2)
    rc, p = plan(524288, 2048, BF16, {"plan": sm.SM_PLAN_PERSISTENT})
    assert rc == OK and (p["lanes_per_row"], p["vecs_per_lane"]) == (128, 2)
    rc, p = plan(100, 70000, BF16, {"plan": sm.SM_PLAN_RESIDENT})
    assert rc == PLAN
    rc, p = plan(100, 500, BF16, {"plan": 9})
    assert rc == PLAN
    rc, p = plan(10 ** 6, 100, F16, {"plan": sm.SM_PLAN_PERSISTENT})
    assert p["grid"] == 256 * 8  # occupancy assumed 8 workgroups per CU on the host path


def test_plan_grid_capped_at_2_32_threads():
    """A dispatch counts its work-items in 32 bits: one-pass grids are capped at 2^32 - 1
    threads and the row kernels stride over the rows beyond (64-bit row indices), forward,
    backward and RMSNorm alike; the two-pass WIDE plan, which gives every wave fixed
    chunks, refuses a grid it cannot launch."""
    M = 1 << 34  # rows of 2 BF16 elements: 2^30 workgroups of 16 rows would be needed
    cap = 0xFFFFFFFF
    for opts in (None, {"plan": sm.SM_PLAN_RESIDENT}, {"plan": sm.SM_PLAN_PERSISTENT}):
        rc, info = sm.sm_softmax_plan_query(1 << 40, 1 << 41, M, 2, 2, 2, BF16, opts, 256)
        p = info.as_dict()
        assert rc == OK and p["plan_name"] in ("resident", "persistent"), (opts, rc, p)
        rows_per_group = p["block"] // p["lanes_per_row"]
        assert p["grid"] * p["block"] <= cap
        if p["plan_name"] == "resident":
            assert p["grid"] == cap // p["block"] < M // rows_per_group
        rc, info = sm.sm_softmax_bwd_plan_query(1 << 40, 1 << 41, 1 << 42, M, 2, 2, 2, 2, BF16,
                                                opts, 256)
        p = info.as_dict()
        assert rc == OK and p["grid"] * p["block"] <= cap, (opts, rc, p)
        rc, info = sm.sm_rmsnorm_plan_query(1 << 40, 2 << 40, 3 << 40, 4 << 40, 0, M, 2, 2, 2, 2,
                                            2, 1e-6, BF16, opts, 256)
        p = info.as_dict()
        assert rc == OK and p["grid"] * p["block"] <= cap, (opts, rc, p)
    rc, _ = sm.sm_softmax_plan_query(1 << 40, 1 << 41, M, 2, 2, 2, BF16, {"plan": sm.SM_PLAN_WIDE},
                                     256)
    assert rc == PLAN


def test_plan_phase_flag():
    rc, p = plan(4, 64, F16)
    assert p["same_phase"] == 1
    rc, p = plan(4, 64, F16, out_ptr=BASE * 2 + 2)
    assert p["same_phase"] == 0
    rc, p = plan(4, 60, F16, si=64, so=60)
    assert p["same_phase"] == 0
    rc, p = plan(4, 60, F16, si=64, so=72)
    assert p["same_phase"] == 1


# ------------------------------------------------------------------ backward entry points

@pytest.mark.parametrize("args,want", [
    ((BASE, BASE * 2, BASE * 3, 4, 8, 8, 8, 8, 9), DTYPE),
    ((BASE, BASE * 2, 0, 4, 8, 8, 8, 8, F32), INVALID),            # null dx
    ((BASE, BASE * 2, BASE * 3, 4, 8, 8, 7, 8, F32), INVALID),     # dy stride < N
    ((BASE, BASE * 2, BASE + 16, 4, 8, 8, 8, 8, F32), OVERLAP),    # dx overlaps y partially
    ((BASE, BASE * 2, BASE * 2 + 4, 4, 8, 8, 8, 8, F32), OVERLAP), # dx overlaps dy partially
    ((BASE, BASE, BASE * 3, 0, 8, 8, 8, 8, F32), OK),              # M == 0
])
def test_backward_validation(args, want):
    assert sm.sm_softmax_bwd(*args, 0) == want
    assert sm.sm_softmax_bwd_ex(*args, None, 0, 0, 0) == want


def test_backward_in_place_passes_validation():
    for y, dy, dx in [(BASE, BASE * 2, BASE), (BASE, BASE * 2, BASE * 2), (BASE, BASE, BASE * 3)]:
        rc = sm.sm_softmax_bwd(y, dy, dx, 4, 8, 8, 8, 8, F32, 0)
        assert rc in (OK, NO_DEVICE), rc


def test_backward_plan_rule():
    def q(M, N, dt, opts=None, dy=BASE * 2, sd=None):
        rc, info = sm.sm_softmax_bwd_plan_query(BASE, dy, BASE * 3, M, N, N, sd or N, N, dt,
                                                opts, 256)
        return rc, info.as_dict()
    rc, p = q(4096, 4096, BF16)
    assert rc == OK and (p["lanes_per_row"], p["vecs_per_lane"]) == (256, 2)
    assert p["model_bytes"] == 3 * 4096 * 4096 * 2 and p["plan_name"] == "resident"
    assert p["grid"] == 4096 and p["nt_loads"] == 1  # 96 MiB moved: streaming loads
    assert p["dy_same_phase"] == 1 and p["same_phase"] == 1
    # one-pass backward rows stream from 32 MiB of traffic up, on 128- to 1024-lane rows
    for (M, N, dt), nt in {(1024, 4096, BF16): 0, (1366, 4096, BF16): 1, (1365, 4096, BF16): 0,
                           (4096, 1024, BF16): 0, (2048, 4096, BF16): 1}.items():
        rc, p = q(M, N, dt)
        assert rc == OK and p["nt_loads"] == nt, (M, N, p)
        assert p["nt_loads"] == (1 if 3 * M * N * 2 >= 32 << 20 and p["lanes_per_row"] >= 128 else 0)
    rc, p = q(4096, 4096, BF16, {"nontemporal": -1})
    assert p["nt_loads"] == 0
    rc, p = q(524288, 2048, BF16)  # 6 GiB moved: streaming loads
    assert rc == OK and p["plan_name"] == "resident" and p["nt_loads"] == 1
    rc, p = q(4096, 4096, BF16, {"plan": 2})
    assert p["plan_name"] == "persistent" and p["grid"] < 4096
    rc, p = q(64, 131072, BF16)
    assert p["plan_name"] == "split" and p["model_bytes"] == 3 * 64 * 131072 * 2
    assert p["workspace_bytes"] == 64 * p["waves_per_row"] * 32 and p["vecs_per_lane"] == 4
    rc, p = q(64, 131072, BF16, {"plan": sm.SM_PLAN_WIDE})
    assert p["plan_name"] == "wide" and p["model_bytes"] == 5 * 64 * 131072 * 2
    assert p["workspace_bytes"] == 64 * p["waves_per_row"] * 8
    rc, p = q(64, 131072, BF16, {"plan": sm.SM_PLAN_SPLIT, "vecs_per_lane": 8})
    assert rc == PLAN  # backward slices hold at most 4 vectors per lane
    rc, p = q(8, 1000, F16, dy=BASE * 2 + 2)
    assert p["dy_same_phase"] == 0
    rc, p = q(8, 1000, F16, {"vecs_per_lane": 8})
    assert rc == PLAN  # backward rows hold at most 4 vectors per lane


# ------------------------------------------------------------------ residual RMSNorm
X, R, W, Y, S = BASE, BASE * 2, BASE * 3, BASE * 4, BASE * 5


def rms_q(M, N, dt, opts=None, r=R, s=0, eps=1e-6, **kw):
    a = dict(x=X, r=r, w=W, y=Y, s=s, sx=N, sr=N, sy=N, ss=N)
    a.update(kw)
    rc, info = sm.sm_rmsnorm_plan_query(a["x"], a["r"], a["w"], a["y"], a["s"], M, N, a["sx"],
                                        a["sr"], a["sy"], a["ss"], eps, dt, opts, 256)
    return rc, info.as_dict()


@pytest.mark.parametrize("kw,want", [
    (dict(dt=9), DTYPE),
    (dict(x=0), INVALID), (dict(w=0), INVALID), (dict(y=0), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(sx=7), INVALID), (dict(sr=7), INVALID), (dict(sy=7), INVALID),
    (dict(y=X + 16), OVERLAP),              # y overlaps x partially
    (dict(y=R + 4), OVERLAP),               # y overlaps the residual partially
    (dict(w=Y + 8), OVERLAP),               # the weight inside y
    (dict(s=Y), OVERLAP),                   # residual_out on y
    (dict(s=X + 4), OVERLAP),               # residual_out overlaps x partially
    (dict(w=S, s=S - 16), OVERLAP),         # the weight inside residual_out
    (dict(y=X), OK), (dict(y=R), OK), (dict(s=R), OK), (dict(s=X, y=Y), OK),  # exactly in place
    (dict(r=0), OK),
])
def test_rmsnorm_validation(kw, want):
    dt = kw.pop("dt", F32)
    eps = kw.pop("eps", 1e-6)
    rc, _ = rms_q(4, 8, dt, eps=eps, **kw)
    assert rc == want, (kw, rc)


def test_rmsnorm_zero_size_and_no_device():
    assert sm.sm_rmsnorm_fwd(X, R, W, Y, 0, 0, 8, 8, 8, 8, 8, 1e-6, F32, 0) == OK
    rc = sm.sm_rmsnorm_fwd(X, R, W, Y, 0, 4, 8, 8, 8, 8, 8, 1e-6, F32, 0)
    assert rc in (OK, NO_DEVICE)


def test_rmsnorm_plan_rule():
    # model_bytes: compulsory HBM bytes (x, y, residual, residual_out per element; w once)
    rc, p = rms_q(64, 8192, BF16)  # 1024 windows: one-pass 256 x 4
    assert rc == OK and p["plan_name"] == "persistent"
    assert (p["lanes_per_row"], p["vecs_per_lane"]) == (256, 4)
    assert p["model_bytes"] == 3 * 64 * 8192 * 2 + 8192 * 2 and p["dy_same_phase"] == 1
    rc, p = rms_q(64, 8192, BF16, s=S)  # + residual_out
    assert p["model_bytes"] == 4 * 64 * 8192 * 2 + 8192 * 2
    rc, p = rms_q(64, 8192, BF16, r=0)  # plain RMSNorm
    assert p["model_bytes"] == 2 * 64 * 8192 * 2 + 8192 * 2
    rc, p = rms_q(4, 32769, BF16)       # few wide rows: SPLIT, V=1, 17 slices of 241 windows
    assert p["plan_name"] == "split" and (p["vecs_per_lane"], p["waves_per_row"]) == (1, 17)
    assert p["slice_windows"] == 241 and p["launches"] == 1
    assert p["workspace_bytes"] == (4 * 17 * 32 + 255) // 256 * 256
    rc, p = rms_q(4, 32769, BF16, {"plan": sm.SM_PLAN_WIDE})  # two launches, x and r read twice
    assert p["plan_name"] == "wide" and p["launches"] == 2
    assert p["model_bytes"] == 5 * 4 * 32769 * 2 + 32769 * 2
    rc, p = rms_q(8, 1 << 20, BF16)     # 128 slices, one round: SPLIT
    assert p["plan_name"] == "split" and p["grid"] == 1024
    rc, p = rms_q(16, 1 << 20, BF16)    # 128 slices in two rounds: two launches without waits
    assert p["plan_name"] == "wide" and p["launches"] == 2
    rc, p = rms_q(16, 1 << 20, BF16, {"plan": sm.SM_PLAN_SPLIT})  # forced: rounds are allowed
    assert p["plan_name"] == "split"
    rc, p = rms_q(1, 1 << 26, BF16)     # slices cannot be resident together: two launches
    assert rc == OK and p["plan_name"] == "wide" and p["vecs_per_lane"] == 4
    rc, p = rms_q(1, 1 << 26, BF16, {"plan": sm.SM_PLAN_SPLIT})
    assert rc == PLAN
    rc, p = rms_q(8, 1000, F16, {"vecs_per_lane": 8})
    assert rc == PLAN                   # rows hold at most 4 vectors per lane
    rc, p = rms_q(8, 1000, F16, r=R + 2)  # residual at another 16-byte phase
    assert p["dy_same_phase"] == 0
    # one-pass rows stream x and the residual from 256 MiB of traffic up (128+ lanes)
    rc, p = rms_q(16384, 4096, F16)     # 384 MiB
    assert p["plan_name"] == "resident" and p["nt_loads"] == 1
    rc, p = rms_q(4096, 4096, BF16)     # 96 MiB
    assert p["nt_loads"] == 0
    rc, p = rms_q(4096, 4096, BF16, {"nontemporal": 1})
    assert p["nt_loads"] == 1
    rc, p = rms_q(16384, 4096, F16, {"nontemporal": -1})
    assert p["nt_loads"] == 0


# ------------------------------------------------------------------ fused attention
def attn(BH=2, Sq=64, Sk=64, d=128, q=BASE, k=BASE * 2, v=BASE * 3, o=BASE * 4, lse=0,
         strides=None, scale=0.125, causal=1, dt=BF16):
    st = strides or (d, Sq * d, d, Sk * d, d, Sk * d, d, Sq * d)
    return sm.sm_attention_fwd(q, k, v, o, lse, BH, Sq, Sk, d, st, scale, causal, dt, 0)


@pytest.mark.parametrize("kw,want", [
    (dict(dt=F32), DTYPE), (dict(dt=9), DTYPE),
    (dict(d=96), INVALID), (dict(d=0), INVALID),
    (dict(q=BASE + 2), INVALID),                       # not 16-byte aligned
    (dict(strides=(130, 64 * 130, 128, 8192, 128, 8192, 128, 8192)), INVALID),  # row stride % 8
    (dict(strides=(120, 64 * 120, 128, 8192, 128, 8192, 128, 8192)), INVALID),  # row stride < d
    (dict(strides=(128, 8192, 128, 8192, 128, 8192, 128, 64)), INVALID),        # o heads overlap
    (dict(BH=1, strides=(128, 8192, (1 << 24) + 8, 0, 128, 8192, 128, 8192)), INVALID),  # k row stride > 2^24
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(o=BASE + 4096), OVERLAP),                    # o inside q
    (dict(o=BASE * 3 + 1024), OVERLAP),                # o inside v
    (dict(lse=BASE * 4 + 64), OVERLAP),                # lse inside o
    (dict(lse=BASE * 5 + 2), INVALID),                 # lse not 4-byte aligned
    (dict(BH=0), OK), (dict(Sq=0), OK),
])
def test_attention_validation(kw, want):
    rc = attn(**kw)
    assert rc == want, (kw, rc)


def test_attention_valid_call_without_device():
    rc = attn(lse=BASE * 5)
    assert rc in (OK, NO_DEVICE)
    rc = attn(Sk=0, k=0, v=0)  # no keys: every query gets zeros
    assert rc in (OK, NO_DEVICE)


def test_noalloc_entry_point_validation():
    """The allocation-free forward validates exactly as sm_softmax_fwd (before any HIP
    call), and its scratch limit in the header matches the binding's."""
    for args, want in [((BASE, BASE * 2, 4, 8, 8, 8, 7), DTYPE),
                       ((BASE, BASE * 2, 4, 8, 7, 8, F32), INVALID),
                       ((BASE, BASE + 16, 4, 8, 8, 8, F32), OVERLAP),
                       ((BASE, BASE, 0, 8, 8, 8, F32), OK),
                       ((0, 0, 4, 0, 0, 0, F32), OK)]:
        assert sm.sm_softmax_fwd_noalloc(*args, 0) == want == sm.sm_softmax_fwd(*args, 0)
    if not gpu_available():
        assert sm.sm_softmax_fwd_noalloc(BASE, BASE * 2, 4, 8, 8, 8, F32, 0) == NO_DEVICE
    text = open(os.path.join(INCLUDE, "sm_softmax.h")).read()
    m = re.search(r"#define SM_NOALLOC_SCRATCH_BYTES \(1u << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == sm.NOALLOC_SCRATCH_BYTES
