// sm_softmax.hip -- host side of the gfx950 row-softmax library: argument
// validation, plan selection, per-device occupancy cache, launches, and the C
// ABI declared in include/sm_softmax.h and include/sm_bench.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <map>
#include <mutex>
#include <vector>

#include "sm_attention.hpp"
#include "sm_bench.h"
#include "sm_bwd.hpp"
#include "sm_kernels.hpp"
#include "sm_launch.hpp"
#include "sm_rmsnorm.hpp"
#include "sm_softmax.h"

namespace smx {

// ------------------------------------------------------------ measurement kernels
// 16-byte copy (bandwidth ceiling, counter calibration) and a read-only sweep
// that evicts earlier data from L2 and MALL without leaving dirty lines behind.
// SC1: device-scope stores, the row kernels' store policy; else plain stores.
template <bool SC1>
__global__ void __launch_bounds__(256) k_copy16(const uint4* src, uint4* dst, int64_t n) {
    const int64_t step = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
        if constexpr (SC1)
            store16(reinterpret_cast<unsigned char*>(dst + i), src[i]);
        else
            dst[i] = src[i];
    }
}

__global__ void __launch_bounds__(256) k_sweep_read16(const uint4* buf, int64_t n) {
    const int64_t step = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    asm volatile("" ::"v"(acc));  // the loads stay; nothing is written
}

// ------------------------------------------------------------ wide kernels
StatsKernelFn wide_stats_kernel(int dtype, int NT) {
    switch (dtype) {
    case kF32: return NT ? &k_wide_stats<kF32, true> : &k_wide_stats<kF32, false>;
    case kF16: return NT ? &k_wide_stats<kF16, true> : &k_wide_stats<kF16, false>;
    case kBF16: return NT ? &k_wide_stats<kBF16, true> : &k_wide_stats<kBF16, false>;
    default: return nullptr;
    }
}
NormKernelFn wide_norm_kernel(int dtype, int NT) {
    switch (dtype) {
    case kF32: return NT ? &k_wide_norm<kF32, true> : &k_wide_norm<kF32, false>;
    case kF16: return NT ? &k_wide_norm<kF16, true> : &k_wide_norm<kF16, false>;
    case kBF16: return NT ? &k_wide_norm<kBF16, true> : &k_wide_norm<kBF16, false>;
    default: return nullptr;
    }
}

namespace {

constexpr int64_t kResidentMaxCols = 8192;  // widest row the one-pass plans take by default
constexpr int kChunk = 1024;                // elements per online-recurrence chunk (wide path)
constexpr int64_t kMaxThreadsPerLaunch = 0xFFFFFFFFLL;

thread_local int t_last_hip_error = 0;

int hip_fail(hipError_t e) {
    t_last_hip_error = (int)e;
    return SM_ERR_HIP;
}

int elem_bytes(int dtype) { return dtype == SM_F32 ? 4 : 2; }

// ------------------------------------------------------------ validation
struct Problem {
    uintptr_t in, out;
    int64_t M, N, in_stride, out_stride;
    int dtype;
};

// Byte span covered by rows 0..M-1 (M >= 1, N >= 1), or -1 on overflow.
int64_t span_bytes(int64_t M, int64_t N, int64_t stride, int es) {
    if (M == 1) return N * es;
    const int64_t lim = INT64_MAX / es - N;
    if (lim < 0 || (M - 1) > lim / stride) return -1;
    return ((M - 1) * stride + N) * es;
}

int validate(const Problem& p) {
    if (p.dtype != SM_F32 && p.dtype != SM_F16 && p.dtype != SM_BF16) return SM_ERR_DTYPE;
    if (p.M < 0 || p.N < 0) return SM_ERR_INVALID;
    if (p.M == 0 || p.N == 0) return SM_OK;
    if (p.N > INT32_MAX) return SM_ERR_INVALID;
    if (!p.in || !p.out) return SM_ERR_INVALID;
    const int es = elem_bytes(p.dtype);
    if ((p.in % es) || (p.out % es)) return SM_ERR_INVALID;
    if (p.M > 1 && (p.in_stride < p.N || p.out_stride < p.N)) return SM_ERR_INVALID;
    const int64_t si = span_bytes(p.M, p.N, p.in_stride, es);
    const int64_t so = span_bytes(p.M, p.N, p.out_stride, es);
    if (si < 0 || so < 0) return SM_ERR_INVALID;
    if (p.in > UINTPTR_MAX - (uint64_t)si || p.out > UINTPTR_MAX - (uint64_t)so) return SM_ERR_INVALID;

    // Overlap: disjoint byte ranges are fine; so is exactly in place.
    const bool disjoint = p.in + (uint64_t)si <= p.out || p.out + (uint64_t)so <= p.in;
    if (disjoint) return SM_OK;
    if (p.in == p.out && (p.M == 1 || p.in_stride == p.out_stride)) return SM_OK;
    if (p.M > 1 && p.in_stride == p.out_stride) {
        // Interleaved rows with a common stride S: row i of out meets row j of
        // in iff |D - k*S| < N (elements) for k = i - j, |k| <= M - 1.
        const int64_t S = p.in_stride;
        const int64_t D = ((int64_t)p.out - (int64_t)p.in) / es;
        int64_t k0 = D / S;
        if (D % S != 0 && D < 0) --k0;  // floor
        for (int64_t k = k0; k <= k0 + 1; ++k) {
            if (k < -(p.M - 1) || k > p.M - 1) continue;
            const int64_t gap = D - k * S;
            if (gap > -p.N && gap < p.N) return SM_ERR_OVERLAP;
        }
        return SM_OK;
    }
    return SM_ERR_OVERLAP;
}

// ------------------------------------------------------------ plan selection
struct RowShape {
    int G, V;
};
// Row shapes (lanes per row, vectors per lane) by 16-byte windows needed,
// narrowest first, measured on MI355X with cold calls. Rows of up to 64 windows
// take one vector per lane in a sub-wave or wave. Wider rows spread over 2-16
// waves with 2-4 vectors per lane, which beat 4-8 vectors per lane in one wave
// (fewer registers, more waves in flight, shorter per-row latency). Rows of
// 129-256 windows take 128 x 2: at the same occupancy a CU then holds twice the
// rows, and so twice the loads, in flight that 256 x 1 holds, and 256 x 2 would
// spend half of its lanes' arithmetic on padding (16384 x 1024 FP32: 21.4 us
// against 25.5 for 256 x 1 and 33.5 for 256 x 2; 65536 x 2048 BF16: 75.4, 77.7
// and 80.0 us; 65536 x 1500 FP16: 60.1 against 76.5 and 91.6 us).
constexpr RowShape kShapes[] = {{16, 1},  {32, 1},  {64, 1},   {64, 2},   {128, 2},
                                {256, 2}, {256, 4}, {512, 4}, {1024, 4}, {1024, 8}};
// ... except in 16-bit calls of at least this many bytes, where one workgroup
// per row takes 256 x 1: with that many rows HBM is saturated with fewer rows in
// flight, and fewer was faster (524288 rows of BF16, N = 2048: 606 against 639
// us; N = 2000: 758 against 928; 262144 x 2048: 307 against 311), while FP32
// rows (262144 x 1024: 356 against 312 us) and smaller calls (131072 x 2048
// BF16: 148 against 145 us) kept 128 x 2.
constexpr int64_t kLongCallBytes = int64_t(2) << 30;
// Calls that move at least this many bytes stream their input past the MALL
// (524288 x 2048 BF16, 4 GiB: 639 against 659 us; below 1 GiB streaming loads
// cost 1-3%).
constexpr int64_t kNtLoadBytes = int64_t(1) << 30;
// SPLIT workgroup width (lanes per slice) and default wait budget (polls).
constexpr int kSplitLanes = 256;
constexpr int kSplitSpinDefault = 1 << 20;

template <size_t K>
bool pick_shape(const RowShape (&tab)[K], int64_t nw, int fixG, int fixV, int& G, int& V) {
    for (const RowShape& s : tab) {
        if ((fixG && s.G != fixG) || (fixV && s.V != fixV)) continue;
        if ((int64_t)s.G * s.V >= nw) {
            G = s.G;
            V = s.V;
            return true;
        }
    }
    if (fixG && fixV) {  // both fixed: any built shape that covers the row
        if ((int64_t)fixG * fixV < nw) return false;
        G = fixG;
        V = fixV;
        return true;
    }
    if (fixG) {  // a fixed G outside the table: smallest V that fits
        for (int v : {1, 2, 4, 8})
            if ((int64_t)fixG * v >= nw) { G = fixG; V = v; return true; }
    } else if (fixV) {
        for (int g : {16, 32, 64, 128, 256, 512, 1024})
            if ((int64_t)g * fixV >= nw) { G = g; V = fixV; return true; }
    }
    return false;
}

bool built_shape(int G, int V, int PF) {
    const bool g_ok = G == 16 || G == 32 || G == 64 || G == 128 || G == 256 || G == 512 || G == 1024;
    const bool v_ok = V == 1 || V == 2 || V == 4 || V == 8;
    return g_ok && v_ok && (!PF || G <= 256);
}

// Automatic choice between one-pass rows and SPLIT: rows of up to 8192 elements
// always run one-pass (the resident limit of the Warpline README's online-softmax
// description); wider rows run one-pass when they fit in kOnePassWideWindows
// 16-byte windows and there are at least kOnePassWideRows of them, else SPLIT.
// On the row-plan grid (BF16, forward) one-pass rows won from 128 rows up at
// widths to 32768 (SPLIT lost 10 to 47% there) and lost to SPLIT below; rows of
// 8192 windows (65536 BF16) did better split at every row count.
constexpr int64_t kOnePassWideWindows = 4096;
constexpr int64_t kOnePassWideRows = 128;

bool one_pass_rule(int64_t M, int64_t N, int64_t nw) {
    return N <= kResidentMaxCols || (nw <= kOnePassWideWindows && M >= kOnePassWideRows);
}

// FP32 forward, refitted on an FP32 row-plan grid (18 row counts x 10 widths, two runs;
// the BF16 rule there: mean regret 6.9%, 57 of 180 cells over 10%). FP32 rows cost more
// VALU per 16-byte window (compensated sums and exponentials), which moves three choices:
// one-pass rows up to 8192 windows from 128 rows (the 1024 x 8 shape beat SPLIT by 27 to
// 36% at width 32768); SPLIT slices of one vector per lane while a row's slices fit one
// round (V = 2 lost 12 to 23% at up to 24 rows); no V = 4 preference in rounds; and the
// two-pass WIDE plan with 8 chunks per wave for rows of at least 2^17 windows that would
// take SPLIT 4 or more rounds (SPLIT lost 11 to 21% there). Mean regret 0.8%, p90 2.4%,
// 2 cells over 10% on the grid it was fitted on.
constexpr int64_t kF32OnePassWideWindows = 8192;
constexpr int64_t kF32WideWindows = int64_t(1) << 17;
constexpr int64_t kF32WideRounds = 4;
constexpr int kF32WideChunksPerWave = 8;

bool fwd_one_pass_rule(int64_t M, int64_t N, int64_t nw, int dtype) {
    return one_pass_rule(M, N, nw) ||
           (dtype == SM_F32 && nw <= kF32OnePassWideWindows && M >= kOnePassWideRows);
}

struct DeviceView {
    int cus;
    // workgroups per CU for a row-kernel instance / for the wide kernels
    int (*occ_row)(void* ctx, int dtype, int G, int V, int PF);
    int (*occ_wide)(void* ctx, int dtype);
    // workgroups per CU for a split-kernel instance (bwd: the backward one)
    int (*occ_split)(void* ctx, int dtype, int V, int bwd);
    void* ctx;
};

// ------------------------------------------------------------ SPLIT geometry
// Slices per row P for V vectors per lane, and the grid: at most half of the
// resident capacity, a multiple of P, so that every row's slices can be resident
// together (with room to spare for other work on the device). Returns false when
// even one row's slices exceed that budget, or a forced grid breaks the rules.
bool split_geometry(int64_t M, int64_t nw, int V, int64_t cap_slots, int64_t fixed_grid,
                    int64_t& P, int64_t& grid) {
    const int64_t S = (int64_t)kSplitLanes * V;
    P = std::max<int64_t>(1, (nw + S - 1) / S);
    if (P > INT32_MAX || M > INT64_MAX / P) return false;
    const int64_t cap = (cap_slots / 2) / P * P;
    if (cap < P) return false;
    const int64_t items = M * P;
    if (fixed_grid > 0) {
        if (fixed_grid % P != 0 || fixed_grid > cap) return false;
        grid = std::min(fixed_grid, items);
    } else {
        grid = std::min(items, cap);
    }
    return true;
}

// Automatic SPLIT shape, in order of preference:
//   1. the smallest V >= vmin whose rows need at most kSplitMaxAutoSlices slices and
//      whose slices of all rows fit in one round (most workgroups in flight);
//   2. with rounds unavoidable, V = vround when rows need at most round_max slices
//      (shorter rounds than the widest slices at the same traffic);
//   3. the largest V that fits at all (fewest slices per row).
// Softmax: vmin = 2, vround = 4, round_max = 16. Residual RMSNorm (it holds x, the
// residual and the weight in registers): vmin = 1, vround = 2, round_max = 8.
// Returns 0 when no V fits. Measured on MI355X, cold BF16 (us, V = 1 / 2 / 4 / 8):
// 1 x 1048576: 7.6 / 6.2 / 5.7 / 6.6; 8 x 262144: 5.8 / 5.4 / 5.6 / 6.9; 16 x 65536:
// 4.6 / 4.5 / 5.1 / 6.4; 64 x 131072: - / 13.8 / 11.3 / 11.1. On the row-plan grid
// (18 row counts x 10 widths) rule 2 took the width-32769 column from 9.4% to 3.1%
// mean regret, while V = 4 at 32 or more slices per row cost 4 to 21% at widths
// from 262144 up.
constexpr int64_t kSplitMaxAutoSlices = 128;
constexpr int64_t kSplitRoundSlices = 16;
// RMSNorm, refitted on its grid once phase-shifted weights load as aligned windows
// (the 4-vector slices got faster there): mean regret 2.8% -> 0.6%
constexpr int64_t kRmsRoundSlices = 8;

int split_auto_v(int64_t M, int64_t nw, int vmin, int vmax, int vround, int64_t round_max,
                 int64_t cus, void* ctx, int dtype, int bwd, int (*occ)(void*, int, int, int),
                 int64_t& P, int64_t& grid) {
    int64_t cp[4] = {0, 0, 0, 0}, cg[4] = {0, 0, 0, 0};
    bool ok[4] = {false, false, false, false};
    int vs[4] = {0, 0, 0, 0}, n = 0;
    for (int v = vmin; v <= vmax; v *= 2, ++n) {
        const int64_t slots = (int64_t)std::max(1, occ(ctx, dtype, v, bwd)) * cus;
        vs[n] = v;
        ok[n] = split_geometry(M, nw, v, slots, 0, cp[n], cg[n]);
    }
    for (int i = 0; i < n; ++i) {  // 1
        if (ok[i] && M * cp[i] <= cg[i] && cp[i] <= kSplitMaxAutoSlices) {
            P = cp[i];
            grid = cg[i];
            return vs[i];
        }
    }
    for (int i = 0; i < n; ++i) {  // 2
        if (ok[i] && vs[i] == vround && cp[i] <= round_max) {
            P = cp[i];
            grid = cg[i];
            return vround;
        }
    }
    for (int i = n - 1; i >= 0; --i) {  // 3
        if (ok[i]) {
            P = cp[i];
            grid = cg[i];
            return vs[i];
        }
    }
    return 0;
}

// no_split: AUTO takes the two-pass WIDE plan where it would take SPLIT, and a forced
// SPLIT is refused. Set when the call is being captured into a graph (SPLIT tags its
// slots with a per-call id fixed at launch, which a graph would replay unchanged, so a
// replay could read the previous replay's statistics before its own peers publish),
// and by the allocation-free entry point for calls in place.
int make_plan(const Problem& p, const sm_softmax_opts& o, const DeviceView& dev, bool no_split,
              sm_plan_info* pi) {
    *pi = sm_plan_info{};
    const int es = elem_bytes(p.dtype);
    const int E = 16 / es;
    const bool in_aligned = (p.in % 16 == 0) && (p.M == 1 || (p.in_stride * es) % 16 == 0);
    const int max_head = in_aligned ? 0 : E - 1;
    const int64_t nw_max = (max_head + p.N + E - 1) / E;
    pi->same_phase = ((p.in - p.out) % 16 == 0) &&
                     (p.M == 1 || (((p.in_stride - p.out_stride) * es) % 16 == 0));

    int plan = o.plan;
    if (plan < SM_PLAN_AUTO || plan > SM_PLAN_SPLIT) return SM_ERR_PLAN;
    const bool auto_plan = plan == SM_PLAN_AUTO;
    if (auto_plan) plan = fwd_one_pass_rule(p.M, p.N, nw_max, p.dtype) ? SM_PLAN_RESIDENT : SM_PLAN_SPLIT;
    if (o.nontemporal < -1 || o.nontemporal > 1) return SM_ERR_PLAN;
    const bool f32 = p.dtype == SM_F32;
    int64_t wide_cpw = 0;  // preferred chunks per wave of an automatic WIDE plan (0: by the grid)
    if (plan == SM_PLAN_SPLIT && no_split) {
        if (!auto_plan) return SM_ERR_PLAN;
        plan = SM_PLAN_WIDE;
    }

    if (plan == SM_PLAN_SPLIT) {
        int64_t P = 0, grid = 0;
        int V = o.vecs_per_lane;
        if (V) {
            if (V != 1 && V != 2 && V != 4 && V != 8) return SM_ERR_PLAN;
            const int64_t slots = (int64_t)std::max(1, dev.occ_split(dev.ctx, p.dtype, V, 0)) * dev.cus;
            if (!split_geometry(p.M, nw_max, V, slots, o.grid, P, grid)) V = 0;
        } else {
            V = split_auto_v(p.M, nw_max, f32 ? 1 : 2, 8, 4, f32 ? 0 : kSplitRoundSlices, dev.cus, dev.ctx,
                             p.dtype, 0, dev.occ_split, P, grid);
            if (V && f32 && auto_plan && o.grid <= 0 && nw_max >= kF32WideWindows &&
                (p.M * P + grid - 1) / grid >= kF32WideRounds) {
                V = 0;
                wide_cpw = kF32WideChunksPerWave;
            }
            if (V && o.grid > 0) {
                const int64_t slots = (int64_t)std::max(1, dev.occ_split(dev.ctx, p.dtype, V, 0)) * dev.cus;
                if (!split_geometry(p.M, nw_max, V, slots, o.grid, P, grid)) V = 0;
            }
        }
        if (V) {
            const int64_t model = 2 * p.M * p.N * es;
            const bool nt = o.nontemporal == 1 || (o.nontemporal == 0 && model >= kNtLoadBytes);
            pi->plan = SM_PLAN_SPLIT;
            pi->lanes_per_row = kSplitLanes;
            pi->vecs_per_lane = V;
            pi->block = kSplitLanes;
            pi->grid = grid;
            pi->waves_per_row = P;
            pi->slice_windows = (int)((nw_max + P - 1) / P);
            pi->launches = 1;
            pi->nt_loads = nt ? 1 : 0;
            pi->workspace_bytes = ((p.M * P * 32 + 255) / 256) * 256;
            pi->model_bytes = model;
            return SM_OK;
        }
        if (!auto_plan) return SM_ERR_PLAN;
        plan = SM_PLAN_WIDE;  // a row's slices cannot all be resident: two passes
    }
    const int64_t model = (plan == SM_PLAN_WIDE ? 3 : 2) * p.M * p.N * es;
    const bool want_nt = o.nontemporal == 1 || (o.nontemporal == 0 && model >= kNtLoadBytes);

    if (plan == SM_PLAN_WIDE) {
        const int WPC = kChunk / E;
        const int64_t nchunks = (nw_max + WPC - 1) / WPC;
        int64_t cpw = o.chunks_per_wave > 0 ? o.chunks_per_wave : wide_cpw;
        if (cpw <= 0) {
            const int64_t target = (int64_t)dev.cus * 32;  // one full wave slot set
            cpw = std::max<int64_t>(1, (p.M * nchunks + target - 1) / target);
        }
        cpw = std::min<int64_t>(cpw, nchunks);
        if (cpw > INT32_MAX) return SM_ERR_PLAN;
        const int64_t wpr = (nchunks + cpw - 1) / cpw;
        if (p.M > INT64_MAX / wpr) return SM_ERR_PLAN;
        const int64_t waves = p.M * wpr;
        const int64_t grid = (waves + 3) / 4;
        if (grid * 256 > kMaxThreadsPerLaunch) return SM_ERR_PLAN;
        pi->plan = SM_PLAN_WIDE;
        pi->block = 256;
        pi->grid = grid;
        pi->chunks_per_wave = (int)cpw;
        pi->waves_per_row = wpr;
        pi->launches = 2;
        pi->nt_loads = want_nt ? 1 : 0;
        pi->workspace_bytes = ((waves * 8 + 255) / 256) * 256;
        pi->model_bytes = model;
        return SM_OK;
    }

    // One-pass plans: a row shape that holds the whole row.
    const int fixG = o.lanes_per_row, fixV = o.vecs_per_lane;
    int G = fixG, V = fixV;
    const bool auto_shape = !(fixG && fixV);
    auto prefetch_for = [&](int g, int v) {
        // Prefetching the next row paid off for rows held inside one wave, not
        // for rows spread over several waves (measured).
        int pf = (o.prefetch > 0) ? 1 : (o.prefetch < 0 ? 0 : (g <= 64 ? 1 : 0));
        return (pf && built_shape(g, v, 1)) ? 1 : 0;
    };
    int64_t slots = 0;  // workgroups resident at once
    if (auto_plan) {
        // Auto: a grid-stride loop avoids relaunching workgroups when the rows fit
        // in at most two rounds of resident workgroups; with more rows, one
        // workgroup per row group kept memory streaming better (524288 x 2048
        // BF16: 659 against 909 us).
        int gp = G, vp = V;
        if (auto_shape && !pick_shape(kShapes, nw_max, fixG, fixV, gp, vp)) return SM_ERR_PLAN;
        const int gpb = row_block(gp) / gp;
        const int occ = std::max(1, dev.occ_row(dev.ctx, p.dtype, gp, vp, prefetch_for(gp, vp)));
        slots = (int64_t)occ * dev.cus;
        if ((p.M + gpb - 1) / gpb <= 2 * slots) {
            plan = SM_PLAN_PERSISTENT;
            G = gp;
            V = vp;
        } else if (auto_shape && !pick_shape(kShapes, nw_max, fixG, fixV, G, V)) {
            return SM_ERR_PLAN;
        }
    } else if (auto_shape && !pick_shape(kShapes, nw_max, fixG, fixV, G, V)) {
        return SM_ERR_PLAN;
    }
    if (plan == SM_PLAN_RESIDENT && !fixG && !fixV && G == 128 && V == 2 &&
        p.dtype != SM_F32 && model >= kLongCallBytes) {
        G = 256;
        V = 1;
    }
    if (!built_shape(G, V, 0) || (int64_t)G * V < nw_max) return SM_ERR_PLAN;
    const int block = row_block(G);
    const int gpb = block / G;
    const int64_t groups = (p.M + gpb - 1) / gpb;
    const int64_t cap = kMaxThreadsPerLaunch / block;
    const int PF = plan == SM_PLAN_PERSISTENT ? prefetch_for(G, V) : 0;
    if (plan == SM_PLAN_PERSISTENT && slots == 0) {
        const int occ = std::max(1, dev.occ_row(dev.ctx, p.dtype, G, V, PF));
        slots = (int64_t)occ * dev.cus;
    }
    // Streaming loads exist for the resident multi-wave shapes.
    const int NT = (want_nt && !PF && G >= 128) ? 1 : 0;
    int64_t grid;
    if (o.grid > 0) {
        grid = o.grid;
    } else if (plan == SM_PLAN_PERSISTENT) {
        grid = slots;
    } else {
        grid = groups;
    }
    grid = std::max<int64_t>(1, std::min<int64_t>(std::min(grid, groups), cap));
    pi->plan = plan;
    pi->lanes_per_row = G;
    pi->vecs_per_lane = V;
    pi->prefetch = PF;
    pi->nt_loads = NT;
    pi->block = block;
    pi->grid = grid;
    pi->launches = 1;
    pi->model_bytes = model;
    return SM_OK;
}

// ------------------------------------------------------------ device cache
struct DevCache {
    int cus = 0;
    std::map<const void*, int> occ;
};
std::mutex g_mu;
std::map<int, DevCache> g_dev;

int occ_of(const void* fn, int block) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    std::lock_guard<std::mutex> lk(g_mu);
    DevCache& d = g_dev[dev];
    auto it = d.occ.find(fn);
    if (it != d.occ.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, block, 0) != hipSuccess || n < 1) n = 1;
    d.occ[fn] = n;
    return n;
}

int occ_row_live(void*, int dtype, int G, int V, int PF) {
    RowKernelFn fn = row_kernel(dtype, G, V, PF, 0);
    return fn ? occ_of(reinterpret_cast<const void*>(fn), row_block(G)) : 1;
}
int occ_wide_live(void*, int dtype) {
    return occ_of(reinterpret_cast<const void*>(wide_stats_kernel(dtype, 0)), 256);
}
// kind: 0 softmax forward, 1 softmax backward, 2 residual RMSNorm
int occ_split_live(void*, int dtype, int V, int kind) {
    const void* fn = kind == 1   ? reinterpret_cast<const void*>(bwd_split_kernel(dtype, V, 0))
                     : kind == 2 ? reinterpret_cast<const void*>(rms_split_kernel(dtype, V, 0))
                                 : reinterpret_cast<const void*>(split_kernel(dtype, V, 0));
    return fn ? occ_of(fn, kSplitLanes) : 1;
}
int occ_row_host(void*, int, int G, int, int) { return std::max(1, 2048 / row_block(G)); }
int occ_wide_host(void*, int) { return 8; }
int occ_split_host(void*, int, int, int) { return 8; }

int live_device(DeviceView* v) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        t_last_hip_error = (int)e;
        return SM_ERR_NO_DEVICE;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        DevCache& d = g_dev[dev];
        if (d.cus == 0) {
            int cus = 0;
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess || cus <= 0) {
                t_last_hip_error = (int)e;
                return SM_ERR_NO_DEVICE;
            }
            d.cus = cus;
        }
        v->cus = d.cus;
    }
    v->occ_row = occ_row_live;
    v->occ_wide = occ_wide_live;
    v->occ_split = occ_split_live;
    v->ctx = nullptr;
    return SM_OK;
}

sm_softmax_opts opts_or_default(const sm_softmax_opts* o) {
    sm_softmax_opts d{};
    return o ? *o : d;
}

// ------------------------------------------------------------ SPLIT synchronisation
// Per (device, stream) count of timed-out SPLIT waits: device memory zeroed once
// at creation and kept until the process ends.
std::mutex g_sync_mu;
std::map<std::pair<int, uintptr_t>, void*> g_sync;

void* split_sync(hipStream_t stream, bool create, hipError_t* err) {
    *err = hipSuccess;
    int dev = 0;
    if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lk(g_sync_mu);
    const auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(stream));
    auto it = g_sync.find(key);
    if (it != g_sync.end()) return it->second;
    if (!create) return nullptr;
    void* ptr = nullptr;
    if ((*err = hipMalloc(&ptr, 256)) != hipSuccess) return nullptr;
    if ((*err = hipMemset(ptr, 0, 256)) != hipSuccess) {
        (void)hipFree(ptr);
        return nullptr;
    }
    g_sync[key] = ptr;
    return ptr;
}

// Call ids that tag SPLIT slots: never 0, different for every call of the
// process, starting from a value that differs between processes.
uint32_t next_tag() {
    static std::atomic<uint32_t> tag{static_cast<uint32_t>(
        std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u) | 1u};
    uint32_t t = tag.fetch_add(1);
    while (t == 0) t = tag.fetch_add(1);
    return t;
}

// ------------------------------------------------------------ launches
// Launch `fn` with its arguments; with events, through hipExtLaunchKernel so
// that the events carry the dispatch's own start/end times.
template <typename... Args>
hipError_t launch_k(const void* fn, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0,
                    hipEvent_t e1, Args... args) {
    void* argv[] = {reinterpret_cast<void*>(&args)...};
    if (e0 || e1) return hipExtLaunchKernel(fn, grid, block, argv, 0, s, e0, e1, 0);
    return hipLaunchKernel(fn, grid, block, argv, 0, s);
}

// Whether a one-pass launch renumbers its workgroups XCD-contiguously: resident
// rows that own their workgroup (128 lanes and up) and share cache lines with
// their neighbours (a row stride that is not a whole number of 128-byte lines).
int xcd_order(const sm_plan_info& pi, bool rows_share_lines) {
    return (pi.plan == SM_PLAN_RESIDENT && pi.lanes_per_row > 64 && rows_share_lines) ? 1 : 0;
}

// sync: SPLIT failure counter to use, or nullptr for the stream's own (created on
// first use).
int launch(const Problem& p, const sm_plan_info& pi, void* ws, const sm_softmax_opts& o,
           hipStream_t stream, void* sync = nullptr) {
    const hipEvent_t ev0 = o.start_event, ev1 = o.stop_event;
    const int es = elem_bytes(p.dtype);
    const auto* in = reinterpret_cast<const unsigned char*>(p.in);
    auto* out = reinterpret_cast<unsigned char*>(p.out);
    const int64_t isb = p.in_stride * es, osb = p.out_stride * es;
    const int N = (int)p.N;
    hipError_t e;
    if (pi.plan == SM_PLAN_SPLIT) {
        if (!sync) sync = split_sync(stream, true, &e);
        if (!sync) return hip_fail(e);
        SplitKernelFn fn = split_kernel(p.dtype, pi.vecs_per_lane, pi.nt_loads);
        if (!fn) return SM_ERR_PLAN;
        const int spin = o.spin_limit > 0 ? o.spin_limit : kSplitSpinDefault;
        // out of place (validation admits only disjoint rows or exactly in place), a
        // slice whose wait runs out can re-read its whole input row
        const int recompute = p.in != p.out ? 1 : 0;
        e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(kSplitLanes),
                     stream, ev0, ev1, in, out, ws, sync, p.M, N, isb, osb, (int)pi.waves_per_row,
                     pi.slice_windows, next_tag(), spin, (int)pi.same_phase, recompute);
        return e == hipSuccess ? SM_OK : hip_fail(e);
    }
    if (pi.plan == SM_PLAN_WIDE) {
        auto* st = reinterpret_cast<float2*>(ws);
        const int cpw = pi.chunks_per_wave;
        const int64_t wpr = pi.waves_per_row;
        e = launch_k(reinterpret_cast<const void*>(wide_stats_kernel(p.dtype, pi.nt_loads)),
                     dim3((unsigned)pi.grid), dim3(256), stream, ev0, nullptr, in, st, p.M, N, isb,
                     cpw, wpr);
        if (e != hipSuccess) return hip_fail(e);
        e = launch_k(reinterpret_cast<const void*>(wide_norm_kernel(p.dtype, pi.nt_loads)),
                     dim3((unsigned)pi.grid), dim3(256), stream, nullptr, ev1, in, out,
                     (const float2*)st, p.M, N, isb, osb, cpw, wpr, (int)pi.same_phase);
        return e == hipSuccess ? SM_OK : hip_fail(e);
    }
    RowKernelFn fn =
        row_kernel(p.dtype, pi.lanes_per_row, pi.vecs_per_lane, pi.prefetch, pi.nt_loads);
    if (!fn) return SM_ERR_PLAN;
    // Resident rows of their own workgroup whose stride is not a whole number of
    // 128-byte lines share a line with the next row: XCD-contiguous order lets one
    // L2 merge both halves of it (cold, MI355X: 524288 x 2000 BF16 691 against 764
    // us, 131072 x 2000 172 against 194 us, 16384 x 4000 38.4 against 38.9 us); on
    // line-aligned rows (524288 x 2048: 649 against 636 us), persistent grids (8192
    // x 1000 FP16: 9.8 against 6.9 us) and rows that share a workgroup (whose
    // consecutive rows already meet in one L2) the hardware's order was as fast or
    // faster.
    const int xcd = xcd_order(pi, isb % 128 != 0 || osb % 128 != 0);
    e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(pi.block), stream,
                 ev0, ev1, in, out, p.M, N, isb, osb, (int)pi.same_phase, xcd);
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

// ------------------------------------------------------------ scratch memory
// WIDE and SPLIT scratch: one buffer per (device, stream), allocated on the first call
// that needs it and grown (at least doubled) when a call needs more, kept until the
// process ends. Calls on one stream run in order, so they can share it; calls on
// different streams never do. A stream-ordered allocation per call (hipMallocAsync or
// hipMallocFromPoolAsync with hipFreeAsync) put about 5 us of extra time on the stream
// per call on MI355X (cold BF16 64 x 131072 SPLIT: 19.5 against 14.5 us from event to
// event). A buffer replaced by a larger one is kept as well (earlier calls on the
// stream may still be running on it), so a stream holds at most about twice the
// largest scratch it needed. Under graph capture the scratch comes from
// hipMallocAsync instead (a graph memory node), freed in the same graph.
struct StreamScratch {
    void* buf = nullptr;
    size_t bytes = 0;
};
std::mutex g_scratch_stream_mu;
std::map<std::pair<int, uintptr_t>, StreamScratch> g_scratch_stream;
std::vector<void*> g_scratch_retired;

hipError_t stream_scratch(hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scratch_stream_mu);
    StreamScratch& st = g_scratch_stream[std::make_pair(dev, reinterpret_cast<uintptr_t>(stream))];
    if (st.bytes < bytes) {
        size_t nb = std::max<size_t>(std::max<size_t>(bytes, 2 * st.bytes), size_t(64) << 10);
        nb = (nb + 65535) / 65536 * 65536;
        void* p = nullptr;
        e = hipMalloc(&p, nb);
        if (e != hipSuccess) return e;
        if (st.buf) g_scratch_retired.push_back(st.buf);
        st.buf = p;
        st.bytes = nb;
    }
    *out = st.buf;
    return hipSuccess;
}

// Whether `stream` is being captured into a graph (the legacy null stream cannot be,
// and is not asked).
hipError_t stream_capturing(hipStream_t stream, bool* capturing) {
    *capturing = false;
    if (!stream) return hipSuccess;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &st);
    *capturing = e == hipSuccess && st == hipStreamCaptureStatusActive;
    return e;
}

// Run `go(ws)` with `bytes` of scratch: the stream's own buffer, or under graph capture
// a stream-ordered allocation released after the launches.
template <class Go>
int with_scratch(size_t bytes, bool capturing, hipStream_t stream, Go go) {
    void* tmp = nullptr;
    hipError_t e;
    if (!capturing) {
        e = stream_scratch(stream, bytes, &tmp);
        if (e != hipSuccess) return hip_fail(e);
        return go(tmp);
    }
    e = hipMallocAsync(&tmp, bytes, stream);
    if (e != hipSuccess) return hip_fail(e);
    int rc = go(tmp);
    e = hipFreeAsync(tmp, stream);
    if (rc == SM_OK && e != hipSuccess) rc = hip_fail(e);
    return rc;
}

int run(const Problem& p, const sm_softmax_opts* opts, void* ws, size_t ws_bytes,
        hipStream_t stream) {
    int rc = validate(p);
    if (rc != SM_OK || p.M == 0 || p.N == 0) return rc;
    DeviceView dv;
    rc = live_device(&dv);
    if (rc != SM_OK) return rc;
    sm_plan_info pi;
    const sm_softmax_opts o = opts_or_default(opts);
    bool capturing = false;
    hipError_t e = stream_capturing(stream, &capturing);
    if (e != hipSuccess) return hip_fail(e);
    rc = make_plan(p, o, dv, capturing, &pi);
    if (rc != SM_OK) return rc;
    if (pi.workspace_bytes == 0) return launch(p, pi, nullptr, o, stream);

    if (ws) {
        if (ws_bytes < (size_t)pi.workspace_bytes || (reinterpret_cast<uintptr_t>(ws) & 15))
            return SM_ERR_WORKSPACE;
        return launch(p, pi, ws, o, stream);
    }
    return with_scratch((size_t)pi.workspace_bytes, capturing, stream,
                        [&](void* tmp) { return launch(p, pi, tmp, o, stream); });
}

// ------------------------------------------------------------ allocation-free forward
// Scratch of sm_softmax_fwd_noalloc: one array per device, held until the process
// ends. Bytes [0, 256) hold that entry point's SPLIT failure counter (a SplitSync;
// device globals start zeroed when the code object loads), bytes [256, 256 +
// SM_NOALLOC_SCRATCH_BYTES) its WIDE or SPLIT workspace. Host code never passes
// `scratch` itself to a kernel (in host code the name is a host-side stand-in): it
// takes the device's address of it from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocSyncBytes = 256;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocSyncBytes + SM_NOALLOC_SCRATCH_BYTES];
namespace {

std::mutex g_scratch_mu;
std::map<int, unsigned char*> g_scratch;  // device -> address of its `scratch`

hipError_t scratch_address(unsigned char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<unsigned char*>(ptr);
    *out = static_cast<unsigned char*>(ptr);
    return hipSuccess;
}

int run_noalloc(const Problem& p, hipStream_t stream) {
    int rc = validate(p);
    if (rc != SM_OK || p.M == 0 || p.N == 0) return rc;
    DeviceView dv;
    rc = live_device(&dv);
    if (rc != SM_OK) return rc;
    bool capturing = false;
    hipError_t e = stream_capturing(stream, &capturing);
    if (e != hipSuccess) return hip_fail(e);
    unsigned char* base = nullptr;
    e = scratch_address(&base);
    if (e != hipSuccess) return hip_fail(e);
    // In place, a SPLIT slice whose wait ran out could only write NaN (its row's input
    // may already be overwritten), and this entry point has no counter the caller can
    // read: rows that AUTO would split take the two-pass WIDE plan instead, so the
    // result never depends on scheduling.
    const sm_softmax_opts o{};
    sm_plan_info pi;
    rc = make_plan(p, o, dv, capturing || p.in == p.out, &pi);
    if (rc != SM_OK) return rc;
    if ((uint64_t)pi.workspace_bytes > (uint64_t)SM_NOALLOC_SCRATCH_BYTES) return SM_ERR_WORKSPACE;
    return launch(p, pi, base + kNoAllocSyncBytes, o, stream, base);
}

// ------------------------------------------------------------ backward
struct BwdProblem {
    uintptr_t y, dy, dx;
    int64_t M, N, y_stride, dy_stride, dx_stride;
    int dtype;
};

int validate_bwd(const BwdProblem& p) {
    if (p.dtype != SM_F32 && p.dtype != SM_F16 && p.dtype != SM_BF16) return SM_ERR_DTYPE;
    if (p.M < 0 || p.N < 0) return SM_ERR_INVALID;
    if (p.M == 0 || p.N == 0) return SM_OK;
    if (!p.y || !p.dy || !p.dx) return SM_ERR_INVALID;
    // each (input, dx) pair obeys the forward rules: sizes, strides, alignment,
    // spans, and no overlap other than exactly in place
    int rc = validate(Problem{p.y, p.dx, p.M, p.N, p.y_stride, p.dx_stride, p.dtype});
    if (rc != SM_OK) return rc;
    return validate(Problem{p.dy, p.dx, p.M, p.N, p.dy_stride, p.dx_stride, p.dtype});
}

// Backward row shapes: y and dy both live in registers, so at most 4 vectors per lane.
constexpr RowShape kShapesBwd[] = {{16, 1},  {32, 1},  {64, 1},  {64, 2},   {128, 2},
                                   {256, 2}, {256, 4}, {512, 4}, {1024, 4}};
// Automatic backward plans launch one workgroup per row group (RESIDENT). With y
// and dy held in their stored encoding every backward shape runs at full
// occupancy, and the resident launch matched or beat the grid-stride loop on
// every measured shape (cold, MI355X): BF16 4096 x 4096 16.9 against 17.1 us,
// FP16 8192 x 4096 31.3 against 32.4 us, 8192 x 8192 59.7 against 63.7 us,
// BF16 524288 x 2048 1035 against 1359 us.

// One-pass backward rows stream y and dy past the MALL from this much traffic up:
// two inputs per output made the streaming loads pay much earlier than in the
// forward (cold, MI355X, dx identical: 65536 x 2048 BF16 (768 MiB) 110.6 against
// 127.2 us; 16384 x 4096 BF16 (384 MiB) 56.7 against 60.5; 4096 x 4096 BF16 (96
// MiB) 16.8 against 17.0; 2048 x 4096 BF16 (48 MiB) 9.85 against 10.0; at 24 MiB
// -1.8% to +1.2%).
constexpr int64_t kBwdNtLoadBytes = int64_t(32) << 20;

int occ_bwd_live(int dtype, int G, int V) {
    BwdRowKernelFn fn = bwd_row_kernel(dtype, G, V, 0);
    return fn ? occ_of(reinterpret_cast<const void*>(fn), row_block(G)) : 1;
}

int make_plan_bwd(const BwdProblem& p, const sm_softmax_opts& o, int cus, bool live,
                  bool no_split, sm_plan_info* pi) {
    *pi = sm_plan_info{};
    const int es = elem_bytes(p.dtype);
    const int E = 16 / es;
    const bool y_aligned = (p.y % 16 == 0) && (p.M == 1 || (p.y_stride * es) % 16 == 0);
    const int64_t nw_max = ((y_aligned ? 0 : E - 1) + p.N + E - 1) / E;
    auto phase = [&](uintptr_t a, int64_t sa) {
        return ((p.y - a) % 16 == 0) && (p.M == 1 || (((p.y_stride - sa) * es) % 16 == 0));
    };
    pi->same_phase = phase(p.dx, p.dx_stride);
    pi->dy_same_phase = phase(p.dy, p.dy_stride);
    if (o.nontemporal < -1 || o.nontemporal > 1) return SM_ERR_PLAN;
    int plan = o.plan;
    if (plan < SM_PLAN_AUTO || plan > SM_PLAN_SPLIT) return SM_ERR_PLAN;
    const bool auto_plan = plan == SM_PLAN_AUTO;
    if (auto_plan) plan = one_pass_rule(p.M, p.N, nw_max) ? SM_PLAN_RESIDENT : SM_PLAN_SPLIT;
    if (plan == SM_PLAN_SPLIT && no_split) {  // graph capture, as in the forward
        if (!auto_plan) return SM_ERR_PLAN;
        plan = SM_PLAN_WIDE;
    }
    if (plan == SM_PLAN_SPLIT) {
        auto occ_fn = live ? occ_split_live : occ_split_host;
        int64_t P = 0, grid = 0;
        int V = o.vecs_per_lane;
        if (V) {
            if (V != 1 && V != 2 && V != 4) return SM_ERR_PLAN;
            const int64_t slots = (int64_t)std::max(1, occ_fn(nullptr, p.dtype, V, 1)) * cus;
            if (!split_geometry(p.M, nw_max, V, slots, o.grid, P, grid)) V = 0;
        } else {
            V = split_auto_v(p.M, nw_max, 2, 4, 4, kSplitRoundSlices, cus, nullptr, p.dtype, 1, occ_fn,
                             P, grid);
            if (V && o.grid > 0) {
                const int64_t slots = (int64_t)std::max(1, occ_fn(nullptr, p.dtype, V, 1)) * cus;
                if (!split_geometry(p.M, nw_max, V, slots, o.grid, P, grid)) V = 0;
            }
        }
        if (V) {
            const int64_t model = 3 * p.M * p.N * es;
            const bool nt = o.nontemporal == 1 || (o.nontemporal == 0 && model >= kNtLoadBytes);
            pi->plan = SM_PLAN_SPLIT;
            pi->lanes_per_row = kSplitLanes;
            pi->vecs_per_lane = V;
            pi->block = kSplitLanes;
            pi->grid = grid;
            pi->waves_per_row = P;
            pi->slice_windows = (int)((nw_max + P - 1) / P);
            pi->launches = 1;
            pi->nt_loads = nt ? 1 : 0;
            pi->workspace_bytes = ((p.M * P * 32 + 255) / 256) * 256;
            pi->model_bytes = model;
            return SM_OK;
        }
        if (!auto_plan) return SM_ERR_PLAN;
        plan = SM_PLAN_WIDE;
    }
    if (plan == SM_PLAN_WIDE) {
        const int WPC = kChunk / E;
        const int64_t nchunks = (nw_max + WPC - 1) / WPC;
        int64_t cpw = o.chunks_per_wave;
        if (cpw <= 0) {
            const int64_t target = (int64_t)cus * 32;
            cpw = std::max<int64_t>(1, (p.M * nchunks + target - 1) / target);
        }
        cpw = std::min<int64_t>(cpw, nchunks);
        if (cpw > INT32_MAX) return SM_ERR_PLAN;
        const int64_t wpr = (nchunks + cpw - 1) / cpw;
        if (p.M > INT64_MAX / wpr) return SM_ERR_PLAN;
        const int64_t waves = p.M * wpr;
        const int64_t grid = (waves + 3) / 4;
        if (grid * 256 > kMaxThreadsPerLaunch) return SM_ERR_PLAN;
        pi->plan = SM_PLAN_WIDE;
        pi->block = 256;
        pi->grid = grid;
        pi->chunks_per_wave = (int)cpw;
        pi->waves_per_row = wpr;
        pi->launches = 2;
        pi->workspace_bytes = ((waves * 8 + 255) / 256) * 256;
        pi->model_bytes = 5 * p.M * p.N * es;
        return SM_OK;
    }
    int G = 0, V = 0;
    if (!pick_shape(kShapesBwd, nw_max, o.lanes_per_row, o.vecs_per_lane, G, V)) return SM_ERR_PLAN;
    if (!bwd_row_kernel(p.dtype, G, V, 0) || (int64_t)G * V < nw_max) return SM_ERR_PLAN;
    const int block = row_block(G);
    const int gpb = block / G;
    const int64_t groups = (p.M + gpb - 1) / gpb;
    const int occ = live ? std::max(1, occ_bwd_live(p.dtype, G, V)) : std::max(1, 2048 / block);
    const int64_t slots = (int64_t)occ * cus;
    const int64_t model = 3 * p.M * p.N * es;
    const bool want_nt = o.nontemporal == 1 || (o.nontemporal == 0 && model >= kBwdNtLoadBytes);
    int64_t grid = o.grid > 0 ? o.grid : (plan == SM_PLAN_PERSISTENT ? slots : groups);
    grid = std::max<int64_t>(1, std::min<int64_t>(std::min(grid, groups),
                                                  kMaxThreadsPerLaunch / block));
    pi->plan = plan;
    pi->lanes_per_row = G;
    pi->vecs_per_lane = V;
    pi->nt_loads = (want_nt && G >= 128) ? 1 : 0;
    pi->block = block;
    pi->grid = grid;
    pi->launches = 1;
    pi->model_bytes = model;
    return SM_OK;
}

int launch_bwd(const BwdProblem& p, const sm_plan_info& pi, void* ws, const sm_softmax_opts& o,
               hipStream_t stream) {
    const hipEvent_t ev0 = o.start_event, ev1 = o.stop_event;
    const int es = elem_bytes(p.dtype);
    const auto* y = reinterpret_cast<const unsigned char*>(p.y);
    const auto* dy = reinterpret_cast<const unsigned char*>(p.dy);
    auto* dx = reinterpret_cast<unsigned char*>(p.dx);
    const int64_t ysb = p.y_stride * es, dysb = p.dy_stride * es, dxsb = p.dx_stride * es;
    const int N = (int)p.N;
    hipError_t e;
    if (pi.plan == SM_PLAN_SPLIT) {
        void* sync = split_sync(stream, true, &e);
        if (!sync) return hip_fail(e);
        BwdSplitKernelFn fn = bwd_split_kernel(p.dtype, pi.vecs_per_lane, pi.nt_loads);
        if (!fn) return SM_ERR_PLAN;
        const int spin = o.spin_limit > 0 ? o.spin_limit : kSplitSpinDefault;
        const int recompute = (p.dx != p.y && p.dx != p.dy) ? 1 : 0;
        e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(kSplitLanes),
                     stream, ev0, ev1, y, dy, dx, ws, sync, p.M, N, ysb, dysb, dxsb,
                     (int)pi.waves_per_row, pi.slice_windows, next_tag(), spin,
                     (int)pi.dy_same_phase, (int)pi.same_phase, recompute);
        return e == hipSuccess ? SM_OK : hip_fail(e);
    }
    if (pi.plan == SM_PLAN_WIDE) {
        auto* part = reinterpret_cast<float2*>(ws);
        const int cpw = pi.chunks_per_wave;
        const int64_t wpr = pi.waves_per_row;
        e = launch_k(reinterpret_cast<const void*>(bwd_dot_kernel(p.dtype)), dim3((unsigned)pi.grid),
                     dim3(256), stream, ev0, nullptr, y, dy, part, p.M, N, ysb, dysb, cpw, wpr,
                     (int)pi.dy_same_phase);
        if (e != hipSuccess) return hip_fail(e);
        e = launch_k(reinterpret_cast<const void*>(bwd_apply_kernel(p.dtype)),
                     dim3((unsigned)pi.grid), dim3(256), stream, nullptr, ev1, y, dy, dx,
                     (const float2*)part, p.M, N, ysb, dysb, dxsb, cpw, wpr, (int)pi.dy_same_phase,
                     (int)pi.same_phase);
        return e == hipSuccess ? SM_OK : hip_fail(e);
    }
    BwdRowKernelFn fn = bwd_row_kernel(p.dtype, pi.lanes_per_row, pi.vecs_per_lane, pi.nt_loads);
    if (!fn) return SM_ERR_PLAN;
    // XCD-contiguous order as in the forward (262144 x 2000 BF16 526 against 596 us,
    // 65536 x 2000 114 against 122 us; 64-lane rows 65536 x 1000 FP16 65.2 against
    // 61.7 us: not for rows that share a workgroup)
    const int xcd = xcd_order(pi, ysb % 128 != 0 || dysb % 128 != 0 || dxsb % 128 != 0);
    e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(pi.block), stream,
                 ev0, ev1, y, dy, dx, p.M, N, ysb, dysb, dxsb, (int)pi.dy_same_phase,
                 (int)pi.same_phase, xcd);
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

int run_bwd(const BwdProblem& p, const sm_softmax_opts* opts, void* ws, size_t ws_bytes,
            hipStream_t stream) {
    int rc = validate_bwd(p);
    if (rc != SM_OK || p.M == 0 || p.N == 0) return rc;
    DeviceView dv;
    rc = live_device(&dv);
    if (rc != SM_OK) return rc;
    const sm_softmax_opts o = opts_or_default(opts);
    sm_plan_info pi;
    bool capturing = false;
    hipError_t e = stream_capturing(stream, &capturing);
    if (e != hipSuccess) return hip_fail(e);
    rc = make_plan_bwd(p, o, dv.cus, true, capturing, &pi);
    if (rc != SM_OK) return rc;
    if (pi.workspace_bytes == 0) return launch_bwd(p, pi, nullptr, o, stream);
    if (ws) {
        if (ws_bytes < (size_t)pi.workspace_bytes || (reinterpret_cast<uintptr_t>(ws) & 15))
            return SM_ERR_WORKSPACE;
        return launch_bwd(p, pi, ws, o, stream);
    }
    return with_scratch((size_t)pi.workspace_bytes, capturing, stream,
                        [&](void* tmp) { return launch_bwd(p, pi, tmp, o, stream); });
}

// ------------------------------------------------------------ residual RMSNorm
struct RmsProblem {
    uintptr_t x, r, w, y, s;  // r and s may be 0
    int64_t M, N, x_stride, r_stride, y_stride, s_stride;
    float eps;
    int dtype;
};

bool spans_meet(uintptr_t a, int64_t sa, uintptr_t b, int64_t sb) {
    return !(a + (uint64_t)sa <= b || b + (uint64_t)sb <= a);
}

int validate_rms(const RmsProblem& p) {
    if (p.dtype != SM_F32 && p.dtype != SM_F16 && p.dtype != SM_BF16) return SM_ERR_DTYPE;
    if (p.M < 0 || p.N < 0) return SM_ERR_INVALID;
    if (p.M == 0 || p.N == 0) return SM_OK;
    if (!p.x || !p.w || !p.y) return SM_ERR_INVALID;
    if (!(p.eps >= 0.f) || p.eps == __builtin_huge_valf()) return SM_ERR_INVALID;
    const int es = elem_bytes(p.dtype);
    if (p.w % es) return SM_ERR_INVALID;
    // every (input, output) pair obeys the softmax rules: sizes, strides, alignment,
    // spans, and no overlap other than exactly in place
    int rc = validate(Problem{p.x, p.y, p.M, p.N, p.x_stride, p.y_stride, p.dtype});
    if (rc != SM_OK) return rc;
    if (p.r) {
        rc = validate(Problem{p.r, p.y, p.M, p.N, p.r_stride, p.y_stride, p.dtype});
        if (rc != SM_OK) return rc;
    }
    const int64_t wspan = p.N * es;
    const int64_t yspan = span_bytes(p.M, p.N, p.y_stride, es);
    if (p.w > UINTPTR_MAX - (uint64_t)wspan) return SM_ERR_INVALID;
    if (spans_meet(p.w, wspan, p.y, yspan)) return SM_ERR_OVERLAP;  // every row reads w
    if (p.s) {
        rc = validate(Problem{p.x, p.s, p.M, p.N, p.x_stride, p.s_stride, p.dtype});
        if (rc != SM_OK) return rc;
        if (p.r) {
            rc = validate(Problem{p.r, p.s, p.M, p.N, p.r_stride, p.s_stride, p.dtype});
            if (rc != SM_OK) return rc;
        }
        const int64_t sspan = span_bytes(p.M, p.N, p.s_stride, es);
        if (spans_meet(p.s, sspan, p.y, yspan) || spans_meet(p.w, wspan, p.s, sspan))
            return SM_ERR_OVERLAP;
    }
    return SM_OK;
}

constexpr int64_t kRmsTwoLaunchSlices = 64;

// One-pass RMSNorm rows stream x and the residual past the MALL from the MALL's
// size of traffic up (cold, MI355X, y identical: 65536 x 2048 BF16 (768 MiB)
// 114.1 against 128.4 us; 16384 x 4096 FP16 (384 MiB) 59.8 against 60.1; 4096 x
// 4096 BF16 (96 MiB) 18.7 against 18.5; 24-48 MiB within 0.2%).
constexpr int64_t kRmsNtLoadBytes = int64_t(256) << 20;

int occ_rms_live(int dtype, int G, int V) {
    RmsRowKernelFn fn = rms_row_kernel(dtype, G, V, 0);
    return fn ? occ_of(reinterpret_cast<const void*>(fn), row_block(G)) : 1;
}

int make_plan_rms(const RmsProblem& p, const sm_softmax_opts& o, int cus, bool live,
                  bool no_split, sm_plan_info* pi) {
    *pi = sm_plan_info{};
    const int es = elem_bytes(p.dtype);
    const int E = 16 / es;
    const bool x_aligned = (p.x % 16 == 0) && (p.M == 1 || (p.x_stride * es) % 16 == 0);
    const int64_t nw_max = ((x_aligned ? 0 : E - 1) + p.N + E - 1) / E;
    auto phase = [&](uintptr_t a, int64_t sa) {
        return ((p.x - a) % 16 == 0) && (p.M == 1 || (((p.x_stride - sa) * es) % 16 == 0));
    };
    pi->same_phase = phase(p.y, p.y_stride);
    pi->dy_same_phase = p.r ? phase(p.r, p.r_stride) : 1;
    // compulsory HBM bytes: x, y (+ residual, residual_out) per element, w once
    const int streams = 2 + (p.r ? 1 : 0) + (p.s ? 1 : 0);
    const int64_t wbytes = p.N * es;
    if (o.nontemporal < -1 || o.nontemporal > 1) return SM_ERR_PLAN;
    int plan = o.plan;
    if (plan < SM_PLAN_AUTO || plan > SM_PLAN_SPLIT) return SM_ERR_PLAN;
    const bool auto_plan = plan == SM_PLAN_AUTO;
    if (auto_plan) plan = one_pass_rule(p.M, p.N, nw_max) ? SM_PLAN_RESIDENT : SM_PLAN_SPLIT;
    auto occ_fn = live ? occ_split_live : occ_split_host;
    if (plan == SM_PLAN_SPLIT || plan == SM_PLAN_WIDE) {
        int64_t P = 0, grid = 0;
        int V = o.vecs_per_lane;
        bool fused = false;
        if (plan == SM_PLAN_SPLIT && no_split) {
            // graph capture: the two launches (publish, then gather) never wait on
            // peers, so a replay's stale words are all rewritten before they are read
            if (!auto_plan) return SM_ERR_PLAN;
        } else if (plan == SM_PLAN_SPLIT) {
            if (V) {
                if (V != 1 && V != 2 && V != 4) return SM_ERR_PLAN;
                const int64_t slots = (int64_t)std::max(1, occ_fn(nullptr, p.dtype, V, 2)) * cus;
                fused = split_geometry(p.M, nw_max, V, slots, o.grid, P, grid);
            } else {
                V = split_auto_v(p.M, nw_max, 1, 4, 2, kRmsRoundSlices, cus, nullptr, p.dtype, 2, occ_fn,
                                 P, grid);
                fused = V != 0;
                // many slices per row and several rounds: two launches without waits
                // measured faster (width 1048576, 8 to 1024 rows: 6 to 15%)
                if (fused && auto_plan && p.M * P > grid && P > kRmsTwoLaunchSlices) fused = false;
                if (fused && o.grid > 0) {
                    const int64_t slots = (int64_t)std::max(1, occ_fn(nullptr, p.dtype, V, 2)) * cus;
                    fused = split_geometry(p.M, nw_max, V, slots, o.grid, P, grid);
                }
            }
            if (!fused && !auto_plan) return SM_ERR_PLAN;
        }
        if (!fused) {
            // two launches of the split kernel (publish, then gather and apply): no
            // workgroup waits, so slices need not be resident together
            if (!V) V = 4;
            if (V != 1 && V != 2 && V != 4) return SM_ERR_PLAN;
            const int64_t S = (int64_t)kSplitLanes * V;
            P = std::max<int64_t>(1, (nw_max + S - 1) / S);
            if (P > INT32_MAX || p.M > INT64_MAX / P) return SM_ERR_PLAN;
            const int64_t slots = (int64_t)std::max(1, occ_fn(nullptr, p.dtype, V, 2)) * cus;
            grid = o.grid > 0 ? o.grid : std::max<int64_t>(1, slots);
            grid = std::min<int64_t>(grid, p.M * P);
            if (grid * kSplitLanes > kMaxThreadsPerLaunch) return SM_ERR_PLAN;
        }
        const int64_t model = (fused ? streams : streams + 1 + (p.r ? 1 : 0)) * p.M * p.N * es + wbytes;
        pi->plan = fused ? SM_PLAN_SPLIT : SM_PLAN_WIDE;
        pi->lanes_per_row = kSplitLanes;
        pi->vecs_per_lane = V;
        pi->block = kSplitLanes;
        pi->grid = grid;
        pi->waves_per_row = P;
        pi->slice_windows = (int)((nw_max + P - 1) / P);
        pi->launches = fused ? 1 : 2;
        pi->nt_loads = (o.nontemporal == 1 || (o.nontemporal == 0 && model >= kNtLoadBytes)) ? 1 : 0;
        pi->workspace_bytes = ((p.M * P * 32 + 255) / 256) * 256;
        pi->model_bytes = model;
        return SM_OK;
    }
    int G = 0, V = 0;
    if (!pick_shape(kShapesBwd, nw_max, o.lanes_per_row, o.vecs_per_lane, G, V)) return SM_ERR_PLAN;
    if (!rms_row_kernel(p.dtype, G, V, 0) || (int64_t)G * V < nw_max) return SM_ERR_PLAN;
    const int block = row_block(G);
    const int gpb = block / G;
    const int64_t groups = (p.M + gpb - 1) / gpb;
    const int occ = live ? std::max(1, occ_rms_live(p.dtype, G, V)) : std::max(1, 2048 / block);
    const int64_t slots = (int64_t)occ * cus;
    if (auto_plan && groups <= 2 * slots) plan = SM_PLAN_PERSISTENT;
    int64_t grid = o.grid > 0 ? o.grid : (plan == SM_PLAN_PERSISTENT ? slots : groups);
    grid = std::max<int64_t>(1, std::min<int64_t>(std::min(grid, groups),
                                                  kMaxThreadsPerLaunch / block));
    const int64_t model = streams * p.M * p.N * es + wbytes;
    pi->plan = plan;
    pi->lanes_per_row = G;
    pi->vecs_per_lane = V;
    pi->nt_loads = ((o.nontemporal == 1 || (o.nontemporal == 0 && model >= kRmsNtLoadBytes)) && G >= 128) ? 1 : 0;
    pi->block = block;
    pi->grid = grid;
    pi->launches = 1;
    pi->model_bytes = model;
    return SM_OK;
}

int launch_rms(const RmsProblem& p, const sm_plan_info& pi, void* ws, const sm_softmax_opts& o,
               hipStream_t stream) {
    const hipEvent_t ev0 = o.start_event, ev1 = o.stop_event;
    const int es = elem_bytes(p.dtype);
    const auto* x = reinterpret_cast<const unsigned char*>(p.x);
    const auto* r = p.r ? reinterpret_cast<const unsigned char*>(p.r) : x;  // never read without flag
    const auto* w = reinterpret_cast<const unsigned char*>(p.w);
    auto* y = reinterpret_cast<unsigned char*>(p.y);
    auto* sp = p.s ? reinterpret_cast<unsigned char*>(p.s) : y;  // never written without flag
    const int64_t xsb = p.x_stride * es, ysb = p.y_stride * es;
    const int64_t rsb = p.r ? p.r_stride * es : xsb, ssb = p.s ? p.s_stride * es : 0;
    auto phase = [&](uintptr_t a, int64_t sa) {
        return ((p.x - a) % 16 == 0) && (p.M == 1 || (((p.x_stride - sa) * es) % 16 == 0));
    };
    int flags = 0;
    if (p.r) flags |= kRmsResidual | (pi.dy_same_phase ? kRmsResPhase : 0);
    if (pi.same_phase) flags |= kRmsOutPhase;
    if (p.s) flags |= kRmsSumOut | (phase(p.s, p.s_stride) ? kRmsSumPhase : 0);
    const int N = (int)p.N;
    hipError_t e;
    if (pi.plan == SM_PLAN_SPLIT || pi.plan == SM_PLAN_WIDE) {
        // only the one-launch form waits on peers and may count a failure
        void* sync = nullptr;
        if (pi.plan == SM_PLAN_SPLIT) {
            sync = split_sync(stream, true, &e);
            if (!sync) return hip_fail(e);
        }
        const bool aliased = p.y == p.x || (p.r && p.y == p.r) ||
                             (p.s && (p.s == p.x || (p.r && p.s == p.r)));
        if (!aliased) flags |= kRmsRecompute;
        RmsSplitKernelFn fn = rms_split_kernel(p.dtype, pi.vecs_per_lane, pi.nt_loads);
        if (!fn) return SM_ERR_PLAN;
        const int spin = o.spin_limit > 0 ? o.spin_limit : kSplitSpinDefault;
        const uint32_t tag = next_tag();
        const int P = (int)pi.waves_per_row;
        if (pi.plan == SM_PLAN_SPLIT) {
            e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(kSplitLanes),
                         stream, ev0, ev1, x, r, w, y, sp, ws, sync, p.M, N, xsb, rsb, ysb, ssb, P,
                         pi.slice_windows, tag, spin, p.eps, flags, 0);
            return e == hipSuccess ? SM_OK : hip_fail(e);
        }
        e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(kSplitLanes),
                     stream, ev0, nullptr, x, r, w, y, sp, ws, sync, p.M, N, xsb, rsb, ysb, ssb, P,
                     pi.slice_windows, tag, spin, p.eps, flags, 1);
        if (e != hipSuccess) return hip_fail(e);
        e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(kSplitLanes),
                     stream, nullptr, ev1, x, r, w, y, sp, ws, sync, p.M, N, xsb, rsb, ysb, ssb, P,
                     pi.slice_windows, tag, spin, p.eps, flags, 2);
        return e == hipSuccess ? SM_OK : hip_fail(e);
    }
    RmsRowKernelFn fn = rms_row_kernel(p.dtype, pi.lanes_per_row, pi.vecs_per_lane, pi.nt_loads);
    if (!fn) return SM_ERR_PLAN;
    // XCD-contiguous order for resident rows that share cache lines, as in softmax
    // (262144 x 2000 BF16 532 against 597-625 us; 65536 x 2000 118 against 123 us)
    if (xcd_order(pi, xsb % 128 != 0 || ysb % 128 != 0 || (p.r && rsb % 128 != 0) ||
                          (p.s && ssb % 128 != 0)))
        flags |= kRmsXcdOrder;
    e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)pi.grid), dim3(pi.block), stream,
                 ev0, ev1, x, r, w, y, sp, p.M, N, xsb, rsb, ysb, ssb, p.eps, flags);
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

int run_rms(const RmsProblem& p, const sm_softmax_opts* opts, void* ws, size_t ws_bytes,
            hipStream_t stream) {
    int rc = validate_rms(p);
    if (rc != SM_OK || p.M == 0 || p.N == 0) return rc;
    DeviceView dv;
    rc = live_device(&dv);
    if (rc != SM_OK) return rc;
    const sm_softmax_opts o = opts_or_default(opts);
    sm_plan_info pi;
    bool capturing = false;
    hipError_t e = stream_capturing(stream, &capturing);
    if (e != hipSuccess) return hip_fail(e);
    rc = make_plan_rms(p, o, dv.cus, true, capturing, &pi);
    if (rc != SM_OK) return rc;
    if (pi.workspace_bytes == 0) return launch_rms(p, pi, nullptr, o, stream);
    if (ws) {
        if (ws_bytes < (size_t)pi.workspace_bytes || (reinterpret_cast<uintptr_t>(ws) & 15))
            return SM_ERR_WORKSPACE;
        return launch_rms(p, pi, ws, o, stream);
    }
    return with_scratch((size_t)pi.workspace_bytes, capturing, stream,
                        [&](void* tmp) { return launch_rms(p, pi, tmp, o, stream); });
}

// ------------------------------------------------------------ fused attention
constexpr int64_t kAttnMaxRowStride = int64_t(1) << 24;  // elements

struct AttnProblem {
    uintptr_t q, k, v, o, lse;  // lse may be 0
    int64_t BH, Sq, Sk, d;
    int64_t q_rs, q_hs, k_rs, k_hs, v_rs, v_hs, o_rs, o_hs;  // elements
    float scale;
    int causal, dtype;
};

// Byte span of a [BH][S][d] tensor with the given strides (elements), or -1.
int64_t span3(int64_t BH, int64_t S, int64_t d, int64_t rs, int64_t hs, int es) {
    if (BH <= 0 || S <= 0) return 0;
    const int64_t last = (BH - 1) * hs + (S - 1) * rs + d;
    if (last <= 0 || last > INT64_MAX / es) return -1;
    return last * es;
}

int validate_attn(const AttnProblem& p) {
    if (p.dtype != SM_F16 && p.dtype != SM_BF16) return SM_ERR_DTYPE;
    if (p.BH < 0 || p.Sq < 0 || p.Sk < 0) return SM_ERR_INVALID;
    if (p.d != 64 && p.d != 128) return SM_ERR_INVALID;
    if (!(p.scale == p.scale) || __builtin_isinf(p.scale)) return SM_ERR_INVALID;
    if (p.BH == 0 || p.Sq == 0) return SM_OK;
    if (p.Sq > INT32_MAX || p.Sk > INT32_MAX) return SM_ERR_INVALID;
    const int es = 2;
    if (!p.q || !p.o || (p.Sk > 0 && (!p.k || !p.v))) return SM_ERR_INVALID;
    // 16-byte rows: base, row and head strides multiples of 8 elements
    // row strides below 2^24 elements: a K/V tile is addressed with 32-bit offsets
    auto aligned = [&](uintptr_t ptr, int64_t rs, int64_t hs) {
        return ptr % 16 == 0 && rs % 8 == 0 && hs % 8 == 0 && rs >= p.d && rs <= kAttnMaxRowStride &&
               hs >= 0;
    };
    if (!aligned(p.q, p.q_rs, p.q_hs) || !aligned(p.o, p.o_rs, p.o_hs)) return SM_ERR_INVALID;
    if (p.Sk > 0 && (!aligned(p.k, p.k_rs, p.k_hs) || !aligned(p.v, p.v_rs, p.v_hs)))
        return SM_ERR_INVALID;
    // output rows of different heads must not share elements
    if (p.BH > 1 && p.o_hs < (p.Sq - 1) * p.o_rs + p.d) return SM_ERR_INVALID;
    if (p.lse && p.lse % 4) return SM_ERR_INVALID;
    const int64_t so = span3(p.BH, p.Sq, p.d, p.o_rs, p.o_hs, es);
    const int64_t sq = span3(p.BH, p.Sq, p.d, p.q_rs, p.q_hs, es);
    const int64_t sk = span3(p.BH, p.Sk, p.d, p.k_rs, p.k_hs, es);
    const int64_t sv = span3(p.BH, p.Sk, p.d, p.v_rs, p.v_hs, es);
    if (so < 0 || sq < 0 || sk < 0 || sv < 0) return SM_ERR_INVALID;
    if (p.BH > INT64_MAX / p.Sq) return SM_ERR_INVALID;
    const int64_t sl = p.lse ? p.BH * p.Sq * 4 : 0;
    // the output is written while the inputs are still being read: no overlap at all
    if (spans_meet(p.o, so, p.q, sq) || (sk && spans_meet(p.o, so, p.k, sk)) ||
        (sv && spans_meet(p.o, so, p.v, sv)))
        return SM_ERR_OVERLAP;
    if (p.lse && (spans_meet(p.lse, sl, p.o, so) || spans_meet(p.lse, sl, p.q, sq) ||
                  (sk && spans_meet(p.lse, sl, p.k, sk)) || (sv && spans_meet(p.lse, sl, p.v, sv))))
        return SM_ERR_OVERLAP;
    const int64_t qblocks = (p.Sq + kAttnBM - 1) / kAttnBM;
    if (p.BH > INT32_MAX / qblocks) return SM_ERR_INVALID;
    return SM_OK;
}

int run_attn(const AttnProblem& p, const sm_softmax_opts* opts, hipStream_t stream) {
    int rc = validate_attn(p);
    if (rc != SM_OK || p.BH == 0 || p.Sq == 0) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        t_last_hip_error = (int)e;
        return SM_ERR_NO_DEVICE;
    }
    const sm_softmax_opts o = opts_or_default(opts);
    AttnKernelFn fn = attention_kernel(p.dtype, (int)p.d, p.causal ? 1 : 0);
    if (!fn) return SM_ERR_PLAN;
    AttnArgs a;
    a.q = reinterpret_cast<const unsigned char*>(p.q);
    a.k = reinterpret_cast<const unsigned char*>(p.k ? p.k : p.q);
    a.v = reinterpret_cast<const unsigned char*>(p.v ? p.v : p.q);
    a.o = reinterpret_cast<unsigned char*>(p.o);
    a.lse = reinterpret_cast<float*>(p.lse);
    a.q_rs = p.q_rs * 2;
    a.q_hs = p.q_hs * 2;
    a.k_rs = p.k_rs * 2;
    a.k_hs = p.k_hs * 2;
    a.v_rs = p.v_rs * 2;
    a.v_hs = p.v_hs * 2;
    a.o_rs = p.o_rs * 2;
    a.o_hs = p.o_hs * 2;
    a.Sq = (int)p.Sq;
    a.Sk = (int)p.Sk;
    a.qblocks = (int)((p.Sq + kAttnBM - 1) / kAttnBM);
    // causal: q-blocks i and qblocks-1-i form one item (equal work per item)
    a.items = p.causal ? (a.qblocks + 1) / 2 : a.qblocks;
    a.scale_log2 = p.scale * 1.44269504088896340736f;
    const int64_t grid = p.BH * a.items;
    e = launch_k(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(kAttnThreads), stream,
                 o.start_event, o.stop_event, a);
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

}  // namespace
}  // namespace smx

using namespace smx;

extern "C" {

int sm_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                     int64_t Sq, int64_t Sk, int64_t d, int64_t q_row_stride,
                     int64_t q_head_stride, int64_t k_row_stride, int64_t k_head_stride,
                     int64_t v_row_stride, int64_t v_head_stride, int64_t o_row_stride,
                     int64_t o_head_stride, float scale, int causal, int dtype, hipStream_t stream) {
    return sm_attention_fwd_ex(q, k, v, o, lse, BH, Sq, Sk, d, q_row_stride, q_head_stride,
                               k_row_stride, k_head_stride, v_row_stride, v_head_stride,
                               o_row_stride, o_head_stride, scale, causal, dtype, nullptr, stream);
}

int sm_attention_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t BH, int64_t Sq, int64_t Sk, int64_t d, int64_t q_row_stride,
                        int64_t q_head_stride, int64_t k_row_stride, int64_t k_head_stride,
                        int64_t v_row_stride, int64_t v_head_stride, int64_t o_row_stride,
                        int64_t o_head_stride, float scale, int causal, int dtype,
                        const sm_softmax_opts* opts, hipStream_t stream) {
    const AttnProblem p{reinterpret_cast<uintptr_t>(q),   reinterpret_cast<uintptr_t>(k),
                        reinterpret_cast<uintptr_t>(v),   reinterpret_cast<uintptr_t>(o),
                        reinterpret_cast<uintptr_t>(lse), BH, Sq, Sk, d, q_row_stride,
                        q_head_stride, k_row_stride, k_head_stride, v_row_stride, v_head_stride,
                        o_row_stride, o_head_stride, scale, causal, dtype};
    return run_attn(p, opts, stream);
}

int sm_rmsnorm_fwd(const void* x, const void* residual, const void* weight, void* y,
                   void* residual_out, int64_t M, int64_t N, int64_t x_stride, int64_t res_stride,
                   int64_t y_stride, int64_t res_out_stride, float eps, int dtype,
                   hipStream_t stream) {
    return sm_rmsnorm_fwd_ex(x, residual, weight, y, residual_out, M, N, x_stride, res_stride,
                             y_stride, res_out_stride, eps, dtype, nullptr, nullptr, 0, stream);
}

int sm_rmsnorm_fwd_ex(const void* x, const void* residual, const void* weight, void* y,
                      void* residual_out, int64_t M, int64_t N, int64_t x_stride,
                      int64_t res_stride, int64_t y_stride, int64_t res_out_stride, float eps,
                      int dtype, const sm_softmax_opts* opts, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    const RmsProblem p{reinterpret_cast<uintptr_t>(x),  reinterpret_cast<uintptr_t>(residual),
                       reinterpret_cast<uintptr_t>(weight), reinterpret_cast<uintptr_t>(y),
                       reinterpret_cast<uintptr_t>(residual_out), M, N, x_stride, res_stride,
                       y_stride, res_out_stride, eps, dtype};
    return run_rms(p, opts, workspace, workspace_bytes, stream);
}

int sm_rmsnorm_plan_query(const void* x, const void* residual, const void* weight, const void* y,
                          const void* residual_out, int64_t M, int64_t N, int64_t x_stride,
                          int64_t res_stride, int64_t y_stride, int64_t res_out_stride, float eps,
                          int dtype, const sm_softmax_opts* opts, int num_cus,
                          sm_plan_info* info) {
    if (!info) return SM_ERR_INVALID;
    const RmsProblem p{reinterpret_cast<uintptr_t>(x),  reinterpret_cast<uintptr_t>(residual),
                       reinterpret_cast<uintptr_t>(weight), reinterpret_cast<uintptr_t>(y),
                       reinterpret_cast<uintptr_t>(residual_out), M, N, x_stride, res_stride,
                       y_stride, res_out_stride, eps, dtype};
    int rc = validate_rms(p);
    if (rc != SM_OK) return rc;
    if (M == 0 || N == 0) {
        *info = sm_plan_info{};
        return SM_OK;
    }
    int cus = num_cus;
    if (cus <= 0) {
        DeviceView dv;
        rc = live_device(&dv);
        if (rc != SM_OK) return rc;
        cus = dv.cus;
    }
    return make_plan_rms(p, opts_or_default(opts), cus, num_cus <= 0, false, info);
}

int sm_softmax_fwd(const void* in, void* out, int64_t M, int64_t N, int64_t in_stride,
                   int64_t out_stride, int dtype, hipStream_t stream) {
    const Problem p{reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out), M, N,
                    in_stride, out_stride, dtype};
    return run(p, nullptr, nullptr, 0, stream);
}

int sm_softmax_fwd_ex(const void* in, void* out, int64_t M, int64_t N, int64_t in_stride,
                      int64_t out_stride, int dtype, const sm_softmax_opts* opts, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    const Problem p{reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out), M, N,
                    in_stride, out_stride, dtype};
    return run(p, opts, workspace, workspace_bytes, stream);
}

int sm_softmax_fwd_noalloc(const void* in, void* out, int64_t M, int64_t N, int64_t in_stride,
                           int64_t out_stride, int dtype, hipStream_t stream) {
    const Problem p{reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out), M, N,
                    in_stride, out_stride, dtype};
    return run_noalloc(p, stream);
}

int sm_softmax_plan_query(const void* in, const void* out, int64_t M, int64_t N, int64_t in_stride,
                          int64_t out_stride, int dtype, const sm_softmax_opts* opts, int num_cus,
                          sm_plan_info* info) {
    if (!info) return SM_ERR_INVALID;
    const Problem p{reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out), M, N,
                    in_stride, out_stride, dtype};
    int rc = validate(p);
    if (rc != SM_OK) return rc;
    if (M == 0 || N == 0) {
        *info = sm_plan_info{};
        return SM_OK;
    }
    DeviceView dv;
    if (num_cus > 0) {
        dv.cus = num_cus;
        dv.occ_row = occ_row_host;
        dv.occ_wide = occ_wide_host;
        dv.occ_split = occ_split_host;
        dv.ctx = nullptr;
    } else {
        rc = live_device(&dv);
        if (rc != SM_OK) return rc;
    }
    return make_plan(p, opts_or_default(opts), dv, false, info);
}

int sm_softmax_bwd(const void* y, const void* dy, void* dx, int64_t M, int64_t N,
                   int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                   hipStream_t stream) {
    const BwdProblem p{reinterpret_cast<uintptr_t>(y), reinterpret_cast<uintptr_t>(dy),
                       reinterpret_cast<uintptr_t>(dx), M, N, y_stride, dy_stride, dx_stride, dtype};
    return run_bwd(p, nullptr, nullptr, 0, stream);
}

int sm_softmax_bwd_ex(const void* y, const void* dy, void* dx, int64_t M, int64_t N,
                      int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                      const sm_softmax_opts* opts, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    const BwdProblem p{reinterpret_cast<uintptr_t>(y), reinterpret_cast<uintptr_t>(dy),
                       reinterpret_cast<uintptr_t>(dx), M, N, y_stride, dy_stride, dx_stride, dtype};
    return run_bwd(p, opts, workspace, workspace_bytes, stream);
}

int sm_softmax_bwd_plan_query(const void* y, const void* dy, const void* dx, int64_t M, int64_t N,
                              int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                              const sm_softmax_opts* opts, int num_cus, sm_plan_info* info) {
    if (!info) return SM_ERR_INVALID;
    const BwdProblem p{reinterpret_cast<uintptr_t>(y), reinterpret_cast<uintptr_t>(dy),
                       reinterpret_cast<uintptr_t>(dx), M, N, y_stride, dy_stride, dx_stride, dtype};
    int rc = validate_bwd(p);
    if (rc != SM_OK) return rc;
    if (M == 0 || N == 0) {
        *info = sm_plan_info{};
        return SM_OK;
    }
    int cus = num_cus;
    if (cus <= 0) {
        DeviceView dv;
        rc = live_device(&dv);
        if (rc != SM_OK) return rc;
        cus = dv.cus;
    }
    return make_plan_bwd(p, opts_or_default(opts), cus, num_cus <= 0, false, info);
}

const char* sm_softmax_strerror(int status) {
    switch (status) {
    case SM_OK: return "success";
    case SM_ERR_INVALID: return "invalid argument (size, stride, pointer or alignment)";
    case SM_ERR_DTYPE: return "unknown dtype";
    case SM_ERR_OVERLAP: return "output overlaps input other than exactly in place";
    case SM_ERR_HIP: return "HIP runtime error";
    case SM_ERR_NO_DEVICE: return "no usable HIP device";
    case SM_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
    case SM_ERR_PLAN: return "plan or row shape cannot cover this problem";
    default: return "unknown status";
    }
}

int sm_softmax_version(void) { return SM_SOFTMAX_VERSION; }

int sm_softmax_last_hip_error(void) { return t_last_hip_error; }

int sm_softmax_sync_failures(hipStream_t stream, unsigned int* count) {
    if (!count) return SM_ERR_INVALID;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e);
    void* sync = split_sync(stream, false, &e);
    if (e != hipSuccess) return hip_fail(e);
    *count = 0;
    if (!sync) return SM_OK;
    uint32_t v = 0;
    e = hipMemcpy(&v, sync, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    *count = v;
    return SM_OK;
}

int sm_bench_copy(const void* src, void* dst, size_t bytes, int grid, int store_scope,
                  hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event) {
    if (!src || !dst || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15) || (store_scope != 0 && store_scope != 1))
        return SM_ERR_INVALID;
    if (bytes == 0) return SM_OK;
    if (grid <= 0) {
        DeviceView dv;
        int rc = live_device(&dv);
        if (rc != SM_OK) return rc;
        grid = 8 * dv.cus;
    }
    const void* fn = store_scope ? reinterpret_cast<const void*>(&k_copy16<true>)
                                 : reinterpret_cast<const void*>(&k_copy16<false>);
    hipError_t e = launch_k(fn, dim3(grid), dim3(256), stream,
                            start_event, stop_event, reinterpret_cast<const uint4*>(src),
                            reinterpret_cast<uint4*>(dst), (int64_t)(bytes / 16));
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

int sm_bench_flush(const void* buf, size_t bytes, hipStream_t stream) {
    if (!buf || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15)) return SM_ERR_INVALID;
    if (bytes == 0) return SM_OK;
    DeviceView dv;
    int rc = live_device(&dv);
    if (rc != SM_OK) return rc;
    hipLaunchKernelGGL(k_sweep_read16, dim3(8 * dv.cus), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(buf), (int64_t)(bytes / 16));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SM_OK : hip_fail(e);
}

}  // extern "C"
