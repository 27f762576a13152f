// sm_split.hpp -- one-launch softmax of wide rows split across workgroups.
//
// A row of N elements is cut into P slices of at most 256 * V 16-byte windows
// (spread evenly: S = ceil(windows / P) each); one workgroup of 256 lanes (4
// waves) holds a slice in registers. Each workgroup
// computes its slice's (max, sum of exp(x - max)), publishes the pair, waits
// until the row's other P - 1 slices have published theirs, merges the P pairs
// in a fixed order (so every slice of the row derives bitwise the same row
// statistics) and writes its slice of the output from registers. This is the
// split plan of "Measured optimization case studies", section "Wide rows: loop
// in one program, or split across programs", with the merge of partial states
// done by the row's own workgroups instead of a second launch: every element is
// read once and written once (2 * M * N * elem bytes, against 3 * M * N * elem
// for the two-pass plan).
//
// Co-residency. Workgroup b takes items b, b + grid, ... (item = row * P +
// slice), so a row's P slices are always P consecutive workgroups of one round.
// The grid is a multiple of P and at most half of the occupancy-derived
// capacity, so on a device that is not otherwise full every workgroup is
// resident at once and every wait ends; other kernels that hold compute units
// only delay the start of some workgroups until they finish. (A start ticket
// drawn from one atomic counter would make progress independent of dispatch
// altogether, but every workgroup hitting one address serialised them: 4 to
// 10 us per call on MI355X, against 1.5 us for the whole exchange.)
//
// Publication without fences. A slot holds up to three 64-bit words, each the
// call's tag (high half) beside one FP32 value (low half): max, sum_hi, sum_lo.
// Each word is written with one relaxed device-scope atomic store and read with
// relaxed device-scope atomic loads; a reader polls the words until each carries
// the tag, and each value comes from that same single-copy-atomic load. No L2
// write-back or invalidate is needed, and no slot is ever cleared: a stale word
// carries another call's tag. Every wait is bounded (spin_limit polls per
// workgroup), so a kernel always drains. A workgroup that runs out counts the
// failure and, when the output does not alias the input (`recompute`), derives
// the row's statistics itself from the whole input row -- the same definition, in
// another summation order -- so the result does not depend on scheduling; in place,
// where the row's other slices may already have overwritten their input, it writes
// NaN over its slice instead.
#pragma once

#include "sm_bwd.hpp"
#include "sm_kernels.hpp"

namespace smx {

struct alignas(32) SplitSlot {
    uint64_t w[4];  // tagged words: max, sum_hi, sum_lo (unused words stay unwritten)
};

// Per-stream status word (library-owned device memory, zero at creation): a
// count of timed-out waits.
struct SplitSync {
    uint32_t failures;
};

constexpr int kSplitBlock = 256;

__device__ __forceinline__ void word_publish(uint64_t* w, float v, uint32_t tag) {
    const uint64_t x = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(w, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll K consecutive tagged words until all carry `tag` (the K loads are issued
// together, so a slot costs one round trip when it is ready), spending at most
// `budget` polls (shared by all the waits of a lane). Returns false when the
// budget runs out.
template <int K>
__device__ __forceinline__ bool words_wait(const uint64_t* w, uint32_t tag, int& budget,
                                           float (&v)[K]) {
    uint64_t x[K];
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] = __hip_atomic_load(w + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < K; ++k) all = all && (uint32_t)(x[k] >> 32) == tag;
        if (all) break;
        if (--budget < 0) return false;
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if ((uint32_t)(x[k] >> 32) != tag)
                x[k] = __hip_atomic_load(w + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = __uint_as_float((uint32_t)x[k]);
    return true;
}

// Wave 0 gathers the P pairs of a row (lane j merges slots j, j + 64, ... in
// order, then the wave's merge tree) and leaves (m, s_hi, s_lo, ok) in LDS.
template <int DT>
__device__ __forceinline__ void split_gather(const SplitSlot* row_slots, int P, uint32_t tag,
                                            int spin_limit, float* lds_stat) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    int budget = spin_limit;
    bool ok = true;
    float m = kNegInf;
    CSum s;
    for (int j = lane; j < P; j += 64) {
        constexpr int K = (DT == kF32) ? 3 : 2;  // max, sum_hi (, sum_lo)
        float v[K];
        if (!words_wait<K>(row_slots[j].w, tag, budget, v)) {
            ok = false;
            break;
        }
        if constexpr (DT == kF32) {
            CSum o;
            o.hi = v[1];
            o.lo = v[2];
            merge_acc(m, s, v[0], o);
        } else {
            merge_fast(m, s.hi, v[0], v[1]);
        }
    }
    if constexpr (DT == kF32) {
        group_merge_acc<64>(m, s);
    } else {
        group_merge_fast<64>(m, s.hi);
    }
    const bool all_ok = __ballot(!ok) == 0;
    if (lane == 0) {
        lds_stat[0] = m;
        lds_stat[1] = s.hi;
        lds_stat[2] = s.lo;
        lds_stat[3] = all_ok ? 1.f : 0.f;
    }
}

// Fallback after a wait ran out: the whole workgroup walks the entire input row
// (window grid as in the slice loads, 256 windows per step) twice -- the row
// maximum, then the sum of exp(x - max) with the same exponential as the slices --
// and returns (m, s_hi, s_lo) on every lane.
template <int DT, bool NT>
__device__ __noinline__ void split_row_stats(const RowGeom<DT> g, int N, float* lds_a,
                                             float* lds_b, float* lds_c, float& m, float& s_hi,
                                             float& s_lo) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int B = kSplitBlock;
    const int lane = threadIdx.x;
    auto window = [&](int64_t w, float (&x)[E]) {
        decode<DT>(load16<NT>(g.base + 16 * (size_t)w), x);
        const int64_t c0 = w * E - g.head;
        if (c0 < 0 || c0 + E > N) {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int64_t c = c0 + k;
                if (c < 0 || c >= N) x[k] = kNegInf;
            }
        }
    };
    float lm = kNegInf;
    for (int64_t w = lane; w < g.nwin; w += B) {
        float x[E];
        window(w, x);
#pragma unroll
        for (int k = 0; k + 1 < E; k += 2) lm = max3f(lm, x[k], x[k + 1]);
    }
    m = row_max<B>(lm, lds_a);
    const float ms = (m == kNegInf) ? 0.f : m;
    if constexpr (DT == kF32) {
        CSum cs;
        for (int64_t w = lane; w < g.nwin; w += B) {
            float x[E];
            window(w, x);
#pragma unroll
            for (int k = 0; k < E; ++k) cs.add(exp_diff_acc(x[k], ms));
        }
        cs = row_csum<B>(cs, lds_b, lds_c);
        s_hi = cs.hi;
        s_lo = cs.lo;
    } else {
        const bool fast = __builtin_fabsf(ms) <= 0x1p125f;
        const float mL = ms * kLog2e;
        float acc = 0.f;
        for (int64_t w = lane; w < g.nwin; w += B) {
            float x[E];
            window(w, x);
#pragma unroll
            for (int k = 0; k < E; ++k)
                acc += fast ? exp2_fast(__builtin_fmaf(x[k], kLog2e, -mL))
                            : exp2_fast((x[k] - ms) * kLog2e);
        }
        s_hi = row_sum<B>(acc, lds_b);
        s_lo = 0.f;
    }
}

template <int DT, int V, bool NT>
__global__ void __launch_bounds__(kSplitBlock)
k_softmax_split(const unsigned char* in, unsigned char* out, SplitSlot* slots, SplitSync* sync,
                int64_t M, int N, int64_t in_sb, int64_t out_sb, int P, int S, uint32_t tag,
                int spin_limit, int same_phase, int recompute) {
    // S: windows per slice (<= B * V; the host spreads a row evenly over its P slices)
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    constexpr int B = kSplitBlock;
    __shared__ float lds_a[B / 64], lds_b[B / 64], lds_c[B / 64];
    __shared__ float lds_stat[4];

    const int lane = threadIdx.x;
    const int64_t items = M * P;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const RowGeom<DT> g(in + row * in_sb, N);
        const int64_t w0 = (int64_t)p * S + lane;  // this lane's first window
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;

        float x[V][E];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t w = w0 + (int64_t)B * v;
            const uint32_t ni = Elem<DT>::neg_inf_word;
            uint4 raw = make_uint4(ni, ni, ni, ni);
            if (w < wend) raw = load16<NT>(g.base + 16 * (size_t)w);
            decode<DT>(raw, x[v]);
        }
        // -inf outside [0, N) in windows that straddle the row's ends
        if (g.head != 0 || (N % E) != 0) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int64_t c0 = (w0 + (int64_t)B * v) * E - g.head;
                if (c0 < 0 || c0 + E > N) {
#pragma unroll
                    for (int k = 0; k < E; ++k) {
                        const int64_t c = c0 + k;
                        if (c < 0 || c >= N) x[v][k] = kNegInf;
                    }
                }
            }
        }

        // slice statistics
        float mp = kNegInf;
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
            for (int k = 0; k + 1 < E; k += 2) mp = max3f(mp, x[v][k], x[v][k + 1]);
        }
        mp = row_max<B>(mp, lds_a);
        const float msp = (mp == kNegInf) ? 0.f : mp;
        CSum sp;
        bool fast_exp = true;
        if constexpr (DT == kF32) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
#pragma unroll
                for (int k = 0; k < E; ++k) sp.add(exp_diff_acc(x[v][k], msp));
            }
            sp = row_csum<B>(sp, lds_b, lds_c);
        } else {
            float acc = 0.f;
            fast_exp = __builtin_fabsf(msp) <= 0x1p125f;
            const float mL = msp * kLog2e;
#pragma unroll
            for (int v = 0; v < V; ++v) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    x[v][k] = fast_exp ? exp2_fast(__builtin_fmaf(x[v][k], kLog2e, -mL))
                                       : exp2_fast((x[v][k] - msp) * kLog2e);
                    acc += x[v][k];
                }
            }
            sp.hi = row_sum<B>(acc, lds_b);
        }

        // publish, then gather the row's P pairs
        SplitSlot* row_slots = slots + row * P;
        if (lane == 0) {
            word_publish(row_slots[p].w, mp, tag);
            word_publish(row_slots[p].w + 1, sp.hi, tag);
            if constexpr (DT == kF32) word_publish(row_slots[p].w + 2, sp.lo, tag);
        }
        split_gather<DT>(row_slots, P, tag, spin_limit, lds_stat);
        __syncthreads();
        float m = lds_stat[0];
        float s = csum_value(lds_stat[1], lds_stat[2]);
        bool ok = lds_stat[3] != 0.f;  // uniform over the workgroup
        if (!ok) {
            if (lane == 0) atomicAdd(&sync->failures, 1u);
            if (recompute) {
                float hi, lo;
                split_row_stats<DT, NT>(g, N, lds_a, lds_b, lds_c, m, hi, lo);
                s = csum_value(hi, lo);
                ok = true;
            }
        }

        // y = exp(x - m) / s: FP32 recomputes exp from x with the row maximum;
        // FP16/BF16 rescale the slice's exponentials by exp(mp - m) / s.
        float r;
        if constexpr (DT == kF32) {
            r = (s == 0.f) ? 0.f : 1.0f / s;
        } else {
            r = (s == 0.f) ? 0.f : exp2_fast((mp - m) * kLog2e) / s;
        }
        if (!ok) r = __builtin_nanf("");
        const float mr = (m == kNegInf) ? 0.f : m;
        unsigned char* orow = out + row * out_sb;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t w = w0 + (int64_t)B * v;
            if (w < wend) {
                float y[E];
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if constexpr (DT == kF32) {
                        y[k] = exp_diff_acc(x[v][k], mr) * r;
                    } else {
                        y[k] = x[v][k] * r;
                    }
                }
                const uint4 enc = encode<DT>(y);
                const int64_t c0 = w * E - g.head;
                if (same_phase && c0 >= 0 && c0 + E <= N) {
                    store16(orow + (size_t)c0 * ES, enc);
                } else {
#pragma unroll
                    for (int k = 0; k < E; ++k) {
                        const int64_t c = c0 + k;
                        if (c >= 0 && c < N) store_elem<DT>(orow + (size_t)c * ES, enc, k);
                    }
                }
            }
        }
        __syncthreads();  // lds_stat is rewritten by the next item's gather
    }
}

// Backward: wave 0 sums the P partial dot products of a row (lane j adds slots
// j, j + 64, ... in order with TwoSum, then the wave's compensated tree) and
// leaves (hi, lo, ok) in LDS.
template <bool ACC>
__device__ __forceinline__ void split_gather_sum(const SplitSlot* row_slots, int P, uint32_t tag,
                                                 int spin_limit, float* lds_stat) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    int budget = spin_limit;
    bool ok = true;
    CSum s;
    for (int j = lane; j < P; j += 64) {
        constexpr int K = ACC ? 2 : 1;  // sum_hi (, sum_lo)
        float v[2] = {0.f, 0.f};
        float (&vk)[K] = *reinterpret_cast<float(*)[K]>(v);
        if (!words_wait<K>(row_slots[j].w + 1, tag, budget, vk)) {
            ok = false;
            break;
        }
        float t, e;
        two_sum(s.hi, v[0], t, e);
        s.hi = t;
        s.lo = (s.lo + v[1]) + e;
    }
    s = group_allreduce_csum<64>(s);
    const bool all_ok = __ballot(!ok) == 0;
    if (lane == 0) {
        lds_stat[1] = s.hi;
        lds_stat[2] = s.lo;
        lds_stat[3] = all_ok ? 1.f : 0.f;
    }
}

// Backward fallback after a wait ran out: the workgroup forms the row's whole dot
// product sum(y * dy) from the inputs (256 windows per step), on every lane.
template <int DT, bool NT>
__device__ __noinline__ float split_row_dot(const RowGeom<DT> g, const unsigned char* dyrow, int N,
                                            int dy_phase, float* lds_hi, float* lds_lo) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int B = kSplitBlock;
    const int lane = threadIdx.x;
    float acc = 0.f;
    CSum cs;
    for (int64_t w = lane; w < g.nwin; w += B) {
        float fy[1][E], fd[1][E];
        decode<DT>(load16<NT>(g.base + 16 * (size_t)w), fy[0]);
        load_dy<DT, 1>(fd, dyrow, g.head, N, w, 0, g.nwin, dy_phase != 0);
        zero_outside<DT, 1>(fy, g.head, N, w, 0);
        zero_outside<DT, 1>(fd, g.head, N, w, 0);
        lane_dot<DT, 1>(fy, fd, acc, cs);
    }
    if constexpr (DT == kF32) {
        cs = row_csum<B>(cs, lds_hi, lds_lo);
        return csum_value(cs.hi, cs.lo);
    } else {
        return row_sum<B>(acc, lds_hi);
    }
}

// One-launch backward of wide rows: a slice's partial dot sum(y * dy) is
// published and merged like the forward's (max, sum) pairs; y and dy stay in
// registers in their stored encoding; dx = y * (dy - dot) is written from them.
template <int DT, int V, bool NT>
__global__ void __launch_bounds__(kSplitBlock)
k_softmax_bwd_split(const unsigned char* y, const unsigned char* dy, unsigned char* dx,
                    SplitSlot* slots, SplitSync* sync, int64_t M, int N, int64_t y_sb,
                    int64_t dy_sb, int64_t dx_sb, int P, int S, uint32_t tag, int spin_limit,
                    int dy_phase, int dx_phase, int recompute) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int B = kSplitBlock;
    __shared__ float lds_hi[B / 64], lds_lo[B / 64];
    __shared__ float lds_stat[4];

    const int lane = threadIdx.x;
    const int64_t items = M * P;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const RowGeom<DT> g(y + row * y_sb, N);
        const int64_t w0 = (int64_t)p * S + lane;
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;

        uint32_t ry[V][4], rd[V][4];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t w = w0 + (int64_t)B * v;
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < wend) raw = load16<NT>(g.base + 16 * (size_t)w);
            ry[v][0] = raw.x;
            ry[v][1] = raw.y;
            ry[v][2] = raw.z;
            ry[v][3] = raw.w;
        }
        load_dy_raw<DT, V, NT>(rd, dy + row * dy_sb, g.head, N, w0, B, wend, dy_phase);
        if (g.head != 0 || (N % E) != 0) {
            zero_raw_outside<DT, V>(ry, g.head, N, w0, B);
            zero_raw_outside<DT, V>(rd, g.head, N, w0, B);
        }
        float acc = 0.f;
        CSum cs;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float fy[1][E], fd[1][E];
            decode_words<DT>(ry[v], fy[0]);
            decode_words<DT>(rd[v], fd[0]);
            lane_dot<DT, 1>(fy, fd, acc, cs);
        }
        if constexpr (DT == kF32) {
            cs = row_csum<B>(cs, lds_hi, lds_lo);
        } else {
            cs.hi = row_sum<B>(acc, lds_hi);
            cs.lo = 0.f;
        }

        SplitSlot* row_slots = slots + row * P;
        if (lane == 0) {
            word_publish(row_slots[p].w + 1, cs.hi, tag);
            if constexpr (DT == kF32) word_publish(row_slots[p].w + 2, cs.lo, tag);
        }
        split_gather_sum<DT == kF32>(row_slots, P, tag, spin_limit, lds_stat);
        __syncthreads();
        const bool ok = lds_stat[3] != 0.f;  // uniform over the workgroup
        float dot = ok ? csum_value(lds_stat[1], lds_stat[2]) : __builtin_nanf("");
        if (!ok) {
            if (lane == 0) atomicAdd(&sync->failures, 1u);
            if (recompute) dot = split_row_dot<DT, NT>(g, dy + row * dy_sb, N, dy_phase, lds_hi, lds_lo);
        }

        unsigned char* dxrow = dx + row * dx_sb;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t w = w0 + (int64_t)B * v;
            if (w < wend) {
                if constexpr (DT != kF32) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ry[v][i]), "+v"(rd[v][i]));
                }
                float fy[1][E], fd[1][E];
                decode_words<DT>(ry[v], fy[0]);
                decode_words<DT>(rd[v], fd[0]);
                store_dx<DT, 1>(fy, fd, dot, dxrow, g.head, N, w, 0, g.nwin, dx_phase);
            }
        }
        __syncthreads();
    }
}

}  // namespace smx
