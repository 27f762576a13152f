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
// failure and, when the output does not alias the input (`recompute`), leaves that
// slice for after its item loop: there wave 0 derives the row's statistics from the
// whole input row -- the same definition, in another summation order -- and the
// workgroup writes the slice from a re-read of its input, so the result does not
// depend on scheduling. (Done inside the loop, the fallback's registers added to the
// live slice and cut the occupancy of the common path; after the loop nothing of a
// slice is live.) In place, where the row's other slices may already have
// overwritten their input, it writes NaN over its slice instead.
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

// Wave 0's fallback after a wait ran out: its 64 lanes walk the whole input row
// (16-byte windows lane, lane + 64, ...) with a per-lane online (max, sum), two
// elements at a time, merged over the wave afterwards: the same definition as the
// slices' statistics, in another order. Kept small: it shares the kernel's register
// budget with the hot path.
template <int DT, bool NT>
__device__ __forceinline__ void wave_row_stats(const RowGeom<DT>& g, int N, float& m, CSum& s) {
    constexpr int E = Elem<DT>::per_vec;
    const int lane = threadIdx.x & 63;
    m = kNegInf;
    s = CSum{};
#pragma unroll 1
    for (int w = lane; w < g.nwin; w += 64) {
        const uint4 raw = load16<NT>(g.base + 16 * (size_t)w);
        const uint32_t word[4] = {raw.x, raw.y, raw.z, raw.w};
        const int c0 = w * E - g.head;
#pragma unroll
        for (int k = 0; k < E; k += 2) {
            float a, b;
            if constexpr (DT == kF32) {
                a = __uint_as_float(word[k]);
                b = __uint_as_float(word[k + 1]);
            } else {
                const f2_t pr = unpack2<DT>(word[k / 2]);
                a = pr.x;
                b = pr.y;
            }
            if (c0 + k < 0 || c0 + k >= N) a = kNegInf;
            if (c0 + k + 1 < 0 || c0 + k + 1 >= N) b = kNegInf;
            const float pm = fmax_nan(a, b);
            const float sh = (pm == kNegInf) ? 0.f : pm;  // shift 0 for an all -inf pair
            if constexpr (DT == kF32) {
                CSum c;
                c.add(exp_diff_acc(a, sh));
                c.add(exp_diff_acc(b, sh));
                merge_acc(m, s, pm, c);
            } else {
                merge_fast(m, s.hi, pm, exp2_fast((a - sh) * kLog2e) + exp2_fast((b - sh) * kLog2e));
            }
        }
    }
    if constexpr (DT == kF32) {
        group_merge_acc<64>(m, s);
    } else {
        group_merge_fast<64>(m, s.hi);
    }
}

// Fallback output of one slice: its windows re-read one at a time and written as
// exp(x - m) / s with the row statistics (m, s) of wave_row_stats.
template <int DT, int V, bool NT>
__device__ __forceinline__ void split_write_from_input(const RowGeom<DT>& g, int N, int64_t w0,
                                                       int64_t wend, unsigned char* orow,
                                                       int same_phase, float m, float s) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    const float r = (s == 0.f) ? 0.f : 1.0f / s;
    const float ms = (m == kNegInf) ? 0.f : m;
#pragma unroll 1
    for (int64_t w = w0; w < wend; w += kSplitBlock) {
        float x[E], y[E];
        decode<DT>(load16<NT>(g.base + 16 * (size_t)w), x);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if constexpr (DT == kF32) {
                y[k] = exp_diff_acc(x[k], ms) * r;
            } else {
                y[k] = exp2_fast((x[k] - ms) * kLog2e) * r;
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

// Slices per workgroup whose output is deferred after a timed-out wait (one per round;
// further timed-out slices of a workgroup with more rounds than this are written NaN)
constexpr int kSplitMaxDeferred = 32;

// Waves per SIMD requested of the 4-vector forward instances: 8, i.e. at most 64 VGPRs
// and about 80 SGPRs (the rest spill to VGPR lanes). Left to itself the compiler takes
// 105 SGPRs, which allows 7 waves, and rows of 16 slices of 4 vectors then fill only 7/8
// of a round (measured, MI355X, cold: BF16 64 x 131072 9.32 -> 8.8 us, 1024 x 131072 120.7
// -> 112.7 us, FP32 64 x 65536 12.86 -> 12.1 us; the spills cost 2-3% where the plan
// does not change, e.g. 1 x 2^20 BF16 5.68 -> 5.81 us). The FP32 1- and 8-vector
// instances, which FP32 rows take for few and for many rows per call, are held at the
// occupancy they had before the timed-out-slice fallback was added (8 and 6 waves; the
// fallback's code otherwise cost each of them a wave). Other instances keep the
// compiler's choice.
template <int DT, int V>
constexpr int kSplitWaves = V == 4 ? 8 : (DT == kF32 && V == 1) ? 8 : (DT == kF32 && V == 8) ? 6 : 1;

template <int DT, int V, bool NT>
__global__ void __launch_bounds__(kSplitBlock)
__attribute__((amdgpu_waves_per_eu(kSplitWaves<DT, V>)))
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
    __shared__ int64_t failed[kSplitMaxDeferred];  // items whose wait ran out (out of place)
    int n_failed = 0;                               // uniform over the workgroup
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
        const float m = lds_stat[0];
        const float s = csum_value(lds_stat[1], lds_stat[2]);
        const bool ok = lds_stat[3] != 0.f;  // uniform over the workgroup
        unsigned char* orow = out + row * out_sb;
        if (!ok) {
            if (lane == 0) atomicAdd(&sync->failures, 1u);
            if (recompute && n_failed < kSplitMaxDeferred) {
                // out of place: the slice is written after the item loop, from the
                // input, once no slice data is live (see below)
                if (lane == 0) failed[n_failed] = item;
                ++n_failed;
                __syncthreads();  // lds_stat is rewritten by the next item's gather
                continue;
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
    // Slices whose wait ran out: wave 0 forms the row's statistics from the whole input
    // row, then every lane rewrites its windows of the slice from the input.
    for (int f = 0; f < n_failed; ++f) {
        const int64_t item = failed[f];
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const RowGeom<DT> g(in + row * in_sb, N);
        const int64_t w0 = (int64_t)p * S + lane;
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;
        if (lane < 64) {
            float mf;
            CSum sf;
            wave_row_stats<DT, NT>(g, N, mf, sf);
            if (lane == 0) {
                lds_stat[0] = mf;
                lds_stat[1] = csum_value(sf.hi, sf.lo);
            }
        }
        __syncthreads();
        split_write_from_input<DT, V, NT>(g, N, w0, wend, out + row * out_sb, same_phase, lds_stat[0],
                                          lds_stat[1]);
        __syncthreads();
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

// Gather of the second launch of a two-launch form: every word was published by the
// earlier launch, so nothing is waited for. All lanes of the workgroup read the row's
// slots (lane t takes slots t, t + 256, ..., four loads issued before any is used), sum
// them in slot order with the compensated step, then reduce over the workgroup in a
// fixed tree, so every workgroup derives bitwise the same total. `ok` is false if a word
// lacks the tag (which the publishing launch rules out). A row of P slices costs P/256
// independent loads per lane instead of P/64 dependent ones on one wave.
template <bool ACC>
__device__ __forceinline__ CSum split_sum_published(const SplitSlot* row_slots, int P, uint32_t tag,
                                                    float* lds_hi, float* lds_lo, bool& ok) {
    constexpr int B = kSplitBlock;
    constexpr int U = 4;
    const int t = threadIdx.x;
    CSum s;
    bool good = true;
    for (int j0 = t; j0 < P; j0 += U * B) {
        uint64_t hw[U], lw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * B;
            hw[u] = lw[u] = 0;
            if (j < P) {
                hw[u] = __hip_atomic_load(row_slots[j].w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if constexpr (ACC)
                    lw[u] = __hip_atomic_load(row_slots[j].w + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + u * B < P) {
                good = good && (uint32_t)(hw[u] >> 32) == tag && (!ACC || (uint32_t)(lw[u] >> 32) == tag);
                float tt, e;
                two_sum(s.hi, __uint_as_float((uint32_t)hw[u]), tt, e);
                s.hi = tt;
                s.lo = (s.lo + (ACC ? __uint_as_float((uint32_t)lw[u]) : 0.f)) + e;
            }
        }
    }
    s = row_csum<B>(s, lds_hi, lds_lo);
    ok = __syncthreads_and(good ? 1 : 0) != 0;
    return s;
}

// Backward fallback after a wait ran out: wave 0's 64 lanes form the row's whole dot
// product sum(y * dy) from the inputs, element by element (compensated with exact
// products for FP32 data, as the slices), reduced over the wave.
template <int DT>
__device__ __forceinline__ float wave_row_dot(const unsigned char* yrow, const unsigned char* dyrow,
                                              int N) {
    constexpr int ES = Elem<DT>::bytes;
    const int lane = threadIdx.x & 63;
    float acc = 0.f;
    CSum cs;
#pragma unroll 1
    for (int c = lane; c < N; c += 64) {
        const float a = load_elem<DT>(yrow + (size_t)c * ES);
        const float b = load_elem<DT>(dyrow + (size_t)c * ES);
        if constexpr (DT == kF32) {
            const float pr = a * b;
            cs.add(pr);
            cs.lo += __builtin_fmaf(a, b, -pr);  // the product's exact rounding error
        } else {
            acc = __builtin_fmaf(a, b, acc);
        }
    }
    if constexpr (DT == kF32) {
        cs = group_allreduce_csum<64>(cs);
        return csum_value(cs.hi, cs.lo);
    } else {
        return group_allreduce<64>(acc, OpAdd{});
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
    __shared__ int64_t failed[kSplitMaxDeferred];  // items whose wait ran out (out of place)
    int n_failed = 0;                               // uniform over the workgroup
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
        const float dot = ok ? csum_value(lds_stat[1], lds_stat[2]) : __builtin_nanf("");
        if (!ok) {
            if (lane == 0) atomicAdd(&sync->failures, 1u);
            if (recompute && n_failed < kSplitMaxDeferred) {  // written after the loop
                if (lane == 0) failed[n_failed] = item;
                ++n_failed;
                __syncthreads();
                continue;
            }
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
    // Slices whose wait ran out: wave 0 forms the row's dot from the whole input rows,
    // then every lane rewrites its windows of dx from a re-read of y and dy.
    for (int f = 0; f < n_failed; ++f) {
        const int64_t item = failed[f];
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const RowGeom<DT> g(y + row * y_sb, N);
        const unsigned char* dyrow = dy + row * dy_sb;
        if (lane < 64) {
            const float d = wave_row_dot<DT>(y + row * y_sb, dyrow, N);
            if (lane == 0) lds_stat[1] = d;
        }
        __syncthreads();
        const float d = lds_stat[1];
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;
#pragma unroll 1
        for (int64_t w = (int64_t)p * S + lane; w < wend; w += B) {
            float fy[1][E], fd[1][E];
            decode<DT>(load16<NT>(g.base + 16 * (size_t)w), fy[0]);
            load_dy<DT, 1>(fd, dyrow, g.head, N, w, 0, g.nwin, dy_phase != 0);
            store_dx<DT, 1>(fy, fd, d, dx + row * dx_sb, g.head, N, w, 0, g.nwin, dx_phase);
        }
        __syncthreads();
    }
}

}  // namespace smx
