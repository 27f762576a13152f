// sm_kernels.hpp -- the gfx950 row-softmax kernels.
//
//   k_softmax_rows<DT, G, V, PF, NT>  one-pass row body (NT: streaming loads). A group of G lanes owns a
//       row and holds all of it in registers: lane l of the group loads the
//       16-byte windows l, l + G, ..., l + (V-1)G of the row's 16-byte-aligned
//       window grid, so every load instruction of a wave covers contiguous
//       memory. G = 16/32/64 keeps a row inside one wave (DPP reductions only);
//       G = 128..1024 spreads a row over G/64 waves of one workgroup with one
//       LDS exchange per reduction. Launched on a grid that covers every row
//       once (resident plan) or on occupancy x CUs workgroups that walk the
//       rows with a grid stride, prefetching the next row (persistent plan).
//   k_wide_stats<DT> / k_wide_norm<DT>  the two passes of the wide-row path.
//
// The arithmetic per row is the fused softmax: max, exp(x - max), sum, one
// reciprocal per row, scale, one rounding to the storage dtype.
#pragma once

#include "sm_device.hpp"

namespace smx {

// Rows hold their elements on a grid of 16-byte windows aligned to 16 bytes.
// `head` is the number of elements between the aligned window start and the
// row's first element (0 when the row starts 16-byte aligned); window w holds
// row columns [w*E - head, w*E - head + E).
template <int DT>
struct RowGeom {
    static constexpr int E = Elem<DT>::per_vec;
    static constexpr int ES = Elem<DT>::bytes;
    const unsigned char* base;  // aligned start of window 0
    int head;
    int nwin;                   // windows that hold at least one row element
    __device__ __forceinline__ RowGeom(const unsigned char* row, int N) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(row);
        head = (int)((a & 15u) / ES);
        base = row - (a & 15u);
        // head + N + E - 1 exceeds INT32_MAX for N within 14 of it: sum in 64 bits
        // (the quotient, at most 2^30 + 4, fits)
        nwin = (int)(((int64_t)head + N + E - 1) / E);
    }
};

// Load the V windows of one lane (windows past the row read as -inf words; a
// window that holds at least one row element lies inside the same 4 KiB page
// as that element, so it can always be read).
template <int DT, int G, int V, bool NT>
__device__ __forceinline__ void load_row(uint4 (&raw)[V], const unsigned char* in, int64_t row,
                                         int64_t M, int N, int64_t in_sb, int lane) {
    if (row >= M) return;
    const RowGeom<DT> g(in + row * in_sb, N);
    const uint32_t ni = Elem<DT>::neg_inf_word;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int w = lane + G * v;
        if (w < g.nwin)
            raw[v] = load16<NT>(g.base + 16 * (size_t)w);
        else
            raw[v] = make_uint4(ni, ni, ni, ni);
    }
}

// Reductions over the row group: within a wave by DPP, across the waves of a
// workgroup through LDS (one barrier).
template <int G>
__device__ __forceinline__ float row_max(float m, float* lds) {
    if constexpr (G <= 64) {
        return group_allreduce<G>(m, OpMax{});
    } else {
        m = group_allreduce<64>(m, OpMax{});
        const int t = threadIdx.x;
        if ((t & 63) == 0) lds[t >> 6] = m;
        __syncthreads();
        float r = lds[0];
#pragma unroll
        for (int w = 1; w < G / 64; ++w) r = fmax_nan(r, lds[w]);
        return r;
    }
}

template <int G>
__device__ __forceinline__ float row_sum(float s, float* lds) {
    if constexpr (G <= 64) {
        return group_allreduce<G>(s, OpAdd{});
    } else {
        s = group_allreduce<64>(s, OpAdd{});
        const int t = threadIdx.x;
        if ((t & 63) == 0) lds[t >> 6] = s;
        __syncthreads();
        float r = lds[0];
#pragma unroll
        for (int w = 1; w < G / 64; ++w) r += lds[w];
        return r;
    }
}

template <int G>
__device__ __forceinline__ CSum row_csum(CSum c, float* lds_hi, float* lds_lo) {
    if constexpr (G <= 64) {
        c = group_allreduce_csum<G>(c);
    } else {
        c = group_allreduce_csum<64>(c);
        const int t = threadIdx.x;
        if ((t & 63) == 0) {
            lds_hi[t >> 6] = c.hi;
            lds_lo[t >> 6] = c.lo;
        }
        __syncthreads();
        CSum r;
        r.hi = lds_hi[0];
        r.lo = lds_lo[0];
#pragma unroll
        for (int w = 1; w < G / 64; ++w) {
            float e, s;
            two_sum(r.hi, lds_hi[w], s, e);
            r.hi = s;
            r.lo = (r.lo + lds_lo[w]) + e;
        }
        c = r;
    }
    return c;
}

template <int G>
__device__ __forceinline__ float row_sum_acc(CSum c, float* lds_hi, float* lds_lo) {
    c = row_csum<G>(c, lds_hi, lds_lo);
    return c.hi + c.lo;
}

// One row: decode, mask, max, exponentials, sum, scale, encode, store.
template <int DT, int G, int V>
__device__ __forceinline__ void process_row(const uint4 (&raw)[V], const unsigned char* in,
                                            unsigned char* out, int64_t row, int N, int64_t in_sb,
                                            int64_t out_sb, int same_phase, int lane, float* lds_a,
                                            float* lds_b, float* lds_c) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    const RowGeom<DT> g(in + row * in_sb, N);

    float x[V][E];
#pragma unroll
    for (int v = 0; v < V; ++v) decode<DT>(raw[v], x[v]);

    // Masked lanes take -inf (exp(-inf) = 0 adds nothing): only windows that
    // straddle the row's ends need it, and only ragged rows have such windows.
    if (g.head != 0 || (N % E) != 0) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int c0 = (lane + G * v) * E - g.head;
            if (c0 < 0 || c0 + E > N) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int c = c0 + k;
                    if (c < 0 || c >= N) x[v][k] = kNegInf;
                }
            }
        }
    }

    // Row maximum.
    float m = kNegInf;
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k + 1 < E; k += 2) m = max3f(m, x[v][k], x[v][k + 1]);
    }
    m = row_max<G>(m, lds_a);
    // A row with no finite maximum (all -inf) shifts by 0 and keeps a zero sum.
    const float ms = (m == kNegInf) ? 0.f : m;

    float s;
    if constexpr (DT == kF32) {
        CSum cs;
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                x[v][k] = exp_diff_acc(x[v][k], ms);
                cs.add(x[v][k]);
            }
        }
        s = row_sum_acc<G>(cs, lds_b, lds_c);
    } else {
        float acc = 0.f;
        if (__builtin_fabsf(ms) <= 0x1p125f) {
            const float mL = ms * kLog2e;
#pragma unroll
            for (int v = 0; v < V; ++v) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    x[v][k] = exp2_fast(__builtin_fmaf(x[v][k], kLog2e, -mL));
                    acc += x[v][k];
                }
            }
        } else {  // |max| near FLT_MAX (BF16 range) or NaN: subtract before scaling
#pragma unroll
            for (int v = 0; v < V; ++v) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    x[v][k] = exp2_fast((x[v][k] - ms) * kLog2e);
                    acc += x[v][k];
                }
            }
        }
        s = row_sum<G>(acc, lds_b);
    }
    // One reciprocal per row; an all-masked row (s == 0) writes zeros and a
    // NaN sum keeps the row NaN.
    const float r = (s == 0.f) ? 0.f : 1.0f / s;

    unsigned char* orow = out + row * out_sb;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int w = lane + G * v;
        if (w < g.nwin) {
            float y[E];
#pragma unroll
            for (int k = 0; k < E; ++k) y[k] = x[v][k] * r;
            const uint4 enc = encode<DT>(y);
            const int c0 = w * E - g.head;
            if (same_phase && c0 >= 0 && c0 + E <= N) {
                store16(orow + (size_t)c0 * ES, enc);
            } else {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int c = c0 + k;
                    if (c >= 0 && c < N) store_elem<DT>(orow + (size_t)c * ES, enc, k);
                }
            }
        }
    }
}

// Workgroup shape: rows that fit in a wave share 256-thread workgroups (several
// row groups per workgroup, no barriers); a row spread over several waves gets
// a workgroup of exactly its G lanes, so its barriers are uniform.
// XCDs of an MI355X; the workgroups of a launch are dealt to them in turn.
constexpr int kXcds = 8;

// This workgroup's index, or with xcd_order a permutation of the grid under which
// each XCD takes a contiguous range of indices: rows that share a cache line at
// their boundary then meet in one L2.
__device__ __forceinline__ int64_t xcd_block(int xcd_order) {
    int64_t b = blockIdx.x;
    if (xcd_order) {
        const int64_t bx = b % kXcds, bj = b / kXcds;
        const int64_t bq = (int64_t)gridDim.x / kXcds, br = (int64_t)gridDim.x % kXcds;
        b = bx < br ? bx * (bq + 1) + bj : br * (bq + 1) + (bx - br) * bq + bj;
    }
    return b;
}

template <int G>
struct RowLaunch {
    static constexpr int block = G > 64 ? G : 256;
    static constexpr int groups = block / G;  // rows in flight per workgroup
    static_assert(G <= 64 || groups == 1, "multi-wave rows own their workgroup");
};

template <int DT, int G, int V, bool PF, bool NT>
__global__ void __launch_bounds__(RowLaunch<G>::block)
k_softmax_rows(const unsigned char* in, unsigned char* out, int64_t M, int N, int64_t in_sb,
               int64_t out_sb, int same_phase, int xcd_order) {
    constexpr int GPB = RowLaunch<G>::groups;
    constexpr int NW = G > 64 ? G / 64 : 1;
    __shared__ float lds_a[NW], lds_b[NW], lds_c[NW];

    const int tid = threadIdx.x;
    const int lane = (GPB == 1) ? tid : (tid % G);
    const int grp = (GPB == 1) ? 0 : (tid / G);
    const int64_t rstep = (int64_t)gridDim.x * GPB;
    int64_t row = xcd_block(xcd_order) * GPB + grp;

    uint4 cur[V];
    load_row<DT, G, V, NT>(cur, in, row, M, N, in_sb, lane);
    while (row < M) {
        const int64_t next = row + rstep;
        if constexpr (PF) {
            uint4 nxt[V];
            load_row<DT, G, V, NT>(nxt, in, next, M, N, in_sb, lane);
            process_row<DT, G, V>(cur, in, out, row, N, in_sb, out_sb, same_phase, lane, lds_a,
                                  lds_b, lds_c);
#pragma unroll
            for (int v = 0; v < V; ++v) cur[v] = nxt[v];
        } else {
            process_row<DT, G, V>(cur, in, out, row, N, in_sb, out_sb, same_phase, lane, lds_a,
                                  lds_b, lds_c);
            load_row<DT, G, V, NT>(cur, in, next, M, N, in_sb, lane);
        }
        row = next;
    }
}

// ------------------------------------------------------------ wide path
// A chunk is 1024 elements of the row's window grid: WPC windows, of which each
// lane of a wave holds WPC/64. Wave gw owns chunks [wr*cpw, (wr+1)*cpw) of row
// gw / wpr (wr = gw % wpr), in both passes.
template <int DT>
struct Wide {
    static constexpr int E = Elem<DT>::per_vec;
    static constexpr int WPC = 1024 / E;  // windows per chunk
    static constexpr int VPL = WPC / 64;  // windows per lane per chunk
};

template <int DT, bool NT>
__device__ __forceinline__ void load_chunk(uint4 (&raw)[Wide<DT>::VPL], const RowGeom<DT>& g,
                                           int64_t c, int lane) {
    constexpr int WPC = Wide<DT>::WPC;
    const uint32_t ni = Elem<DT>::neg_inf_word;
#pragma unroll
    for (int v = 0; v < Wide<DT>::VPL; ++v) {
        const int64_t w = c * WPC + lane + 64 * v;
        if (w < g.nwin)
            raw[v] = load16<NT>(g.base + 16 * (size_t)w);
        else
            raw[v] = make_uint4(ni, ni, ni, ni);
    }
}

template <int DT>
__device__ __forceinline__ void decode_chunk(const uint4 (&raw)[Wide<DT>::VPL],
                                             float (&x)[Wide<DT>::VPL][Elem<DT>::per_vec],
                                             const RowGeom<DT>& g, int N, int64_t c, int lane) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int WPC = Wide<DT>::WPC;
#pragma unroll
    for (int v = 0; v < Wide<DT>::VPL; ++v) decode<DT>(raw[v], x[v]);
    if (g.head != 0 || (N % E) != 0) {
#pragma unroll
        for (int v = 0; v < Wide<DT>::VPL; ++v) {
            const int64_t c0 = (c * WPC + lane + 64 * v) * E - g.head;
            if (c0 < 0 || c0 + E > N) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int64_t cc = c0 + k;
                    if (cc < 0 || cc >= N) x[v][k] = kNegInf;
                }
            }
        }
    }
}

// Pass 1: per-lane online (max, sum) over the wave's chunks; then the wave's
// 64 lane states are merged and written as one (max, sum) pair.
template <int DT, bool NT>
__global__ void __launch_bounds__(256)
k_wide_stats(const unsigned char* in, float2* stats, int64_t M, int N, int64_t in_sb, int cpw,
             int64_t wpr) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int VPL = Wide<DT>::VPL;
    constexpr int WPC = Wide<DT>::WPC;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= M * wpr) return;  // whole waves only
    const int64_t row = gw / wpr;
    const int64_t wr = gw - row * wpr;
    const RowGeom<DT> g(in + row * in_sb, N);
    const int64_t nchunks = ((int64_t)g.nwin + WPC - 1) / WPC;
    const int64_t c_begin = wr * cpw;
    const int64_t c_end = c_begin + cpw < nchunks ? c_begin + cpw : nchunks;

    float m = kNegInf;
    float s = 0.f;
    CSum cs;
    for (int64_t c = c_begin; c < c_end; ++c) {
        uint4 raw[VPL];
        load_chunk<DT, NT>(raw, g, c, lane);
        float x[VPL][E];
        decode_chunk<DT>(raw, x, g, N, c, lane);
        float cm = m;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
#pragma unroll
            for (int k = 0; k + 1 < E; k += 2) cm = max3f(cm, x[v][k], x[v][k + 1]);
        }
        // A lane that has seen only -inf (or NaN) shifts by 0: its sum stays 0, or
        // becomes NaN if a NaN went by, and exp(-inf - (-inf)) is never formed.
        const float sh = (cm == kNegInf) ? 0.f : cm;
        if constexpr (DT == kF32) {
            const float f = exp_diff_acc(m, sh);  // m = -inf -> 0
            cs.hi *= f;
            cs.lo *= f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
#pragma unroll
                for (int k = 0; k < E; ++k) cs.add(exp_diff_acc(x[v][k], sh));
            }
        } else {
            float acc = s * exp2_fast((m - sh) * kLog2e);
            if (__builtin_fabsf(sh) <= 0x1p125f) {
                const float mL = sh * kLog2e;
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
#pragma unroll
                    for (int k = 0; k < E; ++k) acc += exp2_fast(__builtin_fmaf(x[v][k], kLog2e, -mL));
                }
            } else {
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
#pragma unroll
                    for (int k = 0; k < E; ++k) acc += exp2_fast((x[v][k] - sh) * kLog2e);
                }
            }
            s = acc;
        }
        m = cm;
    }
    if constexpr (DT == kF32) {
        group_merge_acc<64>(m, cs);
        s = cs.hi + cs.lo;
    } else {
        group_merge_fast<64>(m, s);
    }
    if (lane == 0) stats[gw] = make_float2(m, s);
}

// Merge the wpr pairs of a row in a fixed order (lane-strided, then the wave
// tree), so every wave of the row obtains bitwise the same (max, sum).
template <int DT>
__device__ __forceinline__ void row_stats(const float2* st, int64_t wpr, int lane, float& m,
                                          float& s) {
    m = kNegInf;
    if constexpr (DT == kF32) {
        CSum cs;
        for (int64_t k = lane; k < wpr; k += 64) {
            const float2 p = st[k];
            CSum o;
            o.hi = p.y;
            merge_acc(m, cs, p.x, o);
        }
        group_merge_acc<64>(m, cs);
        s = cs.hi + cs.lo;
    } else {
        s = 0.f;
        for (int64_t k = lane; k < wpr; k += 64) {
            const float2 p = st[k];
            merge_fast(m, s, p.x, p.y);
        }
        group_merge_fast<64>(m, s);
    }
}

// Pass 2: merge the row's statistics, re-read the wave's chunks, normalise,
// round once, store.
template <int DT, bool NT>
__global__ void __launch_bounds__(256)
k_wide_norm(const unsigned char* in, unsigned char* out, const float2* stats, int64_t M, int N,
            int64_t in_sb, int64_t out_sb, int cpw, int64_t wpr, int same_phase) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    constexpr int VPL = Wide<DT>::VPL;
    constexpr int WPC = Wide<DT>::WPC;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= M * wpr) return;
    const int64_t row = gw / wpr;
    const int64_t wr = gw - row * wpr;
    const RowGeom<DT> g(in + row * in_sb, N);
    const int64_t nchunks = ((int64_t)g.nwin + WPC - 1) / WPC;
    const int64_t c_begin = wr * cpw;
    const int64_t c_end = c_begin + cpw < nchunks ? c_begin + cpw : nchunks;

    float m, s;
    row_stats<DT>(stats + row * wpr, wpr, lane, m, s);
    const float ms = (m == kNegInf) ? 0.f : m;
    const float r = (s == 0.f) ? 0.f : 1.0f / s;
    const bool fast = __builtin_fabsf(ms) <= 0x1p125f;
    const float mL = ms * kLog2e;
    unsigned char* orow = out + row * out_sb;

    for (int64_t c = c_begin; c < c_end; ++c) {
        uint4 raw[VPL];
        load_chunk<DT, NT>(raw, g, c, lane);
        float x[VPL][E];
#pragma unroll
        for (int v = 0; v < VPL; ++v) decode<DT>(raw[v], x[v]);
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int64_t w = c * WPC + lane + 64 * v;
            if (w < g.nwin) {
                float y[E];
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    float e;
                    if constexpr (DT == kF32) {
                        e = exp_diff_acc(x[v][k], ms);
                    } else {
                        e = fast ? exp2_fast(__builtin_fmaf(x[v][k], kLog2e, -mL))
                                 : exp2_fast((x[v][k] - ms) * kLog2e);
                    }
                    y[k] = e * r;
                }
                const uint4 enc = encode<DT>(y);
                const int64_t c0 = w * E - g.head;
                if (same_phase && c0 >= 0 && c0 + E <= N) {
                    store16(orow + (size_t)c0 * ES, enc);
                } else {
#pragma unroll
                    for (int k = 0; k < E; ++k) {
                        const int64_t cc = c0 + k;
                        if (cc >= 0 && cc < N) store_elem<DT>(orow + (size_t)cc * ES, enc, k);
                    }
                }
            }
        }
    }
}

}  // namespace smx
