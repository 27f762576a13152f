// sm_bwd.hpp -- gfx950 kernels of the softmax backward, dx = y * (dy - sum(y * dy)).
//
// The softmax keeps its output y and forms dx from it and the upstream gradient
// dy ("Measured optimization case studies", section "Training: backward kernels
// through autograd"). Per row that is one dot product and one elementwise pass:
// 3 * N * elem bytes (read y, read dy, write dx).
//
//   k_softmax_bwd_rows<DT, G, V>  one-pass: a group of G lanes holds the row of y
//       and of dy in registers (the window grid of the forward kernels, taken
//       from y's 16-byte phase), reduces the dot once (DPP, then one LDS step for
//       multi-wave rows) and writes dx.
//   k_bwd_wide_dot<DT> / k_bwd_wide_apply<DT>  rows wider than the one-pass
//       limit: pass 1 writes one compensated FP32 partial dot per wave, pass 2
//       merges a row's partials in a fixed order, re-reads y and dy, writes dx.
//
// dy may sit at another 16-byte phase than y (then its elements are loaded one
// by one); dx is stored with 16-byte stores when it shares y's phase.
#pragma once

#include "sm_kernels.hpp"

namespace smx {

// Value of a compensated pair. An infinite partial makes TwoSum's error term NaN
// (inf - inf); the pair's value is then the infinite part itself.
__device__ __forceinline__ float csum_value(float hi, float lo) {
    return __builtin_isfinite(hi) ? hi + lo : hi;
}

// Decoded elements of dy for the windows of y: vector loads when dy shares y's
// 16-byte phase, element loads otherwise. Columns outside [0, N) read as 0.
template <int DT, int NV>
__device__ __forceinline__ void load_dy(float (&f)[NV][Elem<DT>::per_vec], const unsigned char* dyrow,
                                        int head, int N, int64_t w0, int wstep, int nwin,
                                        bool dy_phase) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t w = w0 + (int64_t)wstep * v;
        const int64_t c0 = w * E - head;
        if (dy_phase) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < nwin) raw = load16<false>(dyrow - (size_t)head * ES + 16 * (size_t)w);
            decode<DT>(raw, f[v]);
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int64_t c = c0 + k;
                float val = 0.f;
                if (c >= 0 && c < N) {
                    const unsigned char* p = dyrow + (size_t)c * ES;
                    if constexpr (DT == kF32) {
                        val = *reinterpret_cast<const float*>(p);
                    } else if constexpr (DT == kBF16) {
                        val = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
                    } else {
                        val = (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(p));
                    }
                }
                f[v][k] = val;
            }
        }
    }
}

// Zero the elements of windows that straddle the row ends (they may hold data of
// neighbouring rows, including NaN or inf).
template <int DT, int NV>
__device__ __forceinline__ void zero_outside(float (&f)[NV][Elem<DT>::per_vec], int head, int N,
                                             int64_t w0, int wstep) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t c0 = (w0 + (int64_t)wstep * v) * E - head;
        if (c0 < 0 || c0 + E > N) {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int64_t c = c0 + k;
                if (c < 0 || c >= N) f[v][k] = 0.f;
            }
        }
    }
}

// Row dot product of the lane's elements (compensated with exact products for FP32).
template <int DT, int NV>
__device__ __forceinline__ void lane_dot(const float (&fy)[NV][Elem<DT>::per_vec],
                                         const float (&fd)[NV][Elem<DT>::per_vec], float& acc,
                                         CSum& cs) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if constexpr (DT == kF32) {
                const float p = fy[v][k] * fd[v][k];
                const float pe = __builtin_fmaf(fy[v][k], fd[v][k], -p);  // exact product error
                cs.add(p);
                cs.lo += pe;
            } else {
                acc = __builtin_fmaf(fy[v][k], fd[v][k], acc);
            }
        }
    }
}

// dx for the lane's windows: encode and store (16-byte when fully inside the row
// and dx shares y's phase, element stores otherwise).
template <int DT, int NV>
__device__ __forceinline__ void store_dx(const float (&fy)[NV][Elem<DT>::per_vec],
                                         const float (&fd)[NV][Elem<DT>::per_vec], float dot,
                                         unsigned char* dxrow, int head, int N, int64_t w0,
                                         int wstep, int nwin, bool dx_phase) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t w = w0 + (int64_t)wstep * v;
        if (w < nwin) {
            float o[E];
#pragma unroll
            for (int k = 0; k < E; ++k) o[k] = fy[v][k] * (fd[v][k] - dot);
            const uint4 enc = encode<DT>(o);
            const int64_t c0 = w * E - head;
            if (dx_phase && c0 >= 0 && c0 + E <= N) {
                store16(dxrow + (size_t)c0 * ES, enc);
            } else {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int64_t c = c0 + k;
                    if (c >= 0 && c < N) store_elem<DT>(dxrow + (size_t)c * ES, enc, k);
                }
            }
        }
    }
}

// Raw (encoded) words of a second operand on the row's window grid: 16-byte loads when
// it shares the row's 16-byte phase. Otherwise the bytes of window w (columns c0 ..
// c0 + E - 1, c0 = w*E - head) start sb bytes into an aligned 16-byte window, with
// sb = (operand address - head*ES) mod 16 the same for every window of the row: they are
// taken from the two aligned windows around them with a byte funnel shift
// (v_alignbyte_b32), and an aligned window is loaded only where it holds a byte of the
// operand's row [src, src + N*ES). Windows from wend on read as 0; columns outside
// [0, N) hold whatever the loaded windows hold there (callers zero or ignore them).
template <int DT, int NV, bool NT>
__device__ __forceinline__ void load_dy_raw(uint32_t (&r)[NV][4], const unsigned char* dyrow,
                                            int head, int N, int64_t w0, int wstep, int64_t wend,
                                            bool dy_phase) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    const uint32_t sb = (uint32_t)((reinterpret_cast<uintptr_t>(dyrow) - (uintptr_t)head * ES) & 15u);
    const uint32_t q = sb >> 2, rb = sb & 3u;
    const int64_t nbytes = (int64_t)N * ES;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t w = w0 + (int64_t)wstep * v;
        if (dy_phase) {
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < wend) raw = load16<NT>(dyrow - (size_t)head * ES + 16 * (size_t)w);
            r[v][0] = raw.x;
            r[v][1] = raw.y;
            r[v][2] = raw.z;
            r[v][3] = raw.w;
        } else {
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = make_uint4(0u, 0u, 0u, 0u);
            if (w < wend) {
                // byte offset from dyrow of the aligned window holding column c0 (pointer
                // arithmetic on dyrow keeps the loads global, not flat)
                const int64_t lo_off = (w * E - head) * (int64_t)ES - (int64_t)sb;
                if (lo_off < nbytes && lo_off + 16 > 0) lo = load16<NT>(dyrow + lo_off);
                if (lo_off + 16 < nbytes && lo_off + 32 > 0) hi = load16<NT>(dyrow + lo_off + 16);
            }
            // dword k of the 32 bytes (no local arrays: they would be placed in LDS)
            auto dw = [&](int k) -> uint32_t {
                const uint4& t = k < 4 ? lo : hi;
                switch (k & 3) {
                case 0: return t.x;
                case 1: return t.y;
                case 2: return t.z;
                default: return t.w;
                }
            };
            // dwords q .. q+4 (q = sb / 4 in 0..3), then the byte shift rb
            uint32_t d0 = 0u, d1 = 0u, d2 = 0u, d3 = 0u, d4 = 0u;
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const uint32_t a01 = (q & 1u) ? dw(j + 1) : dw(j);
                const uint32_t a23 = (q & 1u) ? dw(j + 3) : dw(j + 2);
                const uint32_t dj = (q & 2u) ? a23 : a01;
                if (j == 0) d0 = dj;
                if (j == 1) d1 = dj;
                if (j == 2) d2 = dj;
                if (j == 3) d3 = dj;
                if (j == 4) d4 = dj;
            }
            r[v][0] = __builtin_amdgcn_alignbyte(d1, d0, rb);
            r[v][1] = __builtin_amdgcn_alignbyte(d2, d1, rb);
            r[v][2] = __builtin_amdgcn_alignbyte(d3, d2, rb);
            r[v][3] = __builtin_amdgcn_alignbyte(d4, d3, rb);
        }
    }
}

// Zero the encoded elements of windows that straddle the row ends (they may hold
// data of neighbouring rows, including NaN or inf); +0 is the all-zero pattern.
template <int DT, int NV>
__device__ __forceinline__ void zero_raw_outside(uint32_t (&r)[NV][4], int head, int N, int64_t w0,
                                                 int wstep) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t c0 = (w0 + (int64_t)wstep * v) * E - head;
        if (c0 < 0 || c0 + E > N) {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int64_t c = c0 + k;
                if (c < 0 || c >= N) {
                    if constexpr (DT == kF32) {
                        r[v][k] = 0u;
                    } else {
                        r[v][k >> 1] &= (k & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                    }
                }
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ void decode_words(const uint32_t (&w)[4], float (&f)[Elem<DT>::per_vec]) {
    decode<DT>(make_uint4(w[0], w[1], w[2], w[3]), f);
}

// One-pass backward. y and dy stay in registers in their stored encoding (half
// the registers of decoded FP32 for 16-bit types, so wide rows keep full
// occupancy) and are decoded twice: for the dot and for dx.
template <int DT, int G, int V, bool NT>
__global__ void __launch_bounds__(RowLaunch<G>::block)
k_softmax_bwd_rows(const unsigned char* y, const unsigned char* dy, unsigned char* dx, int64_t M,
                   int N, int64_t y_sb, int64_t dy_sb, int64_t dx_sb, int dy_phase, int dx_phase,
                   int xcd_order) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int GPB = RowLaunch<G>::groups;
    constexpr int NW = G > 64 ? G / 64 : 1;
    // Two LDS buffers, alternating by row: with one barrier per row, a wave that
    // runs ahead to the next row never overwrites values a slower wave still reads.
    __shared__ float lds_hi[2][NW], lds_lo[2][NW];

    const int tid = threadIdx.x;
    const int lane = (GPB == 1) ? tid : (tid % G);
    const int grp = (GPB == 1) ? 0 : (tid / G);
    const int64_t rstep = (int64_t)gridDim.x * GPB;
    int parity = 0;
    for (int64_t row = xcd_block(xcd_order) * GPB + grp; row < M; row += rstep, parity ^= 1) {
        const RowGeom<DT> g(y + row * y_sb, N);
        uint32_t ry[V][4], rd[V][4];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int w = lane + G * v;
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < g.nwin) raw = load16<NT>(g.base + 16 * (size_t)w);
            ry[v][0] = raw.x;
            ry[v][1] = raw.y;
            ry[v][2] = raw.z;
            ry[v][3] = raw.w;
        }
        load_dy_raw<DT, V, NT>(rd, dy + row * dy_sb, g.head, N, lane, G, g.nwin, dy_phase);
        if (g.head != 0 || (N % E) != 0) {
            zero_raw_outside<DT, V>(ry, g.head, N, lane, G);
            zero_raw_outside<DT, V>(rd, g.head, N, lane, G);
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
        float dot;
        if constexpr (DT == kF32) {
            const CSum c = row_csum<G>(cs, lds_hi[parity], lds_lo[parity]);
            dot = csum_value(c.hi, c.lo);
        } else {
            dot = row_sum<G>(acc, lds_hi[parity]);
        }
        unsigned char* dxrow = dx + row * dx_sb;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t w = lane + (int64_t)G * v;
            if (w < g.nwin) {
                if constexpr (DT != kF32) {
                    // decode again rather than keep the decoded values live across
                    // the reduction (the empty asm hides that the words are unchanged)
#pragma unroll
                    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ry[v][i]), "+v"(rd[v][i]));
                }
                float fy[1][E], fd[1][E];
                decode_words<DT>(ry[v], fy[0]);
                decode_words<DT>(rd[v], fd[0]);
                store_dx<DT, 1>(fy, fd, dot, dxrow, g.head, N, w, 0, g.nwin, dx_phase);
            }
        }
    }
}

// ------------------------------------------------------------ wide rows
template <int DT>
__global__ void __launch_bounds__(256)
k_bwd_wide_dot(const unsigned char* y, const unsigned char* dy, float2* part, int64_t M, int N,
               int64_t y_sb, int64_t dy_sb, int cpw, int64_t wpr, int dy_phase) {
    constexpr int VPL = Wide<DT>::VPL;
    constexpr int WPC = Wide<DT>::WPC;
    constexpr int E = Elem<DT>::per_vec;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= M * wpr) return;  // whole waves only
    const int64_t row = gw / wpr;
    const int64_t wr = gw - row * wpr;
    const RowGeom<DT> g(y + row * y_sb, N);
    const int64_t nchunks = ((int64_t)g.nwin + WPC - 1) / WPC;
    const int64_t c_end = wr * cpw + cpw < nchunks ? wr * cpw + cpw : nchunks;
    float acc = 0.f;
    CSum cs;
    for (int64_t c = wr * cpw; c < c_end; ++c) {
        const int64_t w0 = c * WPC + lane;
        float fy[VPL][E], fd[VPL][E];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int64_t w = w0 + 64 * v;
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < g.nwin) raw = load16<false>(g.base + 16 * (size_t)w);
            decode<DT>(raw, fy[v]);
        }
        load_dy<DT, VPL>(fd, dy + row * dy_sb, g.head, N, w0, 64, g.nwin, dy_phase);
        if (g.head != 0 || (N % E) != 0) {
            zero_outside<DT, VPL>(fy, g.head, N, w0, 64);
            zero_outside<DT, VPL>(fd, g.head, N, w0, 64);
        }
        lane_dot<DT, VPL>(fy, fd, acc, cs);
    }
    if constexpr (DT != kF32) {
        cs.hi = acc;
        cs.lo = 0.f;
    }
    cs = group_allreduce_csum<64>(cs);
    if (lane == 0) part[gw] = make_float2(cs.hi, cs.lo);
}

template <int DT>
__global__ void __launch_bounds__(256)
k_bwd_wide_apply(const unsigned char* y, const unsigned char* dy, unsigned char* dx,
                 const float2* part, int64_t M, int N, int64_t y_sb, int64_t dy_sb, int64_t dx_sb,
                 int cpw, int64_t wpr, int dy_phase, int dx_phase) {
    constexpr int VPL = Wide<DT>::VPL;
    constexpr int WPC = Wide<DT>::WPC;
    constexpr int E = Elem<DT>::per_vec;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= M * wpr) return;
    const int64_t row = gw / wpr;
    const int64_t wr = gw - row * wpr;
    // the row's partial dots in a fixed order: lane-strided, then the wave tree
    CSum cs;
    for (int64_t k = lane; k < wpr; k += 64) {
        const float2 p = part[row * wpr + k];
        float s, e;
        two_sum(cs.hi, p.x, s, e);
        cs.hi = s;
        cs.lo = (cs.lo + p.y) + e;
    }
    cs = group_allreduce_csum<64>(cs);
    const float dot = csum_value(cs.hi, cs.lo);

    const RowGeom<DT> g(y + row * y_sb, N);
    const int64_t nchunks = ((int64_t)g.nwin + WPC - 1) / WPC;
    const int64_t c_end = wr * cpw + cpw < nchunks ? wr * cpw + cpw : nchunks;
    for (int64_t c = wr * cpw; c < c_end; ++c) {
        const int64_t w0 = c * WPC + lane;
        float fy[VPL][E], fd[VPL][E];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int64_t w = w0 + 64 * v;
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (w < g.nwin) raw = load16<false>(g.base + 16 * (size_t)w);
            decode<DT>(raw, fy[v]);
        }
        load_dy<DT, VPL>(fd, dy + row * dy_sb, g.head, N, w0, 64, g.nwin, dy_phase);
        store_dx<DT, VPL>(fy, fd, dot, dx + row * dx_sb, g.head, N, w0, 64, g.nwin, dx_phase);
    }
}

}  // namespace smx
