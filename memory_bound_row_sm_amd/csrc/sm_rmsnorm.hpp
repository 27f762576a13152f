// sm_rmsnorm.hpp -- gfx950 kernels of the fused residual RMSNorm.
//
// Per row (Warpline README, the description of its K1 kernel): s = x + r added in
// FP32 and rounded once to the dtype, q = sum s^2 in FP32, y = s * rsqrt(q / N +
// eps) * w rounded once to the dtype. The rounded sum s can also be written out
// (the residual stream of the next layer); without a residual, s = x.
//
//   k_rmsnorm_rows<DT, G, V, NT>   one-pass: a group of G lanes holds the row's s
//       in registers in its stored encoding (the window grid of the softmax row
//       kernels), reduces q once and writes y (and s).
//   k_rmsnorm_split<DT, V, NT>     rows cut into P slices of 256-lane workgroups
//       that exchange partial sums of squares through tagged words, as the
//       SPLIT softmax does. mode 0: one launch (publish, wait, apply); modes 1
//       and 2 split that into two launches (publish only; then gather the already
//       published partials and apply, re-reading x and r) for rows whose slices
//       cannot all be resident at once.
//
// Algorithmic bytes per element: read x, (r), w; write y, (s) -- with the
// residual and without s: 4 * elem requested (w counted per row, as the pages'
// byte model does), 3 * elem + N * elem / M from HBM.
#pragma once

#include "sm_bwd.hpp"
#include "sm_split.hpp"

namespace smx {

enum RmsFlags : int {
    kRmsResidual = 1,  // r is present
    kRmsResPhase = 2,  // r rows share x rows' 16-byte phase (vector loads)
    kRmsOutPhase = 4,  // y rows share x rows' phase (16-byte stores)
    kRmsSumOut = 8,    // write s
    kRmsSumPhase = 16,  // s rows share x rows' phase
    kRmsXcdOrder = 32,  // one-pass rows: workgroups renumbered XCD-contiguously
    kRmsRecompute = 64  // split: neither output aliases x or r, so a slice whose wait
                        // ran out may re-read the whole row
};

// Store one encoded window of a row (16-byte when inside the row and in phase,
// element stores otherwise).
template <int DT>
__device__ __forceinline__ void store_window(unsigned char* orow, const uint4 enc, int64_t w,
                                             int head, int N, bool phase) {
    constexpr int E = Elem<DT>::per_vec;
    constexpr int ES = Elem<DT>::bytes;
    const int64_t c0 = w * E - head;
    if (phase && c0 >= 0 && c0 + E <= N) {
        store16(orow + (size_t)c0 * ES, enc);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int64_t c = c0 + k;
            if (c >= 0 && c < N) store_elem<DT>(orow + (size_t)c * ES, enc, k);
        }
    }
}

// s = x + r (FP32 add, one rounding to the dtype) on the encoded words of one window.
template <int DT>
__device__ __forceinline__ void add_round(uint32_t (&sx)[4], const uint32_t (&rr)[4]) {
    constexpr int E = Elem<DT>::per_vec;
    float a[E], b[E];
    decode_words<DT>(sx, a);
    decode_words<DT>(rr, b);
#pragma unroll
    for (int k = 0; k < E; ++k) a[k] = a[k] + b[k];
    const uint4 enc = encode<DT>(a);
    sx[0] = enc.x;
    sx[1] = enc.y;
    sx[2] = enc.z;
    sx[3] = enc.w;
}

// Loads of one row's windows [w0 + wstep * v] into s (x, plus r rounded in) and w,
// with columns outside [0, N) zero. `wend` bounds the windows (slice end or nwin).
template <int DT, int NV, bool NT>
__device__ __forceinline__ void rms_load(uint32_t (&rs)[NV][4], uint32_t (&rw)[NV][4],
                                         const RowGeom<DT>& g, const unsigned char* rrow,
                                         const unsigned char* wvec, const unsigned char* xrow,
                                         int N, int64_t w0, int wstep, int64_t wend, int flags) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t w = w0 + (int64_t)wstep * v;
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (w < wend) raw = load16<NT>(g.base + 16 * (size_t)w);
        rs[v][0] = raw.x;
        rs[v][1] = raw.y;
        rs[v][2] = raw.z;
        rs[v][3] = raw.w;
    }
    // the weight vector's phase against this row decides vector or element loads;
    // weights are shared by every row, so they come from cache after the first rows
    const bool w_phase = ((reinterpret_cast<uintptr_t>(wvec) - reinterpret_cast<uintptr_t>(xrow)) & 15u) == 0;
    load_dy_raw<DT, NV, false>(rw, wvec, g.head, N, w0, wstep, wend, w_phase);
    if (flags & kRmsResidual) {
        uint32_t rr[NV][4];
        load_dy_raw<DT, NV, NT>(rr, rrow, g.head, N, w0, wstep, wend, (flags & kRmsResPhase) != 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) add_round<DT>(rs[v], rr[v]);
    }
    // windows that straddle the row ends hold neighbouring rows' elements (of x, and
    // of r when it was loaded by whole windows): zero them after the sum
    if (g.head != 0 || (N % E) != 0) zero_raw_outside<DT, NV>(rs, g.head, N, w0, wstep);
}

// Lane part of q = sum s^2 (FP32 data: exact products and compensated sums).
template <int DT, int NV>
__device__ __forceinline__ void rms_lane_sq(const uint32_t (&rs)[NV][4], float& acc, CSum& cs) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float f[1][E];
        decode_words<DT>(rs[v], f[0]);
        lane_dot<DT, 1>(f, f, acc, cs);
    }
}

// 1 / sqrt(q / N + eps) from the row's q = hi + lo (IEEE division and square root).
__device__ __forceinline__ float rms_scale(float hi, float lo, int N, float eps) {
    const float q = csum_value(hi, lo);
    return 1.0f / __builtin_sqrtf(q / (float)N + eps);
}

// Write y = s * rstd * w (and s itself) for the lane's windows.
template <int DT, int NV>
__device__ __forceinline__ void rms_store(uint32_t (&rs)[NV][4], const uint32_t (&rw)[NV][4],
                                          float rstd, unsigned char* yrow, unsigned char* srow,
                                          const RowGeom<DT>& g, int N, int64_t w0, int wstep,
                                          int64_t wend, int flags) {
    constexpr int E = Elem<DT>::per_vec;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t w = w0 + (int64_t)wstep * v;
        if (w < wend) {
            if constexpr (DT != kF32) {
                // decode again rather than keep decoded values live across the reduction
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(rs[v][i]));
            }
            if (flags & kRmsSumOut)
                store_window<DT>(srow, make_uint4(rs[v][0], rs[v][1], rs[v][2], rs[v][3]), w, g.head,
                                 N, (flags & kRmsSumPhase) != 0);
            float fs[E], fw[E], o[E];
            decode_words<DT>(rs[v], fs);
            decode_words<DT>(rw[v], fw);
#pragma unroll
            for (int k = 0; k < E; ++k) o[k] = (fs[k] * rstd) * fw[k];
            store_window<DT>(yrow, encode<DT>(o), w, g.head, N, (flags & kRmsOutPhase) != 0);
        }
    }
}

template <int DT, int G, int V, bool NT>
__global__ void __launch_bounds__(RowLaunch<G>::block)
k_rmsnorm_rows(const unsigned char* x, const unsigned char* r, const unsigned char* wvec,
               unsigned char* y, unsigned char* s_out, int64_t M, int N, int64_t x_sb, int64_t r_sb,
               int64_t y_sb, int64_t s_sb, float eps, int flags) {
    constexpr int GPB = RowLaunch<G>::groups;
    constexpr int NW = G > 64 ? G / 64 : 1;
    __shared__ float lds_hi[2][NW], lds_lo[2][NW];  // alternating by row: one barrier per row

    const int tid = threadIdx.x;
    const int lane = (GPB == 1) ? tid : (tid % G);
    const int grp = (GPB == 1) ? 0 : (tid / G);
    const int64_t rstep = (int64_t)gridDim.x * GPB;
    int parity = 0;
    for (int64_t row = xcd_block(flags & kRmsXcdOrder) * GPB + grp; row < M; row += rstep, parity ^= 1) {
        const unsigned char* xrow = x + row * x_sb;
        const RowGeom<DT> g(xrow, N);
        uint32_t rs[V][4], rw[V][4];
        rms_load<DT, V, NT>(rs, rw, g, r + row * r_sb, wvec, xrow, N, lane, G, g.nwin, flags);
        float acc = 0.f;
        CSum cs;
        rms_lane_sq<DT, V>(rs, acc, cs);
        if constexpr (DT == kF32) {
            cs = row_csum<G>(cs, lds_hi[parity], lds_lo[parity]);
        } else {
            cs.hi = row_sum<G>(acc, lds_hi[parity]);
            cs.lo = 0.f;
        }
        const float rstd = rms_scale(cs.hi, cs.lo, N, eps);
        rms_store<DT, V>(rs, rw, rstd, y + row * y_sb, s_out + row * s_sb, g, N, lane, G, g.nwin,
                         flags);
    }
}

// Split fallback after a wait ran out: wave 0's 64 lanes form the row's whole sum of
// squares of s = rn(x + r) from the inputs, element by element (the same rounding of
// the sum, and for FP32 data the same exact products and compensated sums as the
// slices), reduced over the wave.
template <int DT>
__device__ __forceinline__ CSum wave_row_sq(const unsigned char* xrow, const unsigned char* rrow,
                                            int N, int flags) {
    constexpr int ES = Elem<DT>::bytes;
    const int lane = threadIdx.x & 63;
    float acc = 0.f;
    CSum cs;
#pragma unroll 1
    for (int c = lane; c < N; c += 64) {
        float v = load_elem<DT>(xrow + (size_t)c * ES);
        if (flags & kRmsResidual) {
            v = v + load_elem<DT>(rrow + (size_t)c * ES);
            if constexpr (DT != kF32) v = unpack2<DT>(pack2<DT>(v, 0.f)).x;  // one rounding
        }
        if constexpr (DT == kF32) {
            const float pr = v * v;
            cs.add(pr);
            cs.lo += __builtin_fmaf(v, v, -pr);
        } else {
            acc = __builtin_fmaf(v, v, acc);
        }
    }
    if constexpr (DT == kF32) {
        cs = group_allreduce_csum<64>(cs);
    } else {
        cs.hi = group_allreduce<64>(acc, OpAdd{});
        cs.lo = 0.f;
    }
    return cs;
}

// mode 0: publish, wait for the row's slices, apply (one launch); mode 1: publish
// only; mode 2: gather the partials published by an earlier launch and apply (every
// word already carries the tag, so no wait can run out; `sync` may be null).
// The 4-vector instances are held at the 6 waves per SIMD they reach without the
// second launch's gather (80 VGPRs; left to the compiler that path costs them a wave).
template <int V>
constexpr int kRmsSplitWaves = V == 4 ? 6 : 1;

template <int DT, int V, bool NT>
__global__ void __launch_bounds__(kSplitBlock) __attribute__((amdgpu_waves_per_eu(kRmsSplitWaves<V>)))
k_rmsnorm_split(const unsigned char* x, const unsigned char* r, const unsigned char* wvec,
                unsigned char* y, unsigned char* s_out, SplitSlot* slots, SplitSync* sync,
                int64_t M, int N, int64_t x_sb, int64_t r_sb, int64_t y_sb, int64_t s_sb, int P,
                int S, uint32_t tag, int spin_limit, float eps, int flags, int mode) {
    constexpr int B = kSplitBlock;
    __shared__ float lds_hi[B / 64], lds_lo[B / 64];
    __shared__ float lds_stat[4];

    const int lane = threadIdx.x;
    const int64_t items = M * P;
    __shared__ int64_t failed[kSplitMaxDeferred];  // items whose wait ran out (recompute)
    int n_failed = 0;                               // uniform over the workgroup
    // Mode 2 on rows of more than 256 slices reads partials that are all published
    // already: a workgroup sums a row's partials with all its lanes and keeps the total
    // while its items stay in that row (rows of more slices than the grid has
    // workgroups). Shorter rows keep wave 0's gather, one load per lane or two.
    const bool wide_gather = mode == 2 && P > kSplitBlock;
    int64_t have_row = -1;  // wide_gather: the row whose total (q_hi, q_lo, q_ok) is held
    float q_hi = 0.f, q_lo = 0.f;
    bool q_ok = true;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const unsigned char* xrow = x + row * x_sb;
        const RowGeom<DT> g(xrow, N);
        const int64_t w0 = (int64_t)p * S + lane;
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;

        SplitSlot* row_slots = slots + row * P;
        if (wide_gather && row != have_row) {  // before the slice's loads: none of it is live
            const CSum q = split_sum_published<DT == kF32>(row_slots, P, tag, lds_hi, lds_lo, q_ok);
            q_hi = q.hi;
            q_lo = q.lo;
            have_row = row;
        }
        uint32_t rs[V][4], rw[V][4];
        rms_load<DT, V, NT>(rs, rw, g, r + row * r_sb, wvec, xrow, N, w0, B, wend, flags);
        if (mode != 2) {
            float acc = 0.f;
            CSum cs;
            rms_lane_sq<DT, V>(rs, acc, cs);
            if constexpr (DT == kF32) {
                cs = row_csum<B>(cs, lds_hi, lds_lo);
            } else {
                cs.hi = row_sum<B>(acc, lds_hi);
                cs.lo = 0.f;
            }
            if (lane == 0) {
                word_publish(row_slots[p].w + 1, cs.hi, tag);
                if constexpr (DT == kF32) word_publish(row_slots[p].w + 2, cs.lo, tag);
            }
        }
        if (mode == 1) {  // publish only: nothing is written
            __syncthreads();  // the next item's reduction rewrites lds_hi
            continue;
        }
        bool ok;  // uniform over the workgroup
        float rstd;
        if (wide_gather) {
            ok = q_ok;
            rstd = rms_scale(q_hi, q_lo, N, eps);
        } else {
            split_gather_sum<DT == kF32>(row_slots, P, tag, spin_limit, lds_stat);
            __syncthreads();
            ok = lds_stat[3] != 0.f;
            rstd = rms_scale(lds_stat[1], lds_stat[2], N, eps);
        }
        if (!ok) {
            if (lane == 0 && sync) atomicAdd(&sync->failures, 1u);
            if ((flags & kRmsRecompute) && n_failed < kSplitMaxDeferred) {  // written after the loop
                if (lane == 0) failed[n_failed] = item;
                ++n_failed;
                __syncthreads();
                continue;
            }
            rstd = __builtin_nanf("");
        }
        rms_store<DT, V>(rs, rw, rstd, y + row * y_sb, s_out + row * s_sb, g, N, w0, B, wend, flags);
        __syncthreads();  // the next item's gather rewrites lds_stat (wide_gather: lds_hi, lds_lo)
    }
    // Slices whose wait ran out: wave 0 forms the row's sum of squares from the whole
    // input rows, then every lane rewrites its windows of y (and s) from a re-read.
    for (int f = 0; f < n_failed; ++f) {
        const int64_t item = failed[f];
        const int64_t row = item / P;
        const int p = (int)(item - row * P);
        const unsigned char* xrow = x + row * x_sb;
        const RowGeom<DT> g(xrow, N);
        if (lane < 64) {
            const CSum q = wave_row_sq<DT>(xrow, r + row * r_sb, N, flags);
            if (lane == 0) {
                lds_stat[1] = q.hi;
                lds_stat[2] = q.lo;
            }
        }
        __syncthreads();
        const float rstd = rms_scale(lds_stat[1], lds_stat[2], N, eps);
        const int64_t wend = ((int64_t)p * S + S < g.nwin) ? (int64_t)p * S + S : g.nwin;
#pragma unroll 1
        for (int64_t w = (int64_t)p * S + lane; w < wend; w += B) {
            uint32_t fs[1][4], fw[1][4];
            rms_load<DT, 1, NT>(fs, fw, g, r + row * r_sb, wvec, xrow, N, w, 0, wend, flags);
            rms_store<DT, 1>(fs, fw, rstd, y + row * y_sb, s_out + row * s_sb, g, N, w, 0, wend, flags);
        }
        __syncthreads();
    }
}

}  // namespace smx
