// sm_attention.hpp -- gfx950 fused attention forward with the online softmax.
//
// O = softmax(scale * Q K^T [causal]) V per (batch-head, query row), never writing
// the score matrix: the step after the row softmax that "Fused Softmax on GPU"
// names in its closing section, "Wrapping Up" (fusing the online softmax with the
// matmul before it, as FlashAttention does), on the attention-logit workload of the
// same pages.
//
// Tiling. A workgroup of 4 waves owns 128 query rows of one head (32 per wave, two
// 16-row subtiles) and walks the keys in blocks of 64. Contractions run on
// v_mfma_f32_16x16x32 (BF16 or FP16 in, FP32 out). Per key block and wave:
//   S^T = K Q^T   (keys x queries): A = K rows from LDS, B = Q rows held in registers
//                 for the whole kernel; a lane ends with 4 consecutive keys of one
//                 query column, so the row statistics of a query live in one lane
//                 column (lanes l, l^16, l^32, l^48).
//   online softmax: scale, mask, block max across the 4 lane groups, rescale the
//                 running sum and the output, p = exp2(s - m), P rounded to the
//                 input dtype as the B operand of the next product.
//   O^T += V^T P^T (d x queries): A = V^T, read from the row-major V tile in LDS
//                 with gfx950's transposed LDS read; B = P straight from the score
//                 registers. The contraction order
//                 over the 32 keys of an MFMA step is permuted identically on both
//                 operands, so no shuffle of P is needed, and the output tile keeps
//                 the query in the lane column, so the rescale is per lane.
// The next key block's K and V are loaded from global memory straight into the
// other of two LDS buffers while the current block is computed (one barrier per
// block).
//
// Causal masking is aligned to the bottom right: query i sees keys j <= i + Sk - Sq.
// A query that sees no key (Sq > Sk) gets zeros and lse = -inf (the all -inf row
// reading of the softmax). lse (optional, FP32) is the natural log-sum-exp of the
// scaled scores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smx {

template <int DT>
struct AttnElem;
template <>
struct AttnElem<1> {  // FP16
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
};
template <>
struct AttnElem<2> {  // BF16
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
};

typedef float attn_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t attn_u4 __attribute__((ext_vector_type(4)));
typedef uint32_t attn_u2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ attn_f4 mfma16(const attn_u4 a, const attn_u4 b, attn_f4 c) {
    typedef typename AttnElem<DT>::v8 v8;
    if constexpr (DT == 2) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                       __builtin_bit_cast(v8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                      __builtin_bit_cast(v8, b), c, 0, 0, 0);
    }
}

constexpr int kAttnBM = 128;  // query rows per q-block (a workgroup's pass)
constexpr int kAttnBN = 64;   // keys per block
constexpr int kAttnThreads = 256;
constexpr int kAttnXcds = 8;  // MI355X: 8 accelerator dies, each with its own L2
// The running shift of a query row is raised only when a block's maximum exceeds it
// by more than this (log2 units): exponentials stay <= 2^8, and most blocks skip the
// rescale of the output accumulators.
constexpr float kAttnLazy = 8.0f;
// s_waitcnt vmcnt(0) with the other counters at their maxima (gfx9 encoding)
constexpr int kVmcnt0 = 0x0F70;

struct AttnArgs {
    const unsigned char* q;
    const unsigned char* k;
    const unsigned char* v;
    unsigned char* o;
    float* lse;
    int64_t q_rs, q_hs, k_rs, k_hs, v_rs, v_hs, o_rs, o_hs;  // bytes
    int Sq, Sk, qblocks;
    int items;         // work items per head: qblocks, or ceil(qblocks / 2) when causal
    float scale_log2;  // scale * log2(e)
};

// Item of workgroup b out of G: workgroups are handed to the XCDs in turn (b % 8),
// so item ids are laid out to give each XCD one contiguous range of items -- whole
// heads -- whose K and V then stay in that XCD's L2. A bijection for any G.
__device__ __forceinline__ int64_t attn_item(int64_t b, int64_t G) {
    const int64_t x = b % kAttnXcds, j = b / kAttnXcds;
    const int64_t q = G / kAttnXcds, r = G % kAttnXcds;
    return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// Two FP32 values rounded to the dtype (nearest even) and packed, low half = first:
// one v_cvt_pk_{bf16,f16}_f32.
template <int DT>
__device__ __forceinline__ uint32_t attn_pack2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef typename AttnElem<DT>::v2 e2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, e2));
}

// Maximum that propagates NaN (IEEE 754-2019 maximum; v_maximum3_f32 on gfx950). fmaxf
// would make the compiler quiet every MFMA and permlane result first (a v_max_f32 x, x, x
// per input: 28 of the 68 VALU instructions of a block's row maxima at d = 128). A NaN
// score gives a NaN row either way (through its exponential and the row sum).
__device__ __forceinline__ float attn_max(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Max / sum over the 4 lane groups of a lane column (lanes l, l^16, l^32, l^48).
// gfx950's v_permlane32_swap / v_permlane16_swap exchange lanes between two registers:
// given two copies of x they return x and its partner lane l^32 / l^16 (position in the
// row kept), with no LDS traffic. The two results are copied to scalars before the
// bit cast: a bit cast of an element of the returned vector reads element 0.
__device__ __forceinline__ float attn_swap_op(float x, bool is_max, bool half32) {
    const uint32_t a = __builtin_bit_cast(uint32_t, x);
    const auto r = half32 ? __builtin_amdgcn_permlane32_swap(a, a, false, false)
                          : __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const uint32_t u0 = r[0], u1 = r[1];
    const float r0 = __builtin_bit_cast(float, u0), r1 = __builtin_bit_cast(float, u1);
    return is_max ? attn_max(r0, r1) : r0 + r1;
}
__device__ __forceinline__ float attn_xgroup(float x, bool is_max) {
    return attn_swap_op(attn_swap_op(x, is_max, true), is_max, false);
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
k_attention_fwd(const AttnArgs a) {
    constexpr int BN = kAttnBN;
    constexpr int KCH = D / 8;      // 16-byte chunks per K/V row
    constexpr int LOADS = BN * KCH / kAttnThreads;  // 16-byte chunks per thread per tile
    constexpr int DSUB = D / 16;    // 16-wide d subtiles of the output
    constexpr int KK = D / 32;      // 32-wide d steps of the score product
    constexpr float kInf = __builtin_huge_valf();
    // two K and two V tiles of BN rows x d, four separate LDS objects (so that the
    // compiler sees that a block's reads and the next block's loads touch different
    // memory and does not wait for the loads): the next block is loaded while the
    // current one is read. Rows are unpadded; the 16-byte chunks of a row are XOR-swizzled
    // (slot = row * KCH + (chunk ^ f(row))) so that the reads below hit distinct banks:
    // K: 16 lanes read chunk kk*4+grp of rows t*16 + col; V: 16 lanes read 2 chunks of
    // 4 consecutive rows (transposed read).
    __shared__ __attribute__((aligned(16))) uint16_t ks0[BN * D], ks1[BN * D];
    __shared__ __attribute__((aligned(16))) uint16_t vs0[BN * D], vs1[BN * D];
    auto kswz = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
    auto vswz = [](int row) { return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to M0 from SGPRs
    const int col = lane & 15;       // lane column: a query (S^T, O^T) or a key/d row (A ops)
    const int grp = lane >> 4;       // lane group 0..3
    const int off = a.Sk - a.Sq;     // causal: query i sees keys j <= i + off

    const int64_t item = attn_item(blockIdx.x, gridDim.x);
    const int64_t bh = item / a.items;
    const int it0 = (int)(item - bh * a.items);
    // causal: q-blocks it0 and qblocks-1-it0 (heavy one first) share an item, so every
    // item walks about the same number of key blocks
    const int qb_hi = CAUSAL ? a.qblocks - 1 - it0 : it0;
    const int npass = (CAUSAL && it0 < qb_hi) ? 2 : 1;

    const unsigned char* qh = a.q + bh * a.q_hs;
    const unsigned char* kh = a.k + bh * a.k_hs;
    const unsigned char* vh = a.v + bh * a.v_hs;
    // a negative scale is folded into Q's sign (exact), so the score maximum is taken
    // on the unscaled products and scaled once
    const float c = __builtin_fabsf(a.scale_log2);
    const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

    // Tiles go from global memory straight into LDS (global_load_lds_dwordx4): wave w's
    // load instruction `it` fills the 64 consecutive 16-byte slots (it * 4 + w) * 64 ..
    // + 63 of a tile, lane l the slot of that range with index l, so each lane fetches the
    // chunk that the swizzle puts in its slot. Offsets are 32-bit (row strides are below
    // 2^24 elements) from the tile's wave-uniform base. Rows past the last key load the
    // last key's row instead: finite data whose scores are masked and whose weights are 0.
    uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const int slot = (it * 4 + wave) * 64 + lane;
        const int r = slot / KCH, pos = slot % KCH;
        koff[it] = (uint32_t)r * (uint32_t)a.k_rs + (uint32_t)(pos ^ kswz(r)) * 16u;
        voff[it] = (uint32_t)r * (uint32_t)a.v_rs + (uint32_t)(pos ^ vswz(r)) * 16u;
    }
    auto issue = [&](int kb, uint16_t* kdst, uint16_t* vdst) {
        const unsigned char* kt = kh + (int64_t)kb * a.k_rs;
        const unsigned char* vtile = vh + (int64_t)kb * a.v_rs;
        const bool full = kb + BN <= a.Sk;
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            uint32_t ko = koff[it], vo = voff[it];
            if (!full) {
                const int slot = (it * 4 + wave) * 64 + lane;
                const int r = slot / KCH, pos = slot % KCH;
                const uint32_t rr = (uint32_t)min(r, a.Sk - 1 - kb);
                ko = rr * (uint32_t)a.k_rs + (uint32_t)(pos ^ kswz(r)) * 16u;
                vo = rr * (uint32_t)a.v_rs + (uint32_t)(pos ^ vswz(r)) * 16u;
            }
            uint16_t* kd = kdst + (it * 4 + wave) * 64 * 8;
            uint16_t* vd = vdst + (it * 4 + wave) * 64 * 8;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + ko),
                                             (__attribute__((address_space(3))) void*)kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vtile + vo),
                                             (__attribute__((address_space(3))) void*)vd, 16, 0, 0);
        }
    };
    // V^T operand through gfx950's transposed LDS read (ds_read_b64_tr_b16): in each
    // 16-lane group, lane i receives element i % 4 of the 8-byte pieces addressed by
    // lanes 4k + i / 4, k = 0..3. Lane (col, grp) addresses key row key0 + col / 4, d
    // columns dbase + 4 * (col % 4) .. + 3, and so receives V[key0 + k][dbase + col].
    auto vt_read = [&](const uint16_t* vtile, int key0, int dbase) -> attn_u2 {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const int row = key0 + (col >> 2);
        const int chunk = (dbase >> 3) + ((col & 3) >> 1);
        const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(
            vtile + row * D + (chunk ^ vswz(row)) * 8 + (col & 1) * 4));
        return __builtin_bit_cast(attn_u2, r);
    };

    for (int pass = 0; pass < npass; ++pass) {
        const int qblk = pass == 0 ? qb_hi : it0;
        const int q0 = qblk * kAttnBM + wave * 32;  // this wave's first query row

        // Q as the B operand of S^T = K Q^T: lane (col, grp) holds row q0 + u*16 + col,
        // d = kk*32 + grp*8 .. +8 (rows past Sq read as zeros and are never stored)
        attn_u4 qb[2][KK];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int qi = q0 + u * 16 + col;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                attn_u4 z = {0u, 0u, 0u, 0u};
                if (qi < a.Sq) {
                    z = *reinterpret_cast<const attn_u4*>(qh + qi * a.q_rs + (kk * 32 + grp * 8) * 2);
                    z ^= qflip;
                }
                qb[u][kk] = z;
            }
        }

        attn_f4 oacc[DSUB][2];
#pragma unroll
        for (int s = 0; s < DSUB; ++s)
#pragma unroll
            for (int u = 0; u < 2; ++u) oacc[s][u] = attn_f4{0.f, 0.f, 0.f, 0.f};
        float m[2] = {-kInf, -kInf};  // running shift per query (scaled, log2 units)
        float ms[2] = {0.f, 0.f};     // m, or 0 while m = -inf
        float l[2] = {0.f, 0.f};      // this lane group's part of the running sum

        // key range of this q-block (causal: up to its last query's diagonal)
        int kend = a.Sk;
        if (CAUSAL) kend = min(a.Sk, max(0, qblk * kAttnBM + kAttnBM - 1 + off + 1));
        const int nblk = (kend + BN - 1) / BN;

        // One key block of this wave: S^T, online softmax, O^T (kcur, vcur: the tiles).
        auto compute = [&](const uint16_t* kcur, const uint16_t* vcur, int kb) {
            // skipped when every key of the block lies past every query's diagonal for this wave
            if (CAUSAL && kb > q0 + 31 + off) return;
            // S^T tiles: t = key subtile (16 keys), u = query subtile
            attn_f4 s[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u) s[t][u] = attn_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int row = t * 16 + col;
                    const attn_u4 ka = *reinterpret_cast<const attn_u4*>(
                        &kcur[row * D + ((kk * 4 + grp) ^ kswz(row)) * 8]);
#pragma unroll
                    for (int u = 0; u < 2; ++u) s[t][u] = mfma16<DT>(ka, qb[u][kk], s[t][u]);
                }
            }
            if constexpr (D == 128) {
                // d = 128: 4 K fragment reads issued ahead of the MFMAs that use them,
                // then one read per MFMA pair (measured 3% faster; d = 64 was faster
                // with the compiler's own order)
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
                for (int i = 0; i < KK * 4 - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }

            // Blocks cut by the end of the keys or by a diagonal of this wave's queries
            // set their hidden scores to -inf; the scale stays folded into the
            // exponent's FMA (-inf * c - m = -inf). With scale 0 the visible scores are
            // set to 0 instead and the FMA scales by 1 (-inf * 0 would be NaN).
            const bool need_mask = (kb + BN > a.Sk) || (CAUSAL && kb + BN - 1 > q0 + off);
            const bool zero_scale = c == 0.f;
            const float cc = (need_mask && zero_scale) ? 1.f : c;
            if (need_mask) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    // key kb + grp*4 + (t*16 + i) is visible iff t*16 + i <= lim
                    int lim = a.Sk - 1;
                    if (CAUSAL) lim = min(lim, q0 + u * 16 + col + off);
                    lim -= kb + grp * 4;
                    if (zero_scale) {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
#pragma unroll
                            for (int i = 0; i < 4; ++i) s[t][u][i] = (t * 16 + i > lim) ? -kInf : 0.f;
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
#pragma unroll
                            for (int i = 0; i < 4; ++i) s[t][u][i] = (t * 16 + i > lim) ? -kInf : s[t][u][i];
                    }
                }
            }
            // Both subtiles' statistics first (trees, not chains), then one rescale
            // branch for the two, then the exponentials of both in one stretch of code.
            float bmax[2];
            bool grow[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float q4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    q4[t] = attn_max(attn_max(s[t][u][0], s[t][u][1]), attn_max(s[t][u][2], s[t][u][3]));
                bmax[u] = attn_max(attn_max(q4[0], q4[1]), attn_max(q4[2], q4[3]));
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bmax[u] = attn_xgroup(bmax[u], true) * cc;  // scaled (c >= 0 keeps the order)
                grow[u] = bmax[u] > m[u] + kAttnLazy;
            }
            if (__any(grow[0] || grow[1])) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float mn = grow[u] ? bmax[u] : m[u];
                    const float sn = (mn == -kInf) ? 0.f : mn;
                    const float alpha = __builtin_amdgcn_exp2f(m[u] - sn);  // m = -inf -> 0
                    m[u] = mn;
                    ms[u] = sn;
                    l[u] *= alpha;
#pragma unroll
                    for (int d = 0; d < DSUB; ++d) oacc[d][u] *= alpha;
                }
            }
            attn_u4 pb[2][2];  // P as the B operand: [u][32-key step]
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float p[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][u][i], cc, -ms[u]));
                float ps[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) ps[t] = (p[t][0] + p[t][1]) + (p[t][2] + p[t][3]);
                l[u] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
                for (int cs = 0; cs < 2; ++cs) {
                    // 32-key step cs: slots 0..3 <- subtile 2cs, slots 4..7 <- subtile 2cs+1
                    const int t0 = 2 * cs, t1 = 2 * cs + 1;
                    pb[u][cs] = attn_u4{attn_pack2<DT>(p[t0][0], p[t0][1]), attn_pack2<DT>(p[t0][2], p[t0][3]),
                                        attn_pack2<DT>(p[t1][0], p[t1][1]), attn_pack2<DT>(p[t1][2], p[t1][3])};
                }
            }

            // O^T += V^T P^T: A = V^T rows d, keys in the same slot order as P.
            // The wave raises its issue priority for this stretch: its MFMAs go out back
            // to back while the other wave on the SIMD fills the shadow with its softmax
            // VALU work (measured at d = 128: -5% causal 256 x 2048^2, -10% 64 x 4096^2,
            // -2% non-causal; d = 64 unchanged; raising it around the score MFMAs too
            // cost 15% at d = 64 and 1% non-causal).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
#pragma unroll
                for (int d = 0; d < DSUB; ++d) {
                    const attn_u2 lo = vt_read(vcur, (2 * cs) * 16 + grp * 4, d * 16);
                    const attn_u2 hi = vt_read(vcur, (2 * cs + 1) * 16 + grp * 4, d * 16);
                    const attn_u4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int u = 0; u < 2; ++u) oacc[d][u] = mfma16<DT>(va, pb[u][cs], oacc[d][u]);
                }
            }
            if constexpr (D == 128) {
                // transposed V reads (2 per MFMA pair): 8 ahead, then 2 per MFMA pair
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
                for (int i = 0; i < 2 * DSUB - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
            }
            __builtin_amdgcn_s_setprio(0);
        
        };

        // One barrier per block: after it, every wave has read tile blk and tile blk+1
        // is in LDS; the loads of tile blk+1 are in flight while tile blk is computed.
        // Unrolled by two so that each block names its LDS buffers at compile time.
        if (nblk > 0) issue(0, ks0, vs0);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        for (int blk = 0; blk < nblk; blk += 2) {
            const int kb = blk * BN;
            if (blk + 1 < nblk) issue(kb + BN, ks1, vs1);
            compute(ks0, vs0, kb);
            __builtin_amdgcn_s_waitcnt(kVmcnt0);  // this wave's loads of the next tile are in LDS
            __syncthreads();
            if (blk + 1 < nblk) {
                if (blk + 2 < nblk) issue(kb + 2 * BN, ks0, vs0);
                compute(ks1, vs1, kb + BN);
                __builtin_amdgcn_s_waitcnt(kVmcnt0);
                __syncthreads();
            }
        }

        // finish: the full row sum over the 4 lane groups, normalise, store
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float lt = attn_xgroup(l[u], false);
            const int qi = q0 + u * 16 + col;
            if (qi >= a.Sq) continue;
            const float r = (lt > 0.f) ? 1.0f / lt : 0.f;
            unsigned char* orow = a.o + bh * a.o_hs + qi * a.o_rs;
#pragma unroll
            for (int d = 0; d < DSUB; ++d) {
                *reinterpret_cast<attn_u2*>(orow + (d * 16 + grp * 4) * 2) =
                    attn_u2{attn_pack2<DT>(oacc[d][u][0] * r, oacc[d][u][1] * r),
                            attn_pack2<DT>(oacc[d][u][2] * r, oacc[d][u][3] * r)};
            }
            if (a.lse && grp == 0) {
                // natural log-sum-exp of the scaled scores: (shift + log2 l) * ln 2
                a.lse[bh * a.Sq + qi] = (lt > 0.f) ? (ms[u] + __builtin_log2f(lt)) * 0.69314718055994530942f
                                                   : -kInf;
            }
        }
    }
}

}  // namespace smx
