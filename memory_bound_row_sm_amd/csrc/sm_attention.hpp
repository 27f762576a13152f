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
// The next key block's K and V are loaded into registers while the current block
// is computed, and written to the other of two LDS buffers after it (one barrier
// per block).
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
    return is_max ? __builtin_fmaxf(r0, r1) : r0 + r1;
}
__device__ __forceinline__ float attn_xgroup(float x, bool is_max) {
    return attn_swap_op(attn_swap_op(x, is_max, true), is_max, false);
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
k_attention_fwd(const AttnArgs a) {
    constexpr int BN = kAttnBN;
    // LDS row strides (elements), chosen by measured bank conflicts: K rows 16 bytes
    // longer than d (272 B at d = 128: 128-B or 288-B K rows had far more conflicts);
    // V rows 32 bytes longer than d, so that the 4 rows one 16-lane transposed read
    // touches fall on disjoint banks
    constexpr int KS = D + 8;
    constexpr int VR = D + 16;
    constexpr int KCH = D / 8;      // 16-byte chunks per K/V row
    constexpr int LOADS = BN * KCH / kAttnThreads;  // 16-byte chunks per thread per tile
    constexpr int DSUB = D / 16;    // 16-wide d subtiles of the output
    constexpr int KK = D / 32;      // 32-wide d steps of the score product
    constexpr float kInf = __builtin_huge_valf();
    // two K and V tiles (row-major): the next block is staged while the current one is read
    __shared__ __attribute__((aligned(16))) uint16_t ks[2 * BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2 * BN * VR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    // Register staging of one K/V tile: chunk t = tid + 256 * it -> row t / KCH, chunk
    // t % KCH, copied row-major into LDS. Lane offsets inside a tile are 32-bit (row
    // strides are below 2^24 elements), added to the tile's wave-uniform base.
    attn_u4 kreg[LOADS], vreg[LOADS];
    constexpr int KR = kAttnThreads / KCH;  // rows covered by one pass of the threads
    const int krow = tid / KCH, kch = tid % KCH;
    const uint32_t k_lane = (uint32_t)krow * (uint32_t)a.k_rs + (uint32_t)kch * 16u;
    const uint32_t k_step = (uint32_t)KR * (uint32_t)a.k_rs;
    const uint32_t v_lane = (uint32_t)krow * (uint32_t)a.v_rs + (uint32_t)kch * 16u;
    const uint32_t v_step = (uint32_t)KR * (uint32_t)a.v_rs;
    auto fetch = [&](int kb) {
        const unsigned char* kt = kh + (int64_t)kb * a.k_rs;
        const unsigned char* vtile = vh + (int64_t)kb * a.v_rs;
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            attn_u4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
            if (kb + krow + KR * it < a.Sk) {
                zk = *reinterpret_cast<const attn_u4*>(kt + (k_lane + (uint32_t)it * k_step));
                zv = *reinterpret_cast<const attn_u4*>(vtile + (v_lane + (uint32_t)it * v_step));
            }
            kreg[it] = zk;
            vreg[it] = zv;
        }
    };
    auto stage = [&](int buf) {
        uint16_t* kdst = ks + buf * (BN * KS);
        uint16_t* vdst = vs + buf * (BN * VR);
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int r = krow + KR * it;
            *reinterpret_cast<attn_u4*>(&kdst[r * KS + kch * 8]) = kreg[it];
            *reinterpret_cast<attn_u4*>(&vdst[r * VR + kch * 8]) = vreg[it];
        }
    };
    // V^T operand through gfx950's transposed LDS read (ds_read_b64_tr_b16): in each
    // 16-lane group, lane i receives element i % 4 of the 8-byte pieces addressed by
    // lanes 4k + i / 4, k = 0..3. Lane (col, grp) addresses key row key0 + col / 4, d
    // columns dbase + 4 * (col % 4) .. + 3, and so receives V[key0 + k][dbase + col].
    const int vrd = (col >> 2) * VR + 4 * (col & 3);
    auto vt_read = [&](const uint16_t* vtile, int key0, int dbase) -> attn_u2 {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(vtile + key0 * VR + dbase + vrd));
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

        // One barrier per block: after it, every wave has read tile blk and tile blk+1
        // is in LDS; the loads of tile blk+1 are in flight while tile blk is computed.
        if (nblk > 0) {
            fetch(0);
            stage(0);
        }
        __syncthreads();
        for (int blk = 0; blk < nblk; ++blk) {
            const int kb = blk * BN;
            const uint16_t* kcur = ks + (blk & 1) * (BN * KS);
            const uint16_t* vcur = vs + (blk & 1) * (BN * VR);
            if (blk + 1 < nblk) fetch(kb + BN);
            // skipped when every key of the block lies past every query's diagonal for this wave
            if (!(CAUSAL && kb > q0 + 31 + off)) {
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
                        const attn_u4 ka = *reinterpret_cast<const attn_u4*>(&kcur[(t * 16 + col) * KS + kk * 32 + grp * 8]);
#pragma unroll
                        for (int u = 0; u < 2; ++u) s[t][u] = mfma16<DT>(ka, qb[u][kk], s[t][u]);
                    }
                }

                // Blocks cut by the end of the keys or by a diagonal of this wave's queries
                // are scaled and masked element by element (cc = 1 then); all others keep the
                // raw products and fold the scale into the exponent's FMA.
                const bool need_mask = (kb + BN > a.Sk) || (CAUSAL && kb + BN - 1 > q0 + off);
                const float cc = need_mask ? 1.f : c;
                attn_u4 pb[2][2];  // P as the B operand: [u][32-key step]
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (need_mask) {
                        // key kb + grp*4 + (t*16 + i) is visible iff t*16 + i <= lim
                        int lim = a.Sk - 1;
                        if (CAUSAL) lim = min(lim, q0 + u * 16 + col + off);
                        lim -= kb + grp * 4;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                s[t][u][i] = (t * 16 + i > lim) ? -kInf : s[t][u][i] * c;
                    }
                    float bmax = -kInf;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) bmax = __builtin_fmaxf(bmax, s[t][u][i]);
                    bmax = attn_xgroup(bmax, true);
                    bmax *= cc;  // scaled (c >= 0 keeps the order)
                    const bool grow = bmax > m[u] + kAttnLazy;
                    if (__any(grow)) {
                        const float mn = grow ? bmax : m[u];
                        const float sn = (mn == -kInf) ? 0.f : mn;
                        const float alpha = __builtin_amdgcn_exp2f(m[u] - sn);  // m = -inf -> 0
                        m[u] = mn;
                        ms[u] = sn;
                        l[u] *= alpha;
#pragma unroll
                        for (int d = 0; d < DSUB; ++d) oacc[d][u] *= alpha;
                    }
                    float p[4][4];
                    float psum = 0.f;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            p[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][u][i], cc, -ms[u]));
                            psum += p[t][i];
                        }
                    l[u] += psum;
#pragma unroll
                    for (int cs = 0; cs < 2; ++cs) {
                        // 32-key step cs: slots 0..3 <- subtile 2cs, slots 4..7 <- subtile 2cs+1
                        const int t0 = 2 * cs, t1 = 2 * cs + 1;
                        pb[u][cs] = attn_u4{attn_pack2<DT>(p[t0][0], p[t0][1]), attn_pack2<DT>(p[t0][2], p[t0][3]),
                                            attn_pack2<DT>(p[t1][0], p[t1][1]), attn_pack2<DT>(p[t1][2], p[t1][3])};
                    }
                }

                // O^T += V^T P^T: A = V^T rows d, keys in the same slot order as P
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
            }
            if (blk + 1 < nblk) stage((blk + 1) & 1);
            __syncthreads();
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
