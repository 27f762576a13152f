// sm_attention.hpp -- gfx950 fused attention forward with the online softmax.
//
// O = softmax(scale * Q K^T [causal]) V per (batch-head, query row), never writing
// the score matrix: the step after the row softmax that "Fused Softmax on GPU"
// names in its closing section (fusing the online softmax with the matmul before
// it, as FlashAttention does), on the attention-logit workload of the same pages.
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
//   O^T += V^T P^T (d x queries): A = V^T from LDS (V is stored transposed in LDS),
//                 B = P straight from the score registers. The contraction order
//                 over the 32 keys of an MFMA step is permuted identically on both
//                 operands, so no shuffle of P is needed, and the output tile keeps
//                 the query in the lane column, so the rescale is per lane.
// The next key block's K and V are loaded into registers while the current block
// is computed, and written to LDS after it (one buffer, two barriers per block).
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
    static __device__ __forceinline__ uint16_t bits(float f) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
};
template <>
struct AttnElem<2> {  // BF16
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ uint16_t bits(float f) {
        return __builtin_bit_cast(uint16_t, (__bf16)f);
    }
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

constexpr int kAttnBM = 128;  // query rows per workgroup
constexpr int kAttnBN = 64;   // keys per block
constexpr int kAttnThreads = 256;

struct AttnArgs {
    const unsigned char* q;
    const unsigned char* k;
    const unsigned char* v;
    unsigned char* o;
    float* lse;
    int64_t q_rs, q_hs, k_rs, k_hs, v_rs, v_hs, o_rs, o_hs;  // bytes
    int Sq, Sk, qblocks;
    float scale_log2;  // scale * log2(e)
};

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(kAttnThreads)
k_attention_fwd(const AttnArgs a) {
    constexpr int BN = kAttnBN;
    constexpr int KS = D + 8;       // K row stride in LDS (elements): 16-byte pad
    constexpr int VS = BN + 8;      // V^T row stride in LDS (elements)
    constexpr int KCH = D / 8;      // 16-byte chunks per K/V row
    constexpr int LOADS = BN * KCH / kAttnThreads;  // 16-byte chunks per thread per tile
    constexpr int DSUB = D / 16;    // 16-wide d subtiles of the output
    constexpr int KK = D / 32;      // 32-wide d steps of the score product
    __shared__ uint16_t ks[BN * KS];
    __shared__ uint16_t vt[D * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;       // lane column: a query (S^T, O^T) or a key/d row (A ops)
    const int grp = lane >> 4;       // lane group 0..3
    const int64_t bh = blockIdx.x / a.qblocks;
    const int q0 = (int)(blockIdx.x % a.qblocks) * kAttnBM + wave * 32;
    const int off = a.Sk - a.Sq;     // causal: query i sees keys j <= i + off

    const unsigned char* qh = a.q + bh * a.q_hs;
    const unsigned char* kh = a.k + bh * a.k_hs;
    const unsigned char* vh = a.v + bh * a.v_hs;

    // Q as the B operand of S^T = K Q^T: lane (col, grp) holds row q0 + u*16 + col,
    // d = kk*32 + grp*8 .. +8 (rows past Sq read as zeros and are never stored)
    attn_u4 qb[2][KK];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qi = q0 + u * 16 + col;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            attn_u4 z = {0u, 0u, 0u, 0u};
            if (qi < a.Sq) z = *reinterpret_cast<const attn_u4*>(qh + qi * a.q_rs + (kk * 32 + grp * 8) * 2);
            qb[u][kk] = z;
        }
    }

    attn_f4 oacc[DSUB][2];
#pragma unroll
    for (int s = 0; s < DSUB; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u) oacc[s][u] = attn_f4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
    float l[2] = {0.f, 0.f};  // this lane group's part of the running sum

    // key range of this workgroup (causal: up to the last query's diagonal)
    const int qlast = (int)(blockIdx.x % a.qblocks) * kAttnBM + kAttnBM - 1;
    int kend = a.Sk;
    if (CAUSAL) kend = min(a.Sk, max(0, qlast + off + 1));
    const int nblk = (kend + BN - 1) / BN;

    // register staging of one K/V tile: chunk c = tid + 256 * it -> row c / KCH, chunk c % KCH
    attn_u4 kreg[LOADS], vreg[LOADS];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int c = tid + kAttnThreads * it;
            const int r = kb + c / KCH, ch = c % KCH;
            attn_u4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
            if (r < a.Sk) {
                zk = *reinterpret_cast<const attn_u4*>(kh + r * a.k_rs + ch * 16);
                zv = *reinterpret_cast<const attn_u4*>(vh + r * a.v_rs + ch * 16);
            }
            kreg[it] = zk;
            vreg[it] = zv;
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int c = tid + kAttnThreads * it;
            const int r = c / KCH, ch = c % KCH;
            *reinterpret_cast<attn_u4*>(&ks[r * KS + ch * 8]) = kreg[it];
            // V transposed: element e of the chunk is V[r][ch*8 + e] -> vt[ch*8 + e][r]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = vreg[it][e];
                vt[(ch * 8 + 2 * e) * VS + r] = (uint16_t)(w & 0xFFFFu);
                vt[(ch * 8 + 2 * e + 1) * VS + r] = (uint16_t)(w >> 16);
            }
        }
    };

    if (nblk > 0) fetch(0);
    for (int blk = 0; blk < nblk; ++blk) {
        const int kb = blk * BN;
        __syncthreads();  // every wave is done reading the previous tile
        stage();
        __syncthreads();
        if (blk + 1 < nblk) fetch(kb + BN);  // next tile in flight during this one

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
                const attn_u4 ka = *reinterpret_cast<const attn_u4*>(&ks[(t * 16 + col) * KS + kk * 32 + grp * 8]);
#pragma unroll
                for (int u = 0; u < 2; ++u) s[t][u] = mfma16<DT>(ka, qb[u][kk], s[t][u]);
            }
        }

        // online softmax on the lane's 16 keys of each query column
        attn_u4 pb[2][2];  // P as the B operand: [u][32-key step]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int qi = q0 + u * 16 + col;
            float bmax = -__builtin_huge_valf();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kj = kb + t * 16 + grp * 4 + i;
                    float x = s[t][u][i] * a.scale_log2;
                    const bool masked = kj >= a.Sk || (CAUSAL && kj > qi + off);
                    x = masked ? -__builtin_huge_valf() : x;
                    s[t][u][i] = x;
                    bmax = __builtin_fmaxf(bmax, x);
                }
            }
            bmax = __builtin_fmaxf(bmax, __shfl_xor(bmax, 16));
            bmax = __builtin_fmaxf(bmax, __shfl_xor(bmax, 32));
            const float mn = __builtin_fmaxf(m[u], bmax);
            // a query with no visible key so far keeps shift 0 and sum 0
            const float ms = (mn == -__builtin_huge_valf()) ? 0.f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[u] - ms);  // m = -inf -> 0
            m[u] = mn;
            float psum = 0.f;
            float p[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[t][i] = __builtin_amdgcn_exp2f(s[t][u][i] - ms);
                    psum += p[t][i];
                }
            l[u] = l[u] * alpha + psum;
#pragma unroll
            for (int d = 0; d < DSUB; ++d) oacc[d][u] *= alpha;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // 32-key step c: slots 0..3 <- subtile 2c, slots 4..7 <- subtile 2c+1
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = 2 * c + h;
                    w[2 * h] = (uint32_t)AttnElem<DT>::bits(p[t][0]) |
                               ((uint32_t)AttnElem<DT>::bits(p[t][1]) << 16);
                    w[2 * h + 1] = (uint32_t)AttnElem<DT>::bits(p[t][2]) |
                                   ((uint32_t)AttnElem<DT>::bits(p[t][3]) << 16);
                }
                pb[u][c] = attn_u4{w[0], w[1], w[2], w[3]};
            }
        }

        // O^T += V^T P^T: A = V^T rows d, keys in the same slot order as P
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int d = 0; d < DSUB; ++d) {
                const uint16_t* vrow = &vt[(d * 16 + col) * VS];
                const attn_u2 lo = *reinterpret_cast<const attn_u2*>(vrow + (2 * c) * 16 + grp * 4);
                const attn_u2 hi = *reinterpret_cast<const attn_u2*>(vrow + (2 * c + 1) * 16 + grp * 4);
                const attn_u4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int u = 0; u < 2; ++u) oacc[d][u] = mfma16<DT>(va, pb[u][c], oacc[d][u]);
            }
        }
    }

    // finish: the full row sum over the 4 lane groups, normalise, store
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float lt = l[u];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int qi = q0 + u * 16 + col;
        if (qi >= a.Sq) continue;
        const float r = (lt > 0.f) ? 1.0f / lt : 0.f;
        unsigned char* orow = a.o + bh * a.o_hs + qi * a.o_rs;
#pragma unroll
        for (int d = 0; d < DSUB; ++d) {
            const uint32_t w0 = (uint32_t)AttnElem<DT>::bits(oacc[d][u][0] * r) |
                                ((uint32_t)AttnElem<DT>::bits(oacc[d][u][1] * r) << 16);
            const uint32_t w1 = (uint32_t)AttnElem<DT>::bits(oacc[d][u][2] * r) |
                                ((uint32_t)AttnElem<DT>::bits(oacc[d][u][3] * r) << 16);
            *reinterpret_cast<attn_u2*>(orow + (d * 16 + grp * 4) * 2) = attn_u2{w0, w1};
        }
        if (a.lse && grp == 0) {
            // natural log-sum-exp of the scaled scores: (m + log2 l) * ln 2
            a.lse[bh * a.Sq + qi] = (lt > 0.f) ? (m[u] + __builtin_log2f(lt)) * 0.69314718055994530942f
                                               : -__builtin_huge_valf();
        }
    }
}

}  // namespace smx
