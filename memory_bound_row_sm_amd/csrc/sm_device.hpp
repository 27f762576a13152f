// sm_device.hpp -- device building blocks of the gfx950 row softmax.
//
// Wave64 only. Everything here is register/LDS code for one group of lanes
// that owns one row: 16-byte vector I/O, conversions, DPP reductions, the
// exponential, and the online (max, sum) merge used by the wide path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smx {

enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <int DT>
struct Elem {
    static constexpr int bytes = (DT == kF32) ? 4 : 2;
    static constexpr int per_vec = 16 / bytes;  // elements in one 16-byte vector
    // bit pattern of two (16-bit types) or one (FP32) -inf in a 32-bit word
    static constexpr uint32_t neg_inf_word = (DT == kF32) ? 0xFF800000u
                                           : (DT == kF16) ? 0xFC00FC00u
                                                          : 0xFF80FF80u;
};

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ conversions
// FP16/BF16 -> FP32 is exact. FP32 -> FP16/BF16 rounds to nearest even
// (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950, two elements per op).

template <int DT>
__device__ __forceinline__ f2_t unpack2(uint32_t w) {
    if constexpr (DT == kBF16) {
        return __builtin_convertvector(__builtin_bit_cast(bf2_t, w), f2_t);
    } else {
        return __builtin_convertvector(__builtin_bit_cast(h2_t, w), f2_t);
    }
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f2_t v = {a, b};
    if constexpr (DT == kBF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2_t));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2_t));
    }
}

template <int DT>
__device__ __forceinline__ void decode(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (DT == kF32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(w[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f2_t p = unpack2<DT>(w[k]);
            f[2 * k] = p.x;
            f[2 * k + 1] = p.y;
        }
    }
}

template <int DT>
__device__ __forceinline__ uint4 encode(const float* f) {
    uint32_t w[4];
    if constexpr (DT == kF32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = __float_as_uint(f[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack2<DT>(f[2 * k], f[2 * k + 1]);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------ 16-byte global I/O
// Row data moves in 16-byte vectors. NT selects the nontemporal (streaming)
// load hint; it is a template parameter because the compiler merges two loads
// that differ only in their cache hint into one plain load.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load16(const unsigned char* p) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    u32x4_t v;
    if constexpr (NT)
        v = __builtin_nontemporal_load(q);
    else
        v = *q;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Output vectors are stored with device scope (sc1). Each XCD has its own L2, so a
// device-scope store writes through it: when the dispatch ends, its release finds no
// dirty output lines to write back. Measured cold on MI355X against plain stores:
// BF16 4096 x 4096 softmax 12.11 -> 11.80 us, FP16 8192 x 2048 -8%, BF16 64 x 131072
// (SPLIT) -16%, 158 plan/workload cells -2.4% geomean; nontemporal stores were 6-12%
// slower. No builtin emits a 16-byte global store with a scope bit, hence the asm;
// the compiler-visible alternative, two 8-byte relaxed device-scope atomic stores per
// vector, writes half lines through the L2 and ran 2.2-2.7x slower on every large
// shape (BF16 4096 x 4096 11.8 -> 27.5 us, causal 524288 x 2048 617 -> 1443 us).
// A store of more than 8 bytes reads its data VGPRs after it issues, and a VALU
// write of those VGPRs must wait two wait states (gfx940 and later). The compiler
// pads its own stores for this but cannot see inside an asm block, so the block
// carries its own s_nop 1; without it, FP32 RMSNorm's residual output took the next
// multiply's result.
__device__ __forceinline__ void store16(unsigned char* p, const uint4 v) {
    const u32x4_t w = u32x4_t{v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(w) : "memory");
}

// Load one stored element and decode it exactly to FP32.
template <int DT>
__device__ __forceinline__ float load_elem(const unsigned char* p) {
    if constexpr (DT == kF32) {
        return *reinterpret_cast<const float*>(p);
    } else if constexpr (DT == kBF16) {
        return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(p));
    }
}

// Store one element (already encoded) of an encoded vector: element k of `v`.
template <int DT>
__device__ __forceinline__ void store_elem(unsigned char* p, const uint4 v, int k) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (DT == kF32) {
        *reinterpret_cast<uint32_t*>(p) = w[k];
    } else {
        const uint32_t word = w[k >> 1];
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)((k & 1) ? (word >> 16) : word);
    }
}

// ------------------------------------------------------------ lane max
// Row maxima use the NaN-propagating maximum (IEEE 754-2019; v_maximum3_f32 on gfx950,
// two elements per instruction). fmaxf would make the compiler quiet every input that
// it cannot prove canonical first (decoded 16-bit values, DPP and LDS results): one
// v_max_f32 x, x, x each. A NaN makes its row NaN either way (through its exponential
// and the row sum).
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmax_nan(fmax_nan(a, b), c); }

// ------------------------------------------------------------ DPP / swizzle
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor16(float v) {
    // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 (within 32 lanes)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float readlane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;     // lane i <- 15 - i within 16 lanes
constexpr int kRowHalfMirror = 0x141; // lane i <- 7 - i within 8 lanes

// All-reduce over aligned groups of G lanes (G = 16, 32 or 64) of one wave.
// Every lane of a group ends with bitwise the same value: each step combines a
// lane with a partner that holds bitwise the same partial as the partner's
// partner (quad xor, mirror, half mirror, swizzle xor 16), and `op` is
// commutative; the last 64-lane step is evaluated once from two lanes.
template <int G, class Op>
__device__ __forceinline__ float group_allreduce(float v, Op op) {
    static_assert(G == 16 || G == 32 || G == 64, "group of 16, 32 or 64 lanes");
    v = op(v, dpp<kQuadXor1>(v));
    v = op(v, dpp<kQuadXor2>(v));
    v = op(v, dpp<kRowMirror>(v));
    v = op(v, dpp<kRowHalfMirror>(v));
    if constexpr (G >= 32) v = op(v, swz_xor16(v));
    if constexpr (G == 64) v = op(readlane(v, 0), readlane(v, 32));
    return v;
}

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmax_nan(a, b); }
};
struct OpAdd {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// ------------------------------------------------------------ exponentials
// Fast path (FP16/BF16 outputs): e = 2^(x*log2e - m*log2e), one FMA and one
// v_exp_f32. The rounding of m*log2e shifts every exponent of the row by the
// same amount and cancels in the normalisation.
__device__ __forceinline__ float exp2_fast(float t) { return __builtin_amdgcn_exp2f(t); }

// Error-free sum (Knuth TwoSum): a + b = s + e exactly, s = fl(a + b).
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// Accurate exp(x - m) for FP32 outputs: d = fl(x - m) with its exact rounding
// error dlo (TwoSum), e = expf(d) (the device library's correctly reduced
// exponential), then e * (1 + dlo) to first order. -inf - m gives exactly 0.
__device__ __forceinline__ float exp_diff_acc(float x, float m) {
    float d, dlo;
    two_sum(x, -m, d, dlo);
    const float e = __builtin_expf(d);
    return (dlo == dlo) ? __builtin_fmaf(e, dlo, e) : e;
}

// Compensated accumulator (sum = hi + lo).
struct CSum {
    float hi = 0.f, lo = 0.f;
    __device__ __forceinline__ void add(float v) {
        float s, e;
        two_sum(hi, v, s, e);
        hi = s;
        lo += e;
    }
};

// All-reduce of a compensated pair over a group of G lanes; same pairing as
// group_allreduce. TwoSum's error term is exact, hence symmetric, so partners
// stay bitwise equal.
template <int G>
__device__ __forceinline__ CSum group_allreduce_csum(CSum c) {
    auto step = [](CSum a, float bh, float bl) {
        CSum r;
        float e;
        two_sum(a.hi, bh, r.hi, e);
        r.lo = (a.lo + bl) + e;
        return r;
    };
    c = step(c, dpp<kQuadXor1>(c.hi), dpp<kQuadXor1>(c.lo));
    c = step(c, dpp<kQuadXor2>(c.hi), dpp<kQuadXor2>(c.lo));
    c = step(c, dpp<kRowMirror>(c.hi), dpp<kRowMirror>(c.lo));
    c = step(c, dpp<kRowHalfMirror>(c.hi), dpp<kRowHalfMirror>(c.lo));
    if constexpr (G >= 32) c = step(c, swz_xor16(c.hi), swz_xor16(c.lo));
    if constexpr (G == 64) {
        CSum a;
        a.hi = readlane(c.hi, 0);
        a.lo = readlane(c.lo, 0);
        c = step(a, readlane(c.hi, 32), readlane(c.lo, 32));
    }
    return c;
}

// ------------------------------------------------------------ online merge
// Merge of two partial states (m, s), s = sum exp(x - m) over each part. A part
// whose maximum is -inf (all of it masked) contributes nothing, and two such
// parts keep the sum of their sums (0, or NaN if a NaN was seen) without
// evaluating exp(-inf - (-inf)) ("Measured optimization case studies", section
// "Wide rows: loop in one program, or split across programs": the merge guard).
__device__ __forceinline__ void merge_fast(float& m, float& s, float m2, float s2) {
    const float mn = fmax_nan(m, m2);
    const float r = s * exp2_fast((m - mn) * kLog2e) + s2 * exp2_fast((m2 - mn) * kLog2e);
    s = (mn == kNegInf) ? s + s2 : r;
    m = mn;
}

// FP32-accurate merge: rescale factors from exp_diff_acc, compensated sums.
__device__ __forceinline__ void merge_acc(float& m, CSum& s, float m2, CSum s2) {
    const float mn = fmax_nan(m, m2);
    if (mn == kNegInf) {  // both parts fully masked: 0, or NaN if a NaN was seen
        s.hi = s.hi + s2.hi;
        s.lo = s.lo + s2.lo;
        m = mn;
        return;
    }
    const float fa = exp_diff_acc(m, mn);   // m = -inf -> 0
    const float fb = exp_diff_acc(m2, mn);
    const float ah = s.hi * fa, al = s.lo * fa;
    const float bh = s2.hi * fb, bl = s2.lo * fb;
    CSum r;
    float e;
    two_sum(ah, bh, r.hi, e);
    r.lo = (al + bl) + e;
    s = r;
    m = mn;
}

template <int G>
__device__ __forceinline__ void group_merge_fast(float& m, float& s) {
    static_assert(G == 64, "wide-path merge runs over whole waves");
    auto stepd = [&](float m2, float s2) { merge_fast(m, s, m2, s2); };
    stepd(dpp<kQuadXor1>(m), dpp<kQuadXor1>(s));
    stepd(dpp<kQuadXor2>(m), dpp<kQuadXor2>(s));
    stepd(dpp<kRowMirror>(m), dpp<kRowMirror>(s));
    stepd(dpp<kRowHalfMirror>(m), dpp<kRowHalfMirror>(s));
    stepd(swz_xor16(m), swz_xor16(s));
    float ma = readlane(m, 0), sa = readlane(s, 0);
    merge_fast(ma, sa, readlane(m, 32), readlane(s, 32));
    m = ma;
    s = sa;
}

template <int G>
__device__ __forceinline__ void group_merge_acc(float& m, CSum& s) {
    static_assert(G == 64, "wide-path merge runs over whole waves");
    auto stepd = [&](float m2, float h2, float l2) {
        CSum o;
        o.hi = h2;
        o.lo = l2;
        merge_acc(m, s, m2, o);
    };
    stepd(dpp<kQuadXor1>(m), dpp<kQuadXor1>(s.hi), dpp<kQuadXor1>(s.lo));
    stepd(dpp<kQuadXor2>(m), dpp<kQuadXor2>(s.hi), dpp<kQuadXor2>(s.lo));
    stepd(dpp<kRowMirror>(m), dpp<kRowMirror>(s.hi), dpp<kRowMirror>(s.lo));
    stepd(dpp<kRowHalfMirror>(m), dpp<kRowHalfMirror>(s.hi), dpp<kRowHalfMirror>(s.lo));
    stepd(swz_xor16(m), swz_xor16(s.hi), swz_xor16(s.lo));
    float ma = readlane(m, 0);
    CSum sa, sb;
    sa.hi = readlane(s.hi, 0);
    sa.lo = readlane(s.lo, 0);
    sb.hi = readlane(s.hi, 32);
    sb.lo = readlane(s.lo, 32);
    merge_acc(ma, sa, readlane(m, 32), sb);
    m = ma;
    s = sa;
}

}  // namespace smx
