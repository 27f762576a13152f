// sm_launch.hpp -- host-side view of the kernel instances (one table per dtype).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smx {

using RowKernelFn = void (*)(const unsigned char*, unsigned char*, int64_t, int, int64_t, int64_t,
                             int, int);
using StatsKernelFn = void (*)(const unsigned char*, float2*, int64_t, int, int64_t, int, int64_t);
using NormKernelFn = void (*)(const unsigned char*, unsigned char*, const float2*, int64_t, int,
                              int64_t, int64_t, int, int64_t, int);

// Row-kernel instance for (lanes per row G, vectors per lane V, prefetch,
// streaming loads), or nullptr when that combination is not built. Defined per
// dtype in sm_rows_{f32,f16,bf16}.hip.
RowKernelFn row_kernel_f32(int G, int V, int PF, int NT);
RowKernelFn row_kernel_f16(int G, int V, int PF, int NT);
RowKernelFn row_kernel_bf16(int G, int V, int PF, int NT);
StatsKernelFn wide_stats_kernel(int dtype, int NT);
NormKernelFn wide_norm_kernel(int dtype, int NT);

inline RowKernelFn row_kernel(int dtype, int G, int V, int PF, int NT) {
    switch (dtype) {
    case 0: return row_kernel_f32(G, V, PF, NT);
    case 1: return row_kernel_f16(G, V, PF, NT);
    case 2: return row_kernel_bf16(G, V, PF, NT);
    default: return nullptr;
    }
}

// Softmax backward (sm_bwd.hip): one-pass rows for G in {16 ... 1024}, V in
// {1, 2, 4}; two-pass wide rows.
using BwdRowKernelFn = void (*)(const unsigned char*, const unsigned char*, unsigned char*, int64_t,
                                int, int64_t, int64_t, int64_t, int, int, int);
using BwdDotKernelFn = void (*)(const unsigned char*, const unsigned char*, float2*, int64_t, int,
                                int64_t, int64_t, int, int64_t, int);
using BwdApplyKernelFn = void (*)(const unsigned char*, const unsigned char*, unsigned char*,
                                  const float2*, int64_t, int, int64_t, int64_t, int64_t, int,
                                  int64_t, int, int);
BwdRowKernelFn bwd_row_kernel(int dtype, int G, int V, int NT);

// One-launch split kernels (sm_split.hip): 256-lane workgroups, one row slice
// each; the slot and sync pointers are SplitSlot* and SplitSync*.
using SplitKernelFn = void (*)(const unsigned char*, unsigned char*, void*, void*, int64_t, int,
                               int64_t, int64_t, int, int, uint32_t, int, int, int);
using BwdSplitKernelFn = void (*)(const unsigned char*, const unsigned char*, unsigned char*, void*,
                                  void*, int64_t, int, int64_t, int64_t, int64_t, int, int,
                                  uint32_t, int, int, int, int);
SplitKernelFn split_kernel(int dtype, int V, int NT);
BwdSplitKernelFn bwd_split_kernel(int dtype, int V, int NT);

// Residual RMSNorm (sm_rmsnorm.hip): one-pass rows (G in {16 ... 1024}, V in {1, 2, 4})
// and split slices (V in {1, 2, 4}); slot and sync pointers as for the split kernels.
using RmsRowKernelFn = void (*)(const unsigned char*, const unsigned char*, const unsigned char*,
                                unsigned char*, unsigned char*, int64_t, int, int64_t, int64_t,
                                int64_t, int64_t, float, int);
using RmsSplitKernelFn = void (*)(const unsigned char*, const unsigned char*, const unsigned char*,
                                  unsigned char*, unsigned char*, void*, void*, int64_t, int,
                                  int64_t, int64_t, int64_t, int64_t, int, int, uint32_t, int,
                                  float, int, int);
RmsRowKernelFn rms_row_kernel(int dtype, int G, int V, int NT);
RmsSplitKernelFn rms_split_kernel(int dtype, int V, int NT);

// Fused attention forward (sm_attention.hip): FP16/BF16, head dim 64 or 128.
struct AttnArgs;
using AttnKernelFn = void (*)(const AttnArgs);
AttnKernelFn attention_kernel(int dtype, int d, int causal);
BwdDotKernelFn bwd_dot_kernel(int dtype);
BwdApplyKernelFn bwd_apply_kernel(int dtype);

// Threads per workgroup of the row kernel for G lanes per row.
inline int row_block(int G) { return G > 64 ? G : 256; }

}  // namespace smx
