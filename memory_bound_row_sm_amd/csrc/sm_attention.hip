// sm_attention.hip -- fused attention forward instances (FP16/BF16 x head dim 64/128 x
// causal or not) and their getter.
#include "sm_attention.hpp"
#include "sm_launch.hpp"

namespace smx {

namespace {
template <int DT, int D>
AttnKernelFn attn_pick_causal(int causal) {
    return causal ? &k_attention_fwd<DT, D, true> : &k_attention_fwd<DT, D, false>;
}

template <int DT>
AttnKernelFn attn_pick_d(int d, int causal) {
    switch (d) {
    case 64: return attn_pick_causal<DT, 64>(causal);
    case 128: return attn_pick_causal<DT, 128>(causal);
    default: return nullptr;
    }
}
}  // namespace

AttnKernelFn attention_kernel(int dtype, int d, int causal) {
    switch (dtype) {
    case 1: return attn_pick_d<1>(d, causal);  // FP16
    case 2: return attn_pick_d<2>(d, causal);  // BF16
    default: return nullptr;
    }
}

}  // namespace smx
