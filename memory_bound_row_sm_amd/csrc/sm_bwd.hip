// sm_bwd.hip -- softmax-backward kernel instances (all dtypes) and their getters.
#include "sm_bwd.hpp"
#include "sm_launch.hpp"

namespace smx {

namespace {
template <int DT, int G>
BwdRowKernelFn bwd_pick_v(int V) {
    switch (V) {
    case 1: return &k_softmax_bwd_rows<DT, G, 1>;
    case 2: return &k_softmax_bwd_rows<DT, G, 2>;
    case 4: return &k_softmax_bwd_rows<DT, G, 4>;
    default: return nullptr;
    }
}

template <int DT>
BwdRowKernelFn bwd_pick(int G, int V) {
    switch (G) {
    case 16: return bwd_pick_v<DT, 16>(V);
    case 32: return bwd_pick_v<DT, 32>(V);
    case 64: return bwd_pick_v<DT, 64>(V);
    case 128: return bwd_pick_v<DT, 128>(V);
    case 256: return bwd_pick_v<DT, 256>(V);
    case 512: return bwd_pick_v<DT, 512>(V);
    case 1024: return bwd_pick_v<DT, 1024>(V);
    default: return nullptr;
    }
}
}  // namespace

BwdRowKernelFn bwd_row_kernel(int dtype, int G, int V) {
    switch (dtype) {
    case kF32: return bwd_pick<kF32>(G, V);
    case kF16: return bwd_pick<kF16>(G, V);
    case kBF16: return bwd_pick<kBF16>(G, V);
    default: return nullptr;
    }
}

BwdDotKernelFn bwd_dot_kernel(int dtype) {
    switch (dtype) {
    case kF32: return &k_bwd_wide_dot<kF32>;
    case kF16: return &k_bwd_wide_dot<kF16>;
    case kBF16: return &k_bwd_wide_dot<kBF16>;
    default: return nullptr;
    }
}

BwdApplyKernelFn bwd_apply_kernel(int dtype) {
    switch (dtype) {
    case kF32: return &k_bwd_wide_apply<kF32>;
    case kF16: return &k_bwd_wide_apply<kF16>;
    case kBF16: return &k_bwd_wide_apply<kBF16>;
    default: return nullptr;
    }
}

}  // namespace smx
