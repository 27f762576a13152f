// sm_bwd.hip -- softmax-backward kernel instances (all dtypes) and their getters.
#include "sm_bwd.hpp"
#include "sm_launch.hpp"

namespace smx {

namespace {
// Streaming-load (NT) instances exist for the multi-wave shapes (G >= 128).
template <int DT, int G, int V>
BwdRowKernelFn bwd_pick_nt(int NT) {
    if (NT) {
        if constexpr (G >= 128) return &k_softmax_bwd_rows<DT, G, V, true>;
        return nullptr;
    }
    return &k_softmax_bwd_rows<DT, G, V, false>;
}

template <int DT, int G>
BwdRowKernelFn bwd_pick_v(int V, int NT) {
    switch (V) {
    case 1: return bwd_pick_nt<DT, G, 1>(NT);
    case 2: return bwd_pick_nt<DT, G, 2>(NT);
    case 4: return bwd_pick_nt<DT, G, 4>(NT);
    default: return nullptr;
    }
}

template <int DT>
BwdRowKernelFn bwd_pick(int G, int V, int NT) {
    switch (G) {
    case 16: return bwd_pick_v<DT, 16>(V, NT);
    case 32: return bwd_pick_v<DT, 32>(V, NT);
    case 64: return bwd_pick_v<DT, 64>(V, NT);
    case 128: return bwd_pick_v<DT, 128>(V, NT);
    case 256: return bwd_pick_v<DT, 256>(V, NT);
    case 512: return bwd_pick_v<DT, 512>(V, NT);
    case 1024: return bwd_pick_v<DT, 1024>(V, NT);
    default: return nullptr;
    }
}
}  // namespace

BwdRowKernelFn bwd_row_kernel(int dtype, int G, int V, int NT) {
    switch (dtype) {
    case kF32: return bwd_pick<kF32>(G, V, NT);
    case kF16: return bwd_pick<kF16>(G, V, NT);
    case kBF16: return bwd_pick<kBF16>(G, V, NT);
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
