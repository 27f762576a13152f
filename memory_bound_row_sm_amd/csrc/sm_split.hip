// sm_split.hip -- instances of the one-launch split kernels (forward V in
// {1, 2, 4, 8}, backward V in {1, 2, 4}; cached or streaming loads) and getters.
#include "sm_launch.hpp"
#include "sm_split.hpp"

namespace smx {

namespace {
template <int DT, int V>
SplitKernelFn split_pick_nt(int NT) {
    if (NT) return reinterpret_cast<SplitKernelFn>(&k_softmax_split<DT, V, true>);
    return reinterpret_cast<SplitKernelFn>(&k_softmax_split<DT, V, false>);
}

template <int DT>
SplitKernelFn split_pick(int V, int NT) {
    switch (V) {
    case 1: return split_pick_nt<DT, 1>(NT);
    case 2: return split_pick_nt<DT, 2>(NT);
    case 4: return split_pick_nt<DT, 4>(NT);
    case 8: return split_pick_nt<DT, 8>(NT);
    default: return nullptr;
    }
}

template <int DT, int V>
BwdSplitKernelFn bwd_split_pick_nt(int NT) {
    if (NT) return reinterpret_cast<BwdSplitKernelFn>(&k_softmax_bwd_split<DT, V, true>);
    return reinterpret_cast<BwdSplitKernelFn>(&k_softmax_bwd_split<DT, V, false>);
}

template <int DT>
BwdSplitKernelFn bwd_split_pick(int V, int NT) {
    switch (V) {
    case 1: return bwd_split_pick_nt<DT, 1>(NT);
    case 2: return bwd_split_pick_nt<DT, 2>(NT);
    case 4: return bwd_split_pick_nt<DT, 4>(NT);
    default: return nullptr;
    }
}
}  // namespace

SplitKernelFn split_kernel(int dtype, int V, int NT) {
    switch (dtype) {
    case kF32: return split_pick<kF32>(V, NT);
    case kF16: return split_pick<kF16>(V, NT);
    case kBF16: return split_pick<kBF16>(V, NT);
    default: return nullptr;
    }
}

BwdSplitKernelFn bwd_split_kernel(int dtype, int V, int NT) {
    switch (dtype) {
    case kF32: return bwd_split_pick<kF32>(V, NT);
    case kF16: return bwd_split_pick<kF16>(V, NT);
    case kBF16: return bwd_split_pick<kBF16>(V, NT);
    default: return nullptr;
    }
}

}  // namespace smx
