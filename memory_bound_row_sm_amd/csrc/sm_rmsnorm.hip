// sm_rmsnorm.hip -- residual-RMSNorm kernel instances (all dtypes) and getters:
// one-pass rows for G in {16 ... 1024}, V in {1, 2, 4} (streaming loads for the
// multi-wave shapes), split slices for V in {1, 2, 4}.
#include "sm_launch.hpp"
#include "sm_rmsnorm.hpp"

namespace smx {

namespace {
template <int DT, int G, int V>
RmsRowKernelFn rms_pick_nt(int NT) {
    if (NT) {
        if constexpr (G >= 128) return &k_rmsnorm_rows<DT, G, V, true>;
        return nullptr;
    }
    return &k_rmsnorm_rows<DT, G, V, false>;
}

template <int DT, int G>
RmsRowKernelFn rms_pick_v(int V, int NT) {
    switch (V) {
    case 1: return rms_pick_nt<DT, G, 1>(NT);
    case 2: return rms_pick_nt<DT, G, 2>(NT);
    case 4: return rms_pick_nt<DT, G, 4>(NT);
    default: return nullptr;
    }
}

template <int DT>
RmsRowKernelFn rms_pick(int G, int V, int NT) {
    switch (G) {
    case 16: return rms_pick_v<DT, 16>(V, NT);
    case 32: return rms_pick_v<DT, 32>(V, NT);
    case 64: return rms_pick_v<DT, 64>(V, NT);
    case 128: return rms_pick_v<DT, 128>(V, NT);
    case 256: return rms_pick_v<DT, 256>(V, NT);
    case 512: return rms_pick_v<DT, 512>(V, NT);
    case 1024: return rms_pick_v<DT, 1024>(V, NT);
    default: return nullptr;
    }
}

template <int DT, int V>
RmsSplitKernelFn rms_split_pick_nt(int NT) {
    if (NT) return reinterpret_cast<RmsSplitKernelFn>(&k_rmsnorm_split<DT, V, true>);
    return reinterpret_cast<RmsSplitKernelFn>(&k_rmsnorm_split<DT, V, false>);
}

template <int DT>
RmsSplitKernelFn rms_split_pick(int V, int NT) {
    switch (V) {
    case 1: return rms_split_pick_nt<DT, 1>(NT);
    case 2: return rms_split_pick_nt<DT, 2>(NT);
    case 4: return rms_split_pick_nt<DT, 4>(NT);
    default: return nullptr;
    }
}
}  // namespace

RmsRowKernelFn rms_row_kernel(int dtype, int G, int V, int NT) {
    switch (dtype) {
    case kF32: return rms_pick<kF32>(G, V, NT);
    case kF16: return rms_pick<kF16>(G, V, NT);
    case kBF16: return rms_pick<kBF16>(G, V, NT);
    default: return nullptr;
    }
}

RmsSplitKernelFn rms_split_kernel(int dtype, int V, int NT) {
    switch (dtype) {
    case kF32: return rms_split_pick<kF32>(V, NT);
    case kF16: return rms_split_pick<kF16>(V, NT);
    case kBF16: return rms_split_pick<kBF16>(V, NT);
    default: return nullptr;
    }
}

}  // namespace smx
