// sm_rows_inst.inl -- instantiates the row kernels of one dtype (SM_DT) and
// returns them through a switch. Included by sm_rows_{f32,f16,bf16}.hip.
//
// Built combinations: G in {16, 32, 64, 128, 256} with V in {1, 2, 4, 8} and
// prefetch on or off; G in {512, 1024} with V in {1, 2, 4, 8}, no prefetch.
#include "sm_kernels.hpp"
#include "sm_launch.hpp"

namespace smx {

namespace {
template <int G, int V>
RowKernelFn pick_pf(int PF) {
    if (PF) {
        if constexpr (G <= 256) return &k_softmax_rows<SM_DT, G, V, true>;
        return nullptr;
    }
    return &k_softmax_rows<SM_DT, G, V, false>;
}

template <int G>
RowKernelFn pick_v(int V, int PF) {
    switch (V) {
    case 1: return pick_pf<G, 1>(PF);
    case 2: return pick_pf<G, 2>(PF);
    case 4: return pick_pf<G, 4>(PF);
    case 8: return pick_pf<G, 8>(PF);
    default: return nullptr;
    }
}
}  // namespace

RowKernelFn SM_ROW_FN(int G, int V, int PF) {
    switch (G) {
    case 16: return pick_v<16>(V, PF);
    case 32: return pick_v<32>(V, PF);
    case 64: return pick_v<64>(V, PF);
    case 128: return pick_v<128>(V, PF);
    case 256: return pick_v<256>(V, PF);
    case 512: return pick_v<512>(V, PF);
    case 1024: return pick_v<1024>(V, PF);
    default: return nullptr;
    }
}

}  // namespace smx
