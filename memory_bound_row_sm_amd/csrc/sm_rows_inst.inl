// sm_rows_inst.inl -- instantiates the row kernels of one dtype (SM_DT) and
// returns them through a switch. Included by sm_rows_{f32,f16,bf16}.hip.
//
// Built combinations: G in {16, 32, 64, 128, 256} with V in {1, 2, 4, 8} and
// prefetch on or off; G in {512, 1024} with V in {1, 2, 4, 8}, no prefetch.
// Streaming-load (NT) instances exist for the resident multi-wave shapes
// (G >= 128, no prefetch), the ones used for calls too large for the MALL.
#include "sm_kernels.hpp"
#include "sm_launch.hpp"

namespace smx {

namespace {
template <int G, int V>
RowKernelFn pick_pf(int PF, int NT) {
    if (PF) {
        if constexpr (G <= 256) {
            if (!NT) return &k_softmax_rows<SM_DT, G, V, true, false>;
        }
        return nullptr;
    }
    if (NT) {
        if constexpr (G >= 128) return &k_softmax_rows<SM_DT, G, V, false, true>;
        return nullptr;
    }
    return &k_softmax_rows<SM_DT, G, V, false, false>;
}

template <int G>
RowKernelFn pick_v(int V, int PF, int NT) {
    switch (V) {
    case 1: return pick_pf<G, 1>(PF, NT);
    case 2: return pick_pf<G, 2>(PF, NT);
    case 4: return pick_pf<G, 4>(PF, NT);
    case 8: return pick_pf<G, 8>(PF, NT);
    default: return nullptr;
    }
}
}  // namespace

RowKernelFn SM_ROW_FN(int G, int V, int PF, int NT) {
    switch (G) {
    case 16: return pick_v<16>(V, PF, NT);
    case 32: return pick_v<32>(V, PF, NT);
    case 64: return pick_v<64>(V, PF, NT);
    case 128: return pick_v<128>(V, PF, NT);
    case 256: return pick_v<256>(V, PF, NT);
    case 512: return pick_v<512>(V, PF, NT);
    case 1024: return pick_v<1024>(V, PF, NT);
    default: return nullptr;
    }
}

}  // namespace smx
