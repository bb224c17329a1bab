// gdn_decode.hip -- instantiations of the one-token GDN / KDA replay decode (the entries a call
// sees bounded by 16 or 32) and the entry of every GDN / KDA replay launch.
#include "gdn_kernels.hpp"

namespace ssm {

template <int DV, int DK, typename TIN, int RC, bool VG>
static hipError_t launch_decode_vg(const GdnArgs& a, int maxe, hipStream_t s) {
    const dim3 grid(a.heads, a.batch), block(DV);
    if (maxe <= 16)
        hipLaunchKernelGGL((gdn_replay_kernel<DV, DK, TIN, RC, 16, 1, true, VG>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gdn_replay_kernel<DV, DK, TIN, RC, 32, 1, true, VG>), grid, block, 0, s, a);
    return hipGetLastError();
}
template <int DV, int DK, typename TIN, int RC>
static hipError_t launch_decode_dd(const GdnArgs& a, int maxe, hipStream_t s) {
    if (a.kda) return launch_decode_vg<DV, DK, TIN, RC, true>(a, maxe, s);  // per-channel gate
    return launch_decode_vg<DV, DK, TIN, RC, false>(a, maxe, s);
}

template <typename TIN, int RC>
static hipError_t dispatch_decode(const GdnArgs& a, int dv, int dk, int maxe, hipStream_t s) {
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_decode_dd<V, K, TIN, RC>(a, maxe, s);
    SSM_GDN_SHAPES(X, 0)
#undef X
    return hipErrorNotSupported;
}

hipError_t gdn_launch_replay(const GdnArgs& a, int dv, int dk, int bf16, int rc, bool spec,
                             int maxe, hipStream_t s) {
    if (spec) return gdn_launch_verify(a, dv, dk, bf16, rc, maxe, s);
    if (maxe > kGdnMaxWin || a.ntok != 1) return hipErrorNotSupported;
    if (bf16) {
        if (rc == 0) return dispatch_decode<bf16_t, 0>(a, dv, dk, maxe, s);
        if (rc == 1) return dispatch_decode<bf16_t, 1>(a, dv, dk, maxe, s);
        return dispatch_decode<bf16_t, 2>(a, dv, dk, maxe, s);
    }
    if (rc == 0) return dispatch_decode<float, 0>(a, dv, dk, maxe, s);
    if (rc == 1) return dispatch_decode<float, 1>(a, dv, dk, maxe, s);
    return dispatch_decode<float, 2>(a, dv, dk, maxe, s);
}

}  // namespace ssm
