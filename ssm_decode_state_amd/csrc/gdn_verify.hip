// gdn_verify.hip -- instantiations of the GDN / KDA speculative verify: up to 8 draft tokens per call
// (rounded up to 4 or 8 queries), at most 24 or 32 entries seen.
#include "gdn_kernels.hpp"

namespace ssm {

template <int DV, int DK, typename TIN, int RC, bool VG>
static hipError_t launch_verify_vg(const GdnArgs& a, int maxe, hipStream_t s) {
    const dim3 grid(a.heads, a.batch), block(DV);
    if (a.ntok <= 4 && maxe <= 24)  // a window of 16 with up to 4 drafts: less LDS, more heads per CU
        hipLaunchKernelGGL((gdn_replay_kernel<DV, DK, TIN, RC, 24, 4, false, VG>), grid, block, 0, s, a);
    else if (a.ntok <= 4)
        hipLaunchKernelGGL((gdn_replay_kernel<DV, DK, TIN, RC, 32, 4, false, VG>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gdn_replay_kernel<DV, DK, TIN, RC, 32, 8, false, VG>), grid, block, 0, s, a);
    return hipGetLastError();
}
template <int DV, int DK, typename TIN, int RC>
static hipError_t launch_verify_dd(const GdnArgs& a, int maxe, hipStream_t s) {
    if (a.kda) return launch_verify_vg<DV, DK, TIN, RC, true>(a, maxe, s);  // per-channel gate
    return launch_verify_vg<DV, DK, TIN, RC, false>(a, maxe, s);
}

template <typename TIN, int RC>
static hipError_t dispatch_verify(const GdnArgs& a, int dv, int dk, int maxe, hipStream_t s) {
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_verify_dd<V, K, TIN, RC>(a, maxe, s);
    SSM_GDN_SHAPES(X, 0)
#undef X
    return hipErrorNotSupported;
}

hipError_t gdn_launch_verify(const GdnArgs& a, int dv, int dk, int bf16, int rc, int maxe,
                             hipStream_t s) {
    if (maxe > kGdnMaxWin || a.ntok < 1 || a.ntok > 8) return hipErrorNotSupported;
    if (bf16) {
        if (rc == 0) return dispatch_verify<bf16_t, 0>(a, dv, dk, maxe, s);
        if (rc == 1) return dispatch_verify<bf16_t, 1>(a, dv, dk, maxe, s);
        return dispatch_verify<bf16_t, 2>(a, dv, dk, maxe, s);
    }
    if (rc == 0) return dispatch_verify<float, 0>(a, dv, dk, maxe, s);
    if (rc == 1) return dispatch_verify<float, 1>(a, dv, dk, maxe, s);
    return dispatch_verify<float, 2>(a, dv, dk, maxe, s);
}

}  // namespace ssm
