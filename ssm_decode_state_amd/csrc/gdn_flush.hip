// gdn_flush.hip -- instantiations of the GDN / KDA UT/WY flush: plain, fused with the window's closing
// decode step, and the read-copy rewrite (init).
#include "gdn_kernels.hpp"

namespace ssm {

template <int DV, int DK, typename TIN, int RC, bool VG>
static hipError_t launch_flush_vg(const GdnArgs& a, int mode_all, int rewrite_only, hipStream_t s) {
    const dim3 grid(a.heads, a.batch), block(DV);
    if (mode_all == 2) {  // fused decode + fold of the L-th lock-step token (and copy rewrite)
        hipLaunchKernelGGL((gdn_flush_kernel<DV, DK, TIN, RC, true, VG>), grid, block, 0, s, a, 0, 0);
    } else {
        hipLaunchKernelGGL((gdn_flush_kernel<DV, DK, TIN, RC, false, VG>), grid, block, 0, s, a,
                           mode_all, rewrite_only);
    }
    return hipGetLastError();
}
template <int DV, int DK, typename TIN, int RC>
static hipError_t launch_flush_dd(const GdnArgs& a, int mode_all, int rewrite_only, hipStream_t s) {
    if (a.kda) return launch_flush_vg<DV, DK, TIN, RC, true>(a, mode_all, rewrite_only, s);  // per-channel gate
    return launch_flush_vg<DV, DK, TIN, RC, false>(a, mode_all, rewrite_only, s);
}

template <typename TIN, int RC>
static hipError_t dispatch_flush(const GdnArgs& a, int dv, int dk, int mode_all, int rewrite_only,
                                 hipStream_t s) {
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_flush_dd<V, K, TIN, RC>(a, mode_all, rewrite_only, s);
    SSM_GDN_SHAPES(X, 0)
#undef X
    return hipErrorNotSupported;
}

hipError_t gdn_launch_flush(const GdnArgs& a, int dv, int dk, int bf16, int rc, int mode_all,
                            int rewrite_only, hipStream_t s) {
    if (bf16) {
        if (rc == 0) return dispatch_flush<bf16_t, 0>(a, dv, dk, mode_all, rewrite_only, s);
        if (rc == 1) return dispatch_flush<bf16_t, 1>(a, dv, dk, mode_all, rewrite_only, s);
        return dispatch_flush<bf16_t, 2>(a, dv, dk, mode_all, rewrite_only, s);
    }
    if (rc == 0) return dispatch_flush<float, 0>(a, dv, dk, mode_all, rewrite_only, s);
    if (rc == 1) return dispatch_flush<float, 1>(a, dv, dk, mode_all, rewrite_only, s);
    return dispatch_flush<float, 2>(a, dv, dk, mode_all, rewrite_only, s);
}

}  // namespace ssm
