// gdn_conv.hip -- instantiations of the conventional (state-writing) GDN / KDA decode step and of
// its snapshot-based speculative form.
#include "gdn_kernels.hpp"

namespace ssm {

template <int DV, int DK, typename TIN>
static hipError_t launch_conv_dd(const GdnConvArgs& a, hipStream_t s) {
    if (a.kda)
        hipLaunchKernelGGL((gdn_conv_kernel<DV, DK, TIN, true>), dim3(a.heads, a.batch), dim3(DV), 0, s, a);
    else
        hipLaunchKernelGGL((gdn_conv_kernel<DV, DK, TIN, false>), dim3(a.heads, a.batch), dim3(DV), 0, s, a);
    return hipGetLastError();
}

template <int DV, int DK, typename TIN, bool VG>
static hipError_t launch_snap_vg(const GdnConvArgs& a, hipStream_t s) {
    const dim3 grid(a.heads, a.batch), block(DV);
    if (a.ntok <= 4)
        hipLaunchKernelGGL((gdn_snap_kernel<DV, DK, TIN, 4, VG>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gdn_snap_kernel<DV, DK, TIN, 8, VG>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int DV, int DK, typename TIN>
static hipError_t launch_snap_dd(const GdnConvArgs& a, hipStream_t s) {
    if (a.kda) return launch_snap_vg<DV, DK, TIN, true>(a, s);
    return launch_snap_vg<DV, DK, TIN, false>(a, s);
}

hipError_t gdn_launch_snapshot(const GdnConvArgs& a, int dv, int dk, int bf16, hipStream_t s) {
    if (a.ntok < 1 || a.ntok > 8 || !a.snap) return hipErrorNotSupported;
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_snap_dd<V, K, T>(a, s);
    if (bf16) { SSM_GDN_SHAPES(X, bf16_t) } else { SSM_GDN_SHAPES(X, float) }
#undef X
    return hipErrorNotSupported;
}

hipError_t gdn_launch_conv(const GdnConvArgs& a, int dv, int dk, int bf16, hipStream_t s) {
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_conv_dd<V, K, T>(a, s);
    if (bf16) { SSM_GDN_SHAPES(X, bf16_t) } else { SSM_GDN_SHAPES(X, float) }
#undef X
    return hipErrorNotSupported;
}

}  // namespace ssm
