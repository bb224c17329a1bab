// gdn_conv.hip -- instantiations of the conventional (state-writing) GDN / KDA decode step.
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

hipError_t gdn_launch_conv(const GdnConvArgs& a, int dv, int dk, int bf16, hipStream_t s) {
#define X(V, K, T) \
    if (dv == V && dk == K) return launch_conv_dd<V, K, T>(a, s);
    if (bf16) { SSM_GDN_SHAPES(X, bf16_t) } else { SSM_GDN_SHAPES(X, float) }
#undef X
    return hipErrorNotSupported;
}

}  // namespace ssm
