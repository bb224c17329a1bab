// m2_conv.hip -- instantiations of the conventional (state-writing) Mamba-2 decode step and of
// its snapshot-based speculative form.
#include "m2_kernels.hpp"

namespace ssm {

template <int P, int N, typename TIN>
static hipError_t launch_conv_pn(const M2ConvArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((m2_conv_kernel<P, N, TIN>), head_grid(a.batch, a.heads), head_block(a.batch, a.heads), 0, s, a);
    return hipGetLastError();
}

template <int P, int N, typename TIN>
static hipError_t launch_snap_pn(const M2ConvArgs& a, hipStream_t s) {
    const dim3 grid = head_grid(a.batch, a.heads), block = head_block(a.batch, a.heads);
    if (a.ntok <= 4)
        hipLaunchKernelGGL((m2_snap_kernel<P, N, TIN, 4>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((m2_snap_kernel<P, N, TIN, 8>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t m2_launch_snapshot(const M2ConvArgs& a, int P, int N, int bf16, hipStream_t s) {
    if (a.ntok < 1 || a.ntok > 8 || !a.snap) return hipErrorNotSupported;
#define X(PP, NN, T) \
    if (P == PP && N == NN) return launch_snap_pn<PP, NN, T>(a, s);
    if (bf16) {
        SSM_M2_SHAPES(X, bf16_t)
    } else {
        SSM_M2_SHAPES(X, float)
    }
#undef X
    return hipErrorNotSupported;
}

hipError_t m2_launch_conv(const M2ConvArgs& a, int P, int N, int bf16, hipStream_t s) {
#define X(PP, NN, T) \
    if (P == PP && N == NN) return launch_conv_pn<PP, NN, T>(a, s);
    if (bf16) {
        SSM_M2_SHAPES(X, bf16_t)
    } else {
        SSM_M2_SHAPES(X, float)
    }
#undef X
    return hipErrorNotSupported;
}

}  // namespace ssm
