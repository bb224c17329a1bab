// m2_fold.hip -- instantiations of the rank-L fold (flush), plain and fused with the window's
// closing decode step.
#include "m2_kernels.hpp"

namespace ssm {

template <int P, int N, typename TIN, int RC>
static hipError_t launch_flush_pn(const M2Args& a, int mode_all, int rewrite_only, hipStream_t s) {
    if (mode_all == 2)  // fused decode + fold of the L-th lock-step token
        hipLaunchKernelGGL((m2_fold_kernel<P, N, TIN, RC, true>), head_grid(a.batch, a.heads),
                           head_block(a.batch, a.heads), 0, s, a, 0, 0);
    else
        hipLaunchKernelGGL((m2_fold_kernel<P, N, TIN, RC, false>), head_grid(a.batch, a.heads),
                           head_block(a.batch, a.heads), 0, s, a, mode_all, rewrite_only);
    return hipGetLastError();
}

template <typename TIN, int RC>
static hipError_t dispatch_flush(const M2Args& a, int P, int N, int mode_all, int rewrite_only,
                                 hipStream_t s) {
#define X(PP, NN, ...) \
    if (P == PP && N == NN) return launch_flush_pn<PP, NN, TIN, RC>(a, mode_all, rewrite_only, s);
    if constexpr (RC == 0) {
        SSM_M2_SHAPES(X, 0)
    } else {
        if (P == 64 && N == 64) return launch_flush_pn<64, 64, TIN, RC>(a, mode_all, rewrite_only, s);
        if (P == 64 && N == 128)
            return launch_flush_pn<64, 128, TIN, RC>(a, mode_all, rewrite_only, s);
    }
#undef X
    return hipErrorNotSupported;
}

hipError_t m2_launch_flush(const M2Args& a, int P, int N, int bf16, int rc, int mode_all,
                           int rewrite_only, hipStream_t s) {
    if (bf16) {
        if (rc == 0) return dispatch_flush<bf16_t, 0>(a, P, N, mode_all, rewrite_only, s);
        if (rc == 1) return dispatch_flush<bf16_t, 1>(a, P, N, mode_all, rewrite_only, s);
        return dispatch_flush<bf16_t, 2>(a, P, N, mode_all, rewrite_only, s);
    }
    if (rc == 0) return dispatch_flush<float, 0>(a, P, N, mode_all, rewrite_only, s);
    if (rc == 1) return dispatch_flush<float, 1>(a, P, N, mode_all, rewrite_only, s);
    return dispatch_flush<float, 2>(a, P, N, mode_all, rewrite_only, s);
}

}  // namespace ssm
