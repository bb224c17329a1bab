// m2_verify.hip -- instantiations of the speculative verify: up to 8 draft tokens per call,
// the query count rounded up to 4 or 8, the entries a call sees bounded by 32 or 64.
#include "m2_kernels.hpp"

namespace ssm {

template <int P, int N, typename TIN, int RC, int MAXQ>
static hipError_t launch_verify_q(const M2Args& a, int maxe, hipStream_t s) {
    const dim3 grid = head_grid(a.batch, a.heads), block = head_block(a.batch, a.heads);
    if (maxe <= 32)
        hipLaunchKernelGGL((m2_replay_kernel<P, N, TIN, RC, MAXQ, 32, false>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((m2_replay_kernel<P, N, TIN, RC, MAXQ, 64, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int P, int N, typename TIN, int RC>
static hipError_t launch_verify_pn(const M2Args& a, int maxe, hipStream_t s) {
    if (a.ntok <= 4) return launch_verify_q<P, N, TIN, RC, 4>(a, maxe, s);
    return launch_verify_q<P, N, TIN, RC, 8>(a, maxe, s);
}

template <typename TIN, int RC>
static hipError_t dispatch_verify(const M2Args& a, int P, int N, int maxe, hipStream_t s) {
#define X(PP, NN, ...) \
    if (P == PP && N == NN) return launch_verify_pn<PP, NN, TIN, RC>(a, maxe, s);
    if constexpr (RC == 0) {
        SSM_M2_SHAPES(X, 0)
    } else {
        if (P == 64 && N == 64) return launch_verify_pn<64, 64, TIN, RC>(a, maxe, s);
        if (P == 64 && N == 128) return launch_verify_pn<64, 128, TIN, RC>(a, maxe, s);
    }
#undef X
    return hipErrorNotSupported;
}

hipError_t m2_launch_verify(const M2Args& a, int P, int N, int bf16, int rc, int maxe,
                            hipStream_t s) {
    if (maxe > 64 || a.ntok < 1 || a.ntok > 8) return hipErrorNotSupported;
    if (bf16) {
        if (rc == 0) return dispatch_verify<bf16_t, 0>(a, P, N, maxe, s);
        if (rc == 1) return dispatch_verify<bf16_t, 1>(a, P, N, maxe, s);
        return dispatch_verify<bf16_t, 2>(a, P, N, maxe, s);
    }
    if (rc == 0) return dispatch_verify<float, 0>(a, P, N, maxe, s);
    if (rc == 1) return dispatch_verify<float, 1>(a, P, N, maxe, s);
    return dispatch_verify<float, 2>(a, P, N, maxe, s);
}

}  // namespace ssm
