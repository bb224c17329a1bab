// m2_decode.hip -- instantiations of the one-token replay decode (MAXQ = 1, the entries a call
// sees bounded by 16 or 32) and the entry of every replay launch.
#include "m2_kernels.hpp"

namespace ssm {

template <int P, int N, typename TIN, int RC>
static hipError_t launch_decode_pn(const M2Args& a, int maxe, hipStream_t s) {
    const dim3 grid = head_grid(a.batch, a.heads), block = head_block(a.batch, a.heads);
    if (maxe <= 16)
        hipLaunchKernelGGL((m2_replay_kernel<P, N, TIN, RC, 1, 16, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((m2_replay_kernel<P, N, TIN, RC, 1, 32, true>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename TIN, int RC>
static hipError_t dispatch_decode(const M2Args& a, int P, int N, int maxe, hipStream_t s) {
#define X(PP, NN, ...) \
    if (P == PP && N == NN) return launch_decode_pn<PP, NN, TIN, RC>(a, maxe, s);
    if constexpr (RC == 0) {
        SSM_M2_SHAPES(X, 0)
    } else {
        if (P == 64 && N == 64) return launch_decode_pn<64, 64, TIN, RC>(a, maxe, s);
        if (P == 64 && N == 128) return launch_decode_pn<64, 128, TIN, RC>(a, maxe, s);
    }
#undef X
    return hipErrorNotSupported;
}

hipError_t m2_launch_replay(const M2Args& a, int P, int N, int bf16, int rc, bool spec, int maxe,
                            hipStream_t s) {
    if (spec) return m2_launch_verify(a, P, N, bf16, rc, maxe, s);
    if (maxe > 32 || a.ntok != 1) return hipErrorNotSupported;
    if (bf16) {
        if (rc == 0) return dispatch_decode<bf16_t, 0>(a, P, N, maxe, s);
        if (rc == 1) return dispatch_decode<bf16_t, 1>(a, P, N, maxe, s);
        return dispatch_decode<bf16_t, 2>(a, P, N, maxe, s);
    }
    if (rc == 0) return dispatch_decode<float, 0>(a, P, N, maxe, s);
    if (rc == 1) return dispatch_decode<float, 1>(a, P, N, maxe, s);
    return dispatch_decode<float, 2>(a, P, N, maxe, s);
}

}  // namespace ssm
