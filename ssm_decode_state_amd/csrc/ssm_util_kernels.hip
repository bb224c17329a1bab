// ssm_util_kernels.hip -- small kernels: pointer commit after a speculative round, int fill,
// natural <-> tile layout conversion, and the device fp8/fp4 codecs exposed for testing.
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

// Resolve pending drafts by moving pointers only (news article, para 3): every head of sequence b
// commits min(n_accept[b], pending) drafts (negative values count as 0).
__global__ void commit_kernel(int* ptr, const int32_t* __restrict__ n_accept, int batch, int heads,
                              int pending) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)batch * heads) return;
    int acc = n_accept[i / heads];
    acc = acc < 0 ? 0 : (acc > pending ? pending : acc);
    ptr[2 * i + 1] += acc;
}

__global__ void fill_i32_kernel(int* p, int value, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

// One thread per 16-byte quad of a tile: quad (q, p) of head hd <-> natural row p, columns 4q..4q+3.
__global__ void pack_kernel(const float* __restrict__ src, float* __restrict__ dst, long nheads,
                            int P, int N, int unpack) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long per = (long)P * N / 4;
    if (i >= nheads * per) return;
    const long hd = i / per;
    const int r = (int)(i % per);
    const int q = r / P, p = r % P;
    const long nat = hd * (long)P * N + (long)p * N + 4 * q;  // float offset, natural layout
    const long til = hd * (long)P * N + (long)r * 4;          // float offset, tile layout
    if (unpack)
        *reinterpret_cast<float4*>(dst + nat) = *reinterpret_cast<const float4*>(src + til);
    else
        *reinterpret_cast<float4*>(dst + til) = *reinterpret_cast<const float4*>(src + nat);
}

// op 0: fp32 -> E4M3 code; 1: E4M3 code -> fp32; 2: fp32 -> E2M1 code; 3: E2M1 code -> fp32.
__global__ void codec_kernel(int op, const void* __restrict__ in, void* __restrict__ out, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (op == 0) static_cast<uint8_t*>(out)[i] = (uint8_t)e4m3_encode(static_cast<const float*>(in)[i]);
    else if (op == 1) static_cast<float*>(out)[i] = e4m3_decode(static_cast<const uint8_t*>(in)[i]);
    else if (op == 2) static_cast<uint8_t*>(out)[i] = (uint8_t)e2m1_encode(static_cast<const float*>(in)[i]);
    else static_cast<float*>(out)[i] = e2m1_decode(static_cast<const uint8_t*>(in)[i]);
}

static unsigned blocks_for(long n, int bs) { return (unsigned)((n + bs - 1) / bs); }

hipError_t launch_commit(int* ptr, const int32_t* n_accept, int batch, int heads, int pending,
                         hipStream_t s) {
    const long n = (long)batch * heads;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(commit_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, ptr, n_accept,
                       batch, heads, pending);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int value, long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, p, value, n);
    return hipGetLastError();
}

hipError_t launch_pack(const float* src, float* dst, long nheads, int P, int N, int unpack,
                       hipStream_t s) {
    const long n = nheads * P * N / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, src, dst, nheads, P,
                       N, unpack);
    return hipGetLastError();
}

hipError_t launch_codec(int op, const void* in, void* out, long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(codec_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, op, in, out, n);
    return hipGetLastError();
}

}  // namespace ssm
