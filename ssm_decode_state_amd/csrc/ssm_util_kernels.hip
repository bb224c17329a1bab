// ssm_util_kernels.hip -- small kernels: pointer commit after a speculative round, int fill,
// natural <-> tile layout conversion, and the device fp8/fp4 codecs exposed for testing.
#include <algorithm>

#include "ssm_device.hpp"
#include "ssm_kernels.hpp"
#include "ssm_replay.h"

namespace ssm {

// Resolve pending drafts by moving pointers only (news article, para 3): every head of sequence b
// commits min(n_accept[b], pending) drafts (negative values count as 0); a clamped value sets the
// accept-clamped bit of the state's flag word.
__global__ void commit_kernel(int* ptr, const int32_t* __restrict__ n_accept, int batch, int heads,
                              int pending, int* flags) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)batch * heads) return;
    const int raw = n_accept[i / heads];
    const int acc = raw < 0 ? 0 : (raw > pending ? pending : raw);
    ptr[kPtrInts * i + 1] += acc;
    if (acc != raw && i % heads == 0) atomicOr(flags, SSM_FLAG_ACCEPT_CLAMPED);
}

// Restore step of snapshot-based speculation: sequence b copies snapshot n_accept[b] - 1 (clamped
// to [0, ndraft]; 0 copies nothing) over its state. Grid (blocks, batch), float4 per thread.
__global__ void snap_select_kernel(float* __restrict__ h, const float* __restrict__ snap,
                                   const int32_t* __restrict__ n_accept, int batch, long seq_floats,
                                   int ndraft) {
    const int b = blockIdx.y;
    int n = n_accept[b];
    n = n < 0 ? 0 : (n > ndraft ? ndraft : n);
    if (n == 0) return;
    const float4* src = reinterpret_cast<const float4*>(snap + ((long)(n - 1) * batch + b) * seq_floats);
    float4* dst = reinterpret_cast<float4*>(h + (long)b * seq_floats);
    const long nq = seq_floats / 4;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += (long)gridDim.x * blockDim.x)
        st_stream(ld_stream(src + i), dst + i);
}

// Rewind to an earlier position inside the buffered window (explainer, "What a Replay-First Design
// Implies": restore state to position p): every head of sequence b drops its newest
// min(n_back[b], count) committed entries (negative values count as 0). Pointers only: replay
// rebuilds the output at any position between the checkpoint and the newest entry.
__global__ void restore_kernel(int* ptr, const int32_t* __restrict__ n_back, int batch, int heads) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)batch * heads) return;
    const int c = ptr[kPtrInts * i + 1];
    int n = n_back[i / heads];
    n = n < 0 ? 0 : (n > c ? c : n);
    ptr[kPtrInts * i + 1] = c - n;
}

// Fork (explainer, "The State-Storage Bottleneck in Branching Workloads": one prefix, several
// continuations): sequence dst[k] becomes a copy of sequence src[k] in every region of the state.
// Grid (x blocks, pair, region); 16-byte copies where the slice allows, 4-byte otherwise.
__global__ void fork_copy_kernel(char* __restrict__ mem, ForkRegions r, ForkPairs p) {
    const int k = blockIdx.y, g = blockIdx.z;
    if (k >= p.n || g >= r.n) return;
    const uint64_t slice = r.slice[g];
    const char* src = mem + r.off[g] + (uint64_t)p.src[k] * slice;
    char* dst = mem + r.off[g] + (uint64_t)p.dst[k] * slice;
    const uint64_t t0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    if (slice % 16 == 0) {
        // four independent 16-byte loads in flight per thread before their stores
        const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
        u32x4_t* d4 = reinterpret_cast<u32x4_t*>(dst);
        const uint64_t n = slice / 16;
        for (uint64_t i = t0; i < n; i += 4 * step) {
            u32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i + u * step < n) v[u] = __builtin_nontemporal_load(s4 + i + u * step);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i + u * step < n) __builtin_nontemporal_store(v[u], d4 + i + u * step);
        }
    } else {
        const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
        uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
        for (uint64_t i = t0; i < slice / 4; i += step) d1[i] = s1[i];
    }
}

// Fresh pointers: start 0, nothing committed, sequence b reads its own checkpoint slot b.
__global__ void ptr_init_kernel(int* ptr, long n, int heads) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) *reinterpret_cast<int4*>(ptr + kPtrInts * i) = make_int4(0, 0, (int)(i / heads), 0);
}

// Readers of every checkpoint slot (shared checkpoints): one 256-thread block per slot scans the
// sequences' slot fields (every head of a sequence holds the same slot; head 0's is read) and
// sums its lanes' counts. No atomics.
__global__ __launch_bounds__(256) void recount_kernel(int* refcnt, const int* __restrict__ ptr,
                                                      int batch, int heads) {
    __shared__ int s_part[4];
    const int s = blockIdx.x;
    int c = 0;
    for (int b = threadIdx.x; b < batch; b += blockDim.x) c += ptr[(long)kPtrInts * b * heads + 2] == s;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) refcnt[s] = s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

__global__ void fill_i32_kernel(int* p, int value, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

// One thread per 16-byte quad of a tile: quad (q, p) of head hd <-> natural row p, columns 4q..4q+3.
__global__ void pack_kernel(const float* __restrict__ src, float* __restrict__ dst, long nheads,
                            int P, int N, int unpack, const int* __restrict__ ptr, int heads) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long per = (long)P * N / 4;
    if (i >= nheads * per) return;
    const long hd = i / per;
    const int r = (int)(i % per);
    const int q = r / P, p = r % P;
    const long th = ptr ? (long)ptr[kPtrInts * hd + 2] * heads + hd % heads : hd;
    const long nat = hd * (long)P * N + (long)p * N + 4 * q;  // float offset, natural layout
    const long til = th * (long)P * N + (long)r * 4;          // float offset, tile layout
    if (unpack)
        *reinterpret_cast<float4*>(dst + nat) = *reinterpret_cast<const float4*>(src + til);
    else
        *reinterpret_cast<float4*>(dst + til) = *reinterpret_cast<const float4*>(src + nat);
}

// op 0: fp32 -> E4M3 code; 1: E4M3 code -> fp32; 2: fp32 -> E2M1 code; 3: E2M1 code -> fp32
// (software codecs). ops 4..7: the same through the gfx950 conversion instructions, encoding
// after clamping to the format's largest magnitude.
__global__ void codec_kernel(int op, const void* __restrict__ in, void* __restrict__ out, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float* fin = static_cast<const float*>(in);
    const uint8_t* cin = static_cast<const uint8_t*>(in);
    uint8_t* cout = static_cast<uint8_t*>(out);
    float* fout = static_cast<float*>(out);
    switch (op) {
        case 0: cout[i] = (uint8_t)e4m3_encode(fin[i]); break;
        case 1: fout[i] = e4m3_decode(cin[i]); break;
        case 2: cout[i] = (uint8_t)e2m1_encode(fin[i]); break;
        case 3: fout[i] = e2m1_decode(cin[i]); break;
        case 4: cout[i] = (uint8_t)(e4m3x2_encode_hw<false>(fminf(fmaxf(fin[i], -448.f), 448.f), 0.f, 0u) & 0xff); break;
        case 5: fout[i] = e4m3x2_decode_hw<false>(cin[i]).x; break;
        case 6: cout[i] = (uint8_t)(e2m1x2_encode_hw<0>(fminf(fmaxf(fin[i], -6.f), 6.f), 0.f, 0u) & 0xf); break;
        case 7: fout[i] = e2m1x2_decode_hw<0>(cin[i]).x; break;
        // packed words (n = number of 32-bit words): the helpers the read-copy kernels use
        case 8: {
            float o[4];
            e4m3_word_decode(static_cast<const uint32_t*>(in)[i], o);
            for (int k = 0; k < 4; ++k) fout[4 * i + k] = o[k];
            break;
        }
        case 9: {
            float o[8];
            e2m1_word_decode(static_cast<const uint32_t*>(in)[i], o);
            for (int k = 0; k < 8; ++k) fout[8 * i + k] = o[k];
            break;
        }
        case 10:
            static_cast<uint32_t*>(out)[i] =
                e4m3_word_encode(fin[4 * i], fin[4 * i + 1], fin[4 * i + 2], fin[4 * i + 3]);
            break;
        default:
            static_cast<uint32_t*>(out)[i] =
                e2m1_half_encode(fin[8 * i], fin[8 * i + 1], fin[8 * i + 2], fin[8 * i + 3]) |
                (e2m1_half_encode(fin[8 * i + 4], fin[8 * i + 5], fin[8 * i + 6], fin[8 * i + 7]) << 16);
            break;
    }
}

static unsigned blocks_for(long n, int bs) { return (unsigned)((n + bs - 1) / bs); }

hipError_t launch_commit(int* ptr, const int32_t* n_accept, int batch, int heads, int pending,
                         int* flags, hipStream_t s) {
    const long n = (long)batch * heads;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(commit_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, ptr, n_accept,
                       batch, heads, pending, flags);
    return hipGetLastError();
}

hipError_t launch_snap_select(float* h, const float* snap, const int32_t* n_accept, int batch,
                              long seq_floats, int ndraft, hipStream_t s) {
    if (batch == 0 || seq_floats == 0) return hipSuccess;
    // seq_floats = H * P * N, a multiple of 64; about 8 float4 per thread per block row
    const long nq = seq_floats / 4;
    const unsigned bx = (unsigned)std::min<long>(blocks_for(nq, 256 * 8), 1024);
    hipLaunchKernelGGL(snap_select_kernel, dim3(bx, (unsigned)batch), dim3(256), 0, s, h, snap,
                       n_accept, batch, seq_floats, ndraft);
    return hipGetLastError();
}

hipError_t launch_restore(int* ptr, const int32_t* n_back, int batch, int heads, hipStream_t s) {
    const long n = (long)batch * heads;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(restore_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, ptr, n_back,
                       batch, heads);
    return hipGetLastError();
}

hipError_t launch_fork_copy(char* mem, const ForkRegions& r, const ForkPairs& p, hipStream_t s) {
    if (p.n == 0 || r.n == 0) return hipSuccess;
    uint64_t most = 0;
    for (int g = 0; g < r.n; ++g) {
        if (r.slice[g] % 4 != 0 || r.off[g] % 16 != 0) return hipErrorInvalidValue;
        most = r.slice[g] > most ? r.slice[g] : most;
    }
    const unsigned bx = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>((most / 64 + 255) / 256, 64));
    hipLaunchKernelGGL(fork_copy_kernel, dim3(bx, (unsigned)p.n, (unsigned)r.n), dim3(256), 0, s,
                       mem, r, p);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int value, long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, p, value, n);
    return hipGetLastError();
}

hipError_t launch_pack(const float* src, float* dst, long nheads, int P, int N, int unpack,
                       const int* ptr, int heads, hipStream_t s) {
    const long n = nheads * P * N / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, src, dst, nheads, P,
                       N, unpack, ptr, heads);
    return hipGetLastError();
}

hipError_t launch_ptr_init(int* ptr, int batch, int heads, hipStream_t s) {
    const long n = (long)batch * heads;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(ptr_init_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, ptr, n, heads);
    return hipGetLastError();
}

hipError_t launch_recount(int* refcnt, const int* ptr, int batch, int heads, int nslot,
                          hipStream_t s) {
    if (nslot == 0) return hipSuccess;
    hipLaunchKernelGGL(recount_kernel, dim3((unsigned)nslot), dim3(256), 0, s, refcnt, ptr, batch,
                       heads);
    return hipGetLastError();
}

// Measurement reference: one pass of plain streaming reads over n16 16-byte units, the practical
// read ceiling the decode kernels are compared with. Read the way the decode kernels read a state
// tile: every wavefront takes a contiguous chunk of 64 * kU units (32 KiB), its lanes issue kU
// non-temporal 16-byte loads at once (each instruction covering 1 KiB), and the wavefronts of the
// grid stride over the chunks; units past the last whole chunk are read one per lane. Every value
// read feeds a per-wave XOR that lane 0 stores, so no load is dead.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, long n16,
                                                         uint32_t* __restrict__ out) {
    constexpr int kU = 32;
    constexpr long kChunk = 64L * kU;
    const int lane = threadIdx.x & 63;
    const long wave = (long)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const long nwaves = (long)gridDim.x * (blockDim.x / 64);
    const long nchunks = n16 / kChunk;
    uint32_t acc = 0;
    for (long c = wave; c < nchunks; c += nwaves) {
        const u32x4_t* p = src + c * kChunk + lane;
        u32x4_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(p + 64 * u);
        __builtin_amdgcn_sched_barrier(0);  // all kU loads in flight before the first use
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (long i = nchunks * kChunk + wave * 64 + lane; i < n16; i += nwaves * 64) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0) out[wave] = acc;
}

hipError_t launch_stream_read(const void* src, long bytes, uint32_t* out, int blocks, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(src), bytes / 16, out);
    return hipGetLastError();
}

hipError_t launch_codec(int op, const void* in, void* out, long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(codec_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, op, in, out, n);
    return hipGetLastError();
}

}  // namespace ssm
