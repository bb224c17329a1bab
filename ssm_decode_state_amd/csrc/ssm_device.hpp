// ssm_device.hpp -- device helpers shared by the gfx950 kernels of the ReplaySSM library.
//
// Wave64 throughout (CDNA4). Nothing here depends on a particular layer type.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef uint16_t bf16_t;  // storage of bfloat16 inputs (upper half of an fp32)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Streaming (non-temporal) 16-byte accesses for data touched once per launch.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float4 v, float4* p) {
    const f32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}

// Ring slot of entry e (0-based after the checkpoint): (start + e) mod cap for start < cap and
// e < cap, without an integer division (keeps the address arithmetic branch-free).
__device__ __forceinline__ int ring_slot(int start, int e, int cap) {
    const int s = start + e;
    return s >= cap ? s - cap : s;
}

// Cache-policy operands of gfx950 buffer stores (sc0 = 1, nt = 2, sc1 = 16): write-through at
// system scope, and the same with the streaming hint.
enum : int { kStoreWT = 1 | 16, kStoreWTNT = 1 | 2 | 16 };
// Third dword of a raw buffer resource: untyped access, 32-bit data format.
constexpr int kRawBufferWord3 = 0x00020000;

// Streaming access to a state tile through a wave-uniform base and a 32-bit per-lane byte
// offset: each access is an SGPR base plus one shared VGPR offset, so a tile that is loaded at
// the start of a kernel and stored at its end keeps no per-access 64-bit addresses alive.
struct TileIO {
    char* base;     // wave-uniform
    uint32_t lane;  // this lane's byte offset
    __device__ __forceinline__ float4 load(uint32_t off) const {
        return ld_stream(reinterpret_cast<const float4*>((base + off) + lane));
    }
    // POL = 0: a non-temporal global store; otherwise a buffer store with that cache-policy
    // operand through a resource based at the tile
    template <int POL = 0>
    __device__ __forceinline__ void store(uint32_t off, float4 v) const {
        if constexpr (POL == 0) {
            st_stream(v, reinterpret_cast<float4*>((base + off) + lane));
        } else {
            const u32x4_t t = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                               __float_as_uint(v.w)};
            __builtin_amdgcn_raw_buffer_store_b128(
                t, __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, kRawBufferWord3),
                (int)(off + lane), 0, POL);
        }
    }
};

// Unpack one 16-byte unit of T (fp32 or bf16 bits) into floats.
template <typename T> struct Unit;
template <> struct Unit<float> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void unpack(uint4 u, float* d) {
        d[0] = __uint_as_float(u.x); d[1] = __uint_as_float(u.y);
        d[2] = __uint_as_float(u.z); d[3] = __uint_as_float(u.w);
    }
};
template <> struct Unit<bf16_t> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void unpack(uint4 u, float* d) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = __uint_as_float(w[i] << 16);
            d[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

// Load E contiguous elements of T as raw bits (no conversion) with the widest access possible.
template <typename T, int E>
__device__ __forceinline__ void load_raw(const T* __restrict__ src, T (&d)[E]) {
    constexpr int kBytes = E * (int)sizeof(T);
    if constexpr (kBytes % 16 == 0) {
#pragma unroll
        for (int u = 0; u < kBytes / 16; ++u) {
            const uint4 t = reinterpret_cast<const uint4*>(src)[u];
            __builtin_memcpy(&d[u * (16 / sizeof(T))], &t, 16);
        }
    } else if constexpr (kBytes % 8 == 0) {
#pragma unroll
        for (int u = 0; u < kBytes / 8; ++u) {
            const uint2 t = reinterpret_cast<const uint2*>(src)[u];
            __builtin_memcpy(&d[u * (8 / sizeof(T))], &t, 8);
        }
    } else if constexpr (kBytes % 4 == 0) {
#pragma unroll
        for (int u = 0; u < kBytes / 4; ++u) {
            const uint32_t t = reinterpret_cast<const uint32_t*>(src)[u];
            __builtin_memcpy(&d[u * (4 / sizeof(T))], &t, 4);
        }
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i) d[i] = src[i];
    }
}

// Stores with an explicit cache policy, for the per-token ring appends and outputs of the replay
// kernels: gfx950 buffer stores through a resource whose base is wave-uniform (one head's ring
// rows, one output row) and a per-lane byte offset, checked by the hardware against the
// resource's size. The policy is the store's cache-policy operand: sc0 | sc1 (system scope, so
// the L2 writes the line through rather than holding it dirty) and nt (streaming). Those few
// thin writes inside a saturated read stream cost far more than their bytes; written through
// they cost less (measured on the replay and verify kernels). Of the bulk tile writes, the
// Gated DeltaNet flush and conventional kernels take write-through streaming stores too
// (TileIO::store's policy argument); the Mamba-2 fold's copy writes measured faster with the
// default policy.

struct PolicyStore {
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ PolicyStore(const void* base, uint32_t bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                                 kRawBufferWord3)) {}
    // B bytes (16, 8, 4 or 2) from src at byte offset off
    template <int POL, int B>
    __device__ __forceinline__ void bytes(uint32_t off, const void* src) const {
        static_assert(B == 16 || B == 8 || B == 4 || B == 2, "store width");
        if constexpr (B == 16) {
            u32x4_t v;
            __builtin_memcpy(&v, src, 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)off, 0, POL);
        } else if constexpr (B == 8) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            u32x2_t v;
            __builtin_memcpy(&v, src, 8);
            __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, (int)off, 0, POL);
        } else if constexpr (B == 4) {
            uint32_t v;
            __builtin_memcpy(&v, src, 4);
            __builtin_amdgcn_raw_buffer_store_b32(v, rsrc, (int)off, 0, POL);
        } else {
            unsigned short v;
            __builtin_memcpy(&v, src, 2);
            __builtin_amdgcn_raw_buffer_store_b16(v, rsrc, (int)off, 0, POL);
        }
    }
};

// Wave-local ordering point for LDS written by some lanes and read by others of the same wave:
// the LDS unit executes one wave's operations in order, so a compiler-level barrier with
// wavefront-scope fences is enough.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Pair of values {v[l], v[l ^ M]} (in an unspecified order) for a lane exchange mask M, taken
// without LDS where gfx950 allows: M = 16 and 32 by v_permlane16_swap / v_permlane32_swap (with
// both operands v, the odd rows of one swap with the even rows of the other), M = 1 and 2 by
// DPP quad permutes; other masks by ds_bpermute. A commutative op on the pair gives the xor
// exchange, identical in both lanes of every pair.
template <int M> struct XorPair {
    __device__ __forceinline__ static void get(float v, float& a, float& b) {
        if constexpr (M == 16 || M == 32) {
            const auto p = M == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                                   : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            a = __uint_as_float(p[0]);
            b = __uint_as_float(p[1]);
        } else if constexpr (M == 1 || M == 2) {
            constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
            a = v;
            b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
        } else {
            a = v;
            b = shfl_xor(v, M);
        }
    }
};

// Sum over lanes that differ only in the bits of `lo..hi` (masks lo, 2lo, ..., hi).
template <int LO, int HI>
__device__ __forceinline__ float xor_reduce_sum(float v) {
    if constexpr (LO <= HI) {
        float a, b;
        XorPair<LO>::get(v, a, b);
        return xor_reduce_sum<2 * LO, HI>(a + b);
    } else {
        return v;
    }
}
template <int LO, int HI>
__device__ __forceinline__ float xor_reduce_max(float v) {
    if constexpr (LO <= HI) {
        float a, b;
        XorPair<LO>::get(v, a, b);
        return xor_reduce_max<2 * LO, HI>(fmaxf(a, b));
    } else {
        return v;
    }
}

// Sum over aligned groups of GS lanes (GS a power of two up to 64), left in every lane of the
// group. Quad steps by DPP quad_perm; then, with every quad (half row) holding its sum, the
// half-row and row mirrors (lane i <-> 7 - i, 15 - i) pair each half with the other; rows by
// permlane16/32 swaps.
template <int GS>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(GS >= 1 && GS <= 64 && (GS & (GS - 1)) == 0, "group size");
    if constexpr (GS >= 2) { float a, b; XorPair<1>::get(v, a, b); v = a + b; }
    if constexpr (GS >= 4) { float a, b; XorPair<2>::get(v, a, b); v = a + b; }
    if constexpr (GS >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (GS >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    if constexpr (GS >= 32) { float a, b; XorPair<16>::get(v, a, b); v = a + b; }
    if constexpr (GS >= 64) { float a, b; XorPair<32>::get(v, a, b); v = a + b; }
    return v;
}

// Value of v in lane `lane`. The index MUST be wave-uniform: a per-lane index is silently
// replaced by the first active lane's (v_readlane takes a scalar lane select). Use __shfl for
// per-lane indices.
__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A 64-bit wave-uniform value moved to scalar registers: the compiler forms 64-bit products
// such as a row index times a stride in vector registers, and everything derived from them
// (ring and input addresses) would then stay there too.
__device__ __forceinline__ long uniform64(long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long)(((unsigned long long)hi << 32) | lo);
}

// fp32 MFMA 16x16x4 (v_mfma_f32_16x16x4f32): D = A (16x4) * B (4x16) + C. Operand lanes:
// A[m][k] from lane m + 16k, B[k][c] from lane c + 16k, D[m][c] in lane c + 16(m/4), register m%4.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// fp32 MFMA 4x4x1 over 16 blocks (v_mfma_f32_4x4x1f32): block b = lane / 4 computes
// D[i][j] += A[i] B[j] with A[i] from lane 4b + i, B[j] from lane 4b + j, D[i][j] in lane 4b + j,
// register i. With a = u_{lane%4}[n] and b = h[lane][n], lane p accumulates sum_n u_i[n] h[p][n]
// in register i: four row dot products of the wave's 64 rows per instruction.
__device__ __forceinline__ f32x4 mfma4x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// OCP low-precision codecs, written from the format definitions (OCP OFP8 E4M3: bias 7, three
// mantissa bits, max 448, no infinity; OCP MX E2M1: bias 1, one mantissa bit, max 6).
// Encoding: round to nearest, ties to even, saturating at the largest finite magnitude; the code's
// sign bit is the sign bit of the fp32 input.
// ---------------------------------------------------------------------------------------------

// Magnitude code of |v| on a grid with MB mantissa bits, minimum normal exponent EMIN and largest
// magnitude code MAXC. |v| * 2^k scalings are exact, and rintf rounds half to even.
template <int MB, int EMIN, int MAXC>
__device__ __forceinline__ uint32_t encode_mag(float a) {
    // a >= 0, finite. Saturate first: every value above the largest finite rounds to it.
    const float amax = __uint_as_float(((uint32_t)(((MAXC >> MB) + EMIN - 1) + 127) << 23) |
                                       ((uint32_t)(MAXC & ((1 << MB) - 1)) << (23 - MB)));
    if (a >= amax) return MAXC;
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // floor(log2 a) for normal a
    if (e < EMIN) e = EMIN;                                  // subnormal range: quantum 2^(EMIN-MB)
    const float q = ldexpf(a, MB - e);                       // a / 2^(e-MB), exact
    const uint32_t n = (uint32_t)rintf(q);                   // in [0, 2^(MB+1)]
    // code = (biased exponent << MB) + mantissa; for the subnormal range the biased exponent is 0
    // and n < 2^MB, and n == 2^(MB+1) rolls over into the next binade correctly.
    const uint32_t be = (uint32_t)(e - EMIN);  // 0 for the lowest binade (normal or subnormal)
    return (be << MB) + n;
}

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t s = (__float_as_uint(v) >> 31) << 7;
    return s | encode_mag<3, -6, 0x7E>(fabsf(v));
}
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    const uint32_t s = (__float_as_uint(v) >> 31) << 3;
    return s | encode_mag<1, 0, 0x7>(fabsf(v));
}

// Software decode of an E4M3 code (no NaN codes are ever written).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xF, m = c & 7;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80) ? -mag : mag;
}
// Software decode of an E2M1 code.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
    const uint32_t twice = (0xC8643210u >> ((c & 7) * 4)) & 0xF;  // 2*|value|: 0,1,2,3,4,6,8,12
    const float mag = (float)twice * 0.5f;
    return (c & 8) ? -mag : mag;
}

// Hardware conversions (gfx950): two codes per instruction; the half/byte selector is a
// compile-time operand. Used only where a device test has shown them equal to the software codecs
// above for every code and for the tested inputs.
template <bool HI>
__device__ __forceinline__ float2 e4m3x2_decode_hw(uint32_t word) {
    const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
    return make_float2(v[0], v[1]);
}
template <int BYTE>
__device__ __forceinline__ float2 e2m1x2_decode_hw(uint32_t word) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, BYTE);
    return make_float2(v[0], v[1]);
}
// Encode two values (already inside +-448) into the selected 16-bit half of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_encode_hw(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}
// Encode two values (already inside +-6) into byte BYTE of `old`.
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_encode_hw(float a, float b, uint32_t old) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, BYTE);
}

// Packed-word codecs built on the instructions above. Byte i of an E4M3 word is element i;
// nibble i of an E2M1 word (low nibble first) is element i. Encoders take fp32 values already
// multiplied by the inverse scale and saturate like the software encoders.
__device__ __forceinline__ void e4m3_word_decode(uint32_t w, float (&o)[4]) {
    const float2 lo = e4m3x2_decode_hw<false>(w), hi = e4m3x2_decode_hw<true>(w);
    o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}
__device__ __forceinline__ void e2m1_word_decode(uint32_t w, float (&o)[8]) {
    const float2 b0 = e2m1x2_decode_hw<0>(w), b1 = e2m1x2_decode_hw<1>(w);
    const float2 b2 = e2m1x2_decode_hw<2>(w), b3 = e2m1x2_decode_hw<3>(w);
    o[0] = b0.x; o[1] = b0.y; o[2] = b1.x; o[3] = b1.y;
    o[4] = b2.x; o[5] = b2.y; o[6] = b3.x; o[7] = b3.y;
}
__device__ __forceinline__ float sat(float x, float m) { return fminf(fmaxf(x, -m), m); }
__device__ __forceinline__ uint32_t e4m3_word_encode(float a, float b, float c, float d) {
    const uint32_t lo = e4m3x2_encode_hw<false>(sat(a, 448.f), sat(b, 448.f), 0u);
    return e4m3x2_encode_hw<true>(sat(c, 448.f), sat(d, 448.f), lo);
}
// Four E2M1 codes (16 bits) from four values.
__device__ __forceinline__ uint32_t e2m1_half_encode(float a, float b, float c, float d) {
    const uint32_t lo = e2m1x2_encode_hw<0>(sat(a, 6.f), sat(b, 6.f), 0u);
    return e2m1x2_encode_hw<1>(sat(c, 6.f), sat(d, 6.f), lo) & 0xffffu;
}

}  // namespace ssm
