// rc_codec.hpp -- the low-precision read copy of a state tile (news article, para 4: a
// low-precision copy of the checkpoint serves the reads while the recurrence keeps the fp32
// checkpoint), shared by the Mamba-2 and Gated DeltaNet kernels.
//
// A head's tile has ROWS rows (Mamba-2 P = 64, GDN dv) of N elements (Mamba-2 N, GDN dk):
//   fp8 row copy: s = max(amax_row / 448, 2^-126) (1 if zero), code = RNE_sat_e4m3(h * (1/s)),
//     value*s.
//   fp4 copy (NVFP4 reading): s_t = max(amax_tile / 2688, 2^-117) (1 if zero); per 16-element
//     block s_b = value(RNE_sat_e4m3(amax_blk / (6 s_t))), S = s_b s_t,
//     code = RNE_sat_e2m1(h * (1/S)) (all zero when S == 0), value*S.
//   The floors keep every scale normal with a finite reciprocal (a nonzero E4M3 block scale is at
//   least 2^-9, so S >= 2^-126): a row or tile of tiny values, e.g. a sequence that decayed with
//   no input, would otherwise get an infinite reciprocal and encode 0 * inf = NaN.
// Codes: fp8 byte at ((n/16)*ROWS + p)*16 + n%16 of the head's code block; fp4 nibble of byte
// ((n/32)*ROWS + p)*16 + (n%32)/2, low nibble = even n. Block scales [p][N/16]; row and tile
// scales fp32.
#pragma once
#include "ssm_device.hpp"

namespace ssm {

constexpr float kRcScaleFloorFp8 = 0x1p-126f;      // smallest normal fp32
constexpr float kRcScaleFloorFp4Tile = 0x1p-117f;  // 2^-126 / 2^-9 (smallest E4M3 subnormal)

// Device pointers of one layer's read copy.
struct RcView {
    uint8_t* codes;
    void* scale;    // fp8: fp32 row scales; fp4: E4M3 block-scale codes
    float* tscale;  // fp4: fp32 tile scales
};

// One row of the decoded copy, held by the lane that owns the row. load() only issues the reads
// (so a kernel can put them in flight next to its other early loads); dots() waits for them,
// decodes, and accumulates the row's dot products with MAXQ query vectors (s_q, row stride CS)
// into acc[j] for j < nq.
template <int ROWS, int N, int RC>
struct RcRow {
    static_assert(N == 64 || N == 128, "read copy: N in {64, 128}");
    static_assert(RC == 1 || RC == 2, "read copy kind");
    static constexpr int kU = RC == 1 ? N / 16 : N / 32;  // 16-byte code units per row
    static constexpr int kSB = RC == 1 ? 1 : (N / 16 + 3) / 4;  // scale words
    u32x4_t u[kU];
    uint32_t sbw[kSB];  // fp8: the fp32 row scale's bits; fp4: the row's E4M3 block-scale codes
    float st;           // fp4 tile scale

    __device__ __forceinline__ void load(const RcView& v, long head, int row) {
        const u32x4_t* codes = reinterpret_cast<const u32x4_t*>(
            v.codes + head * (long)(RC == 1 ? ROWS * N : ROWS * N / 2));
#pragma unroll
        for (int k = 0; k < kU; ++k) u[k] = __builtin_nontemporal_load(codes + k * ROWS + row);
        if constexpr (RC == 1) {
            sbw[0] = static_cast<const uint32_t*>(v.scale)[head * ROWS + row];
            st = 1.f;
        } else {
            const uint8_t* sbp = static_cast<const uint8_t*>(v.scale) + (head * ROWS + row) * (N / 16);
            if constexpr (N / 16 >= 8) {
                const uint2 t = *reinterpret_cast<const uint2*>(sbp);
                sbw[0] = t.x; sbw[1] = t.y;
            } else {
                sbw[0] = *reinterpret_cast<const uint32_t*>(sbp);
            }
            st = v.tscale[head];
        }
    }

    template <int CS, int MAXQ>
    __device__ __forceinline__ void dots(int nq, const float* s_q, float (&acc)[MAXQ]) const {
        if constexpr (RC == 1) {
            const float s = __uint_as_float(sbw[0]);
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
                float val[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float o[4];
                    e4m3_word_decode(w[q], o);
#pragma unroll
                    for (int i = 0; i < 4; ++i) val[4 * q + i] = o[i];
                }
#pragma unroll
                for (int j = 0; j < MAXQ; ++j) {
                    if (j >= nq) break;
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) d += val[i] * s_q[j * CS + 16 * k + i];
                    acc[j] += s * d;
                }
            }
        } else {
            // the row's block scales S = value(code) * s_t, two codes per conversion instruction
            // (the codes are finite and non-negative: the writer saturates them at 448)
            float S_blk[N / 16];
#pragma unroll
            for (int w = 0; w < kSB; ++w) {
                const float2 lo = e4m3x2_decode_hw<false>(sbw[w]), hi = e4m3x2_decode_hw<true>(sbw[w]);
                const float sv[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * w + i < N / 16) S_blk[4 * w + i] = sv[i] * st;
            }
#pragma unroll
            for (int k = 0; k < kU; ++k) {
                const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int blk = 2 * k + half;
                    const float S = S_blk[blk];
                    float val[16];  // elements 16 half .. 16 half + 15 of the 32-element unit
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        float o[8];
                        e2m1_word_decode(w[2 * half + q], o);
#pragma unroll
                        for (int i = 0; i < 8; ++i) val[8 * q + i] = o[i];
                    }
#pragma unroll
                    for (int j = 0; j < MAXQ; ++j) {
                        if (j >= nq) break;
                        float d = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) d += val[i] * s_q[j * CS + 16 * blk + i];
                        acc[j] += S * d;
                    }
                }
            }
        }
    }
};

// No read copy: nothing to hold (the kernels read the fp32 tile instead).
template <int ROWS, int N>
struct RcRow<ROWS, N, 0> {
    __device__ __forceinline__ void load(const RcView&, long, int) {}
};

// E4M3 code of the fp4 block scale, RNE_sat_e4m3(RN(ab / d6)) for ab >= 0 and d6 > 0, without a
// division in the common case. q = ab * rd6 with rd6 = RN(1/d6) is within about 2^-23 (relative)
// of ab / d6, so the interval [q (1 - 2^-21), q (1 + 2^-21)] holds both ab / d6 and its rounding
// RN(ab / d6). Rounding to E4M3 is monotonic: when both ends of the interval give the same code,
// that is the code of RN(ab / d6); otherwise (an E4M3 rounding boundary within a few fp32 ulps of
// the quotient) the quotient is divided out exactly. Quotients in the subnormal fp32 range, where
// the relative bound does not hold, lie far below 2^-10 and every candidate encodes to 0. The
// encodes are the gfx950 conversion instruction, two values per instruction, on values clamped
// to the format's largest finite magnitude.
__device__ __forceinline__ uint32_t block_scale_code(float ab, float d6, float rd6) {
    const float q = ab * rd6;
    const uint32_t lohi = e4m3x2_encode_hw<false>(sat(q * (1.f - 0x1p-21f), 448.f),
                                                  sat(q * (1.f + 0x1p-21f), 448.f), 0u);
    uint32_t code = lohi & 0xffu;
    if (code != ((lohi >> 8) & 0xffu))  // rare: a rounding boundary is within reach
        code = e4m3x2_encode_hw<false>(sat(ab / d6, 448.f), 0.f, 0u) & 0xffu;
    return code;
}

// Largest magnitude among this lane's values of a tile held in MFMA accumulator order (hb[pb][nb]
// holds row row0 + 16 pb + l%16, columns 16 nb + 4 (l/16) .. + 3). The caller reduces it over the
// lanes (and waves) that hold the head's tile: the fp4 tile scale.
template <int N>
__device__ __forceinline__ float rc_local_amax(const f32x4 (&hb)[4][N / 16]) {
    float amax = 0.f;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(hb[pb][nb][r]));
    return amax;
}

// Write the copy of rows row0 .. row0 + 63 of a head's tile from its fp32 values in MFMA
// accumulator order (see rc_local_amax). fp4 needs amax_tile, the largest magnitude over the whole
// head tile; `tile_writer` is true in exactly one lane of the head, which stores the tile scale.
// s_tab: 128 floats of LDS private to the calling wavefront (fp4 only; may hold anything).
template <int ROWS, int N, int RC>
__device__ __forceinline__ void rc_write_blocks(const RcView& v, long head, int row0, int li, int lg,
                                                const f32x4 (&hb)[4][N / 16], float amax_tile,
                                                bool tile_writer, float* s_tab) {
    static_assert(N == 64 || N == 128, "read copy: N in {64, 128}");
    // the lane indices pass through an empty asm here, so that the compiler cannot compute the
    // copy's store addresses at the top of the calling kernel and hold them across its loops
    asm volatile("" : "+v"(li), "+v"(lg));
    constexpr int kNB = N / 16;
    if constexpr (RC == 1) {
        uint8_t* codes = v.codes + head * (long)(ROWS * N);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            float amax = 0.f;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(hb[pb][nb][r]));
            amax = xor_reduce_max<16, 32>(amax);  // the row is spread over lanes li + 16 lg
            const float sc = amax > 0.f ? fmaxf(amax / 448.f, kRcScaleFloorFp8) : 1.f;
            const float inv = 1.f / sc;
            const int p = row0 + 16 * pb + li;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const uint32_t w = e4m3_word_encode(hb[pb][nb][0] * inv, hb[pb][nb][1] * inv,
                                                    hb[pb][nb][2] * inv, hb[pb][nb][3] * inv);
                *reinterpret_cast<uint32_t*>(codes + ((long)nb * ROWS + p) * 16 + 4 * lg) = w;
            }
            if (lg == 0) static_cast<float*>(v.scale)[head * ROWS + p] = sc;
        }
    } else {
        const float st = amax_tile > 0.f ? fmaxf(amax_tile / 2688.f, kRcScaleFloorFp4Tile) : 1.f;
        const float d6 = 6.f * st;
        const float rd6 = 1.f / d6;  // correctly rounded, once per tile
        // The element codes take h * RN(1/S) with S = RN(value(sb) * st): with st fixed for the
        // tile, S and its reciprocal depend on the block-scale code alone, so the wave divides
        // once per code (two codes per lane) and every block looks its reciprocal up. Code 0
        // (S = 0) maps to 0; code 127 is NaN and never produced (block codes saturate at 448).
        wave_sync();  // this wave may have read the table's LDS just before
#pragma unroll
        for (int c = li + 16 * lg; c < 128; c += 64) {
            const float S = e4m3x2_decode_hw<false>((uint32_t)c).x * st;
            s_tab[c] = (c != 0 && c < 127) ? 1.f / S : 0.f;
        }
        wave_sync();
        uint8_t* codes = v.codes + head * (long)(ROWS * N / 2);
        uint8_t* sbp = static_cast<uint8_t*>(v.scale) + head * (long)ROWS * (N / 16);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const int p = row0 + 16 * pb + li;
            // every block's scale code first, then the table reads back to back, then the codes:
            // no branch between a table read and its use, so the reads share one wait
            uint32_t sb[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                float ab = fmaxf(fmaxf(fabsf(hb[pb][nb][0]), fabsf(hb[pb][nb][1])),
                                 fmaxf(fabsf(hb[pb][nb][2]), fabsf(hb[pb][nb][3])));
                ab = xor_reduce_max<16, 32>(ab);  // the 16-element block spans lanes li + 16 lg
                sb[nb] = block_scale_code(ab, d6, rd6);
            }
            float inv[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) inv[nb] = s_tab[sb[nb]];  // RN(1/S), 0 for sb == 0
            uint32_t sbw[(kNB + 3) / 4] = {};  // the row's block-scale codes, byte nb
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                // S > 0 exactly when sb != 0; a zero block's codes are 0 (not the -0 of h * 0)
                const uint32_t c = e2m1_half_encode(hb[pb][nb][0] * inv[nb], hb[pb][nb][1] * inv[nb],
                                                    hb[pb][nb][2] * inv[nb], hb[pb][nb][3] * inv[nb]);
                *reinterpret_cast<uint16_t*>(codes + ((long)(nb / 2) * ROWS + p) * 16 + 8 * (nb % 2) +
                                             2 * lg) = (uint16_t)(sb[nb] != 0u ? c : 0u);
                sbw[nb / 4] |= sb[nb] << (8 * (nb % 4));
            }
            if (lg == 0) {  // one store of the row's N/16 block-scale codes
                if constexpr (kNB == 8)
                    *reinterpret_cast<uint2*>(sbp + (long)p * (N / 16)) = make_uint2(sbw[0], sbw[1]);
                else
                    *reinterpret_cast<uint32_t*>(sbp + (long)p * (N / 16)) = sbw[0];
            }
        }
        if (tile_writer) v.tscale[head] = st;
    }
}

}  // namespace ssm
