// m2_kernels.hpp -- Mamba-2 ReplaySSM kernel templates for gfx950 (wave64). Instantiated by
// m2_decode.hip, m2_verify.hip, m2_fold.hip and m2_conv.hip (one translation unit each).
//
// Pages: "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding" -- the deskofai.com
// news article (paragraphs counted from the first body paragraph) and the nexus-ai-blog.com
// explainer (cited by section heading). The Mamba-2 recurrence is the published one (Dao & Gu,
// "Transformers are SSMs", 2024): h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T, y_t = h_t C_t + D x_t.
//
// Work decomposition. One wavefront owns one (sequence, head) pair; four heads per 256-thread
// workgroup. The P x N fp32 checkpoint tile is stored "quad-interleaved": element (p, n) at float
// ((n/4)*P + p)*4 + n%4. For P = 64 lane p therefore holds row p and every 16-byte load of the
// wave covers 1 KiB of contiguous memory; the row dot products h[p,:] . C need no cross-lane
// reduction. For P < 64 the wave holds 64/P copies of the rows, each lane group taking every
// (64/P)-th quad, and the groups are summed with shuffles at the end.
#pragma once
#include "rc_codec.hpp"
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

template <int P, int N> struct M2Geo {
    static_assert(P == 16 || P == 32 || P == 64, "Mamba-2 tile rows: 16, 32 or 64");
    static_assert(N == 16 || N == 32 || N == 64 || N == 128, "Mamba-2 tile columns: 16..128");
    static constexpr int kNQ = N / 4;     // 16-byte quads per row
    static constexpr int kGrp = 64 / P;   // lane groups (copies of the rows) per wave
    static constexpr int kQPL = kNQ / kGrp;  // quads per lane
    static_assert(kNQ % kGrp == 0, "N too small for P");
    static constexpr int kSeg = N / 4;    // B.C dot: elements per lane segment (4 segments)
};

constexpr int kHeadsPerBlock = 4;
constexpr int kMaxEntries = 64;  // ring entries a wave can address (cap <= 63)


// ---------------------------------------------------------------------------------------------
// Replay decode / speculative verify.
//
// For each query token j (entry index kq_j - 1 after the checkpoint, 0-based) the output is
//   y_j = e^{s0_j} h_c C_j + sum_{e < kq_j} e^{s_{e,j}} dt_e (B_e . C_j) x_e + D x_{kq_j - 1}
// with s_{e,j} = A * sum_{m = e+1 .. kq_j - 1} dt_m and s0_j = A * sum_{m < kq_j} dt_m
// (news, para 2: outputs from checkpoint + buffered inputs, no state write).
// Entries e < count come from the ring; entries count .. count+ntok-1 are this call's tokens,
// read from the caller's input; their x, B and dt rows are appended to the ring (news, para 3).
// C enters only its own token's output, so the ring does not keep it.
// COMMIT: decode (count += ntok at the end); otherwise the tokens stay pending drafts.
//
// Memory order matters here: the vector-memory counter retires in order, so every small load
// (pointers, dt, B segments, x rows, C) is issued BEFORE the checkpoint stream; the coefficient
// work then only waits for those, and the 32 KiB tile keeps streaming underneath it.
// MAXE bounds the entries a call can see (count + ntok <= MAXE).
// ---------------------------------------------------------------------------------------------
template <int P, int N, typename TIN, int RC, int MAXQ, int MAXE, bool COMMIT>
__global__ __launch_bounds__(256) void m2_replay_kernel(M2Args a) {
    using G = M2Geo<P, N>;
    constexpr int kEPC = 16 / (int)sizeof(TIN);          // elements per 16-byte chunk
    constexpr int kCPR = P / kEPC;                       // chunks per x row
    constexpr int kXL = (MAXE * kCPR + 63) / 64;         // x-row chunks per lane
    constexpr int kBCE = N / kEPC;                       // 16-byte chunks per B row
    constexpr int kBL = (MAXE * kBCE + 63) / 64;         // B chunks per lane
    static_assert(kBCE >= 2 && kBCE <= 64 && 64 % kBCE == 0, "B row chunks");
    constexpr int kCE = N >= 64 ? N / 64 : 1;            // C elements per lane
    static_assert(MAXE % 16 == 0 && MAXE <= 64, "MAXE");
    constexpr int kCS = N + 4;  // C row stride: the 4 rows an MFMA operand read takes hit distinct banks
    __shared__ __attribute__((aligned(16))) float s_c[kHeadsPerBlock][MAXQ][kCS];
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[kHeadsPerBlock][MAXE * kCPR];
    __shared__ __attribute__((aligned(16))) float s_w[kHeadsPerBlock][MAXE][MAXQ];

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * (int)(blockDim.x >> 6) + wave;  // one head per wave
    if (h >= a.heads) return;  // whole wave; no block-level barriers below
    const int b = blockIdx.y;
    const int head = b * a.heads + h;
    const int hpg = a.heads / a.groups;
    const int grp = h / hpg;
    const int bg = b * a.groups + grp;
    const int cap = a.cap, nq = a.ntok;
    const int H = a.heads, Gn = a.groups;

    const HeadPtr pt = head_ptr(a.ptr, a.hstart, a.hcount, head, b);
    const int start = pt.start;
    const int count = pt.count;
    const long th = a.share ? (long)pt.slot * H + h : head;  // this head's checkpoint tile
    const int kmax = count + nq;
    const float A = a.A[h];
    const float D = a.D[h];
    const int row = lane % P, gq = lane / P;

    const TIN* inx = static_cast<const TIN*>(a.in_x);
    const TIN* inB = static_cast<const TIN*>(a.in_B);
    const TIN* inC = static_cast<const TIN*>(a.in_C);
    TIN* rx = static_cast<TIN*>(a.ring_x);
    TIN* rB = static_cast<TIN*>(a.ring_B);

    // ---- 1. small loads (branch-free: invalid entries read a valid row and are masked later) -
    const long tok0 = (long)b * nq;  // this sequence's first token in the call's inputs
    // C of each query: lane holds elements n = lane + 64 i (N >= 64) or n = lane (N < 64)
    TIN craw[MAXQ][kCE];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
        const int jj = j < nq ? j : 0;
#pragma unroll
        for (int i = 0; i < kCE; ++i) {
            const int n = (lane + 64 * i) % N;
            craw[j][i] = inC[((tok0 + jj) * Gn + grp) * N + n];
        }
    }
    // dt of entry e = lane
    const float* dsrc = lane < count ? a.ring_dt + head * cap + ring_slot(start, min(lane, cap - 1), cap)
                                     : a.in_dt + (tok0 + min(max(lane - count, 0), nq - 1)) * H + h;
    float dte = *dsrc;
    dte = lane < kmax ? dte : 0.f;
    // B rows of every entry in 16-byte chunks, chunk idx = lane + 64 i -> (entry idx / kBCE,
    // part idx % kBCE): each load instruction covers whole rows, 1 KiB per ring run
    u32x4_t braw[kBL];
#pragma unroll
    for (int i = 0; i < kBL; ++i) {
        const int e = (lane + 64 * i) / kBCE, part = lane % kBCE;
        const TIN* src = e < count ? rB + ((long)bg * cap + ring_slot(start, min(e, cap - 1), cap)) * N
                                   : inB + ((tok0 + min(max(e - count, 0), nq - 1)) * Gn + grp) * N;
        braw[i] = *reinterpret_cast<const u32x4_t*>(src + part * kEPC);
    }
    // x rows of every entry, in 16-byte chunks: chunk idx -> (row e = idx / kCPR, part idx % kCPR)
    u32x4_t xraw[kXL];
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
        const int idx = lane + 64 * i;
        const int e = idx / kCPR, part = idx % kCPR;
        const TIN* src = e < count ? rx + ((long)head * cap + ring_slot(start, min(e, cap - 1), cap)) * P
                                   : inx + ((tok0 + min(max(e - count, 0), nq - 1)) * H + h) * P;
        xraw[i] = *reinterpret_cast<const u32x4_t*>(src + part * kEPC);
    }

    // ---- 2. the checkpoint stream (explainer, "Why Decoding, Not Prefill, Is the Hard Part":
    //         decode time goes to reading the state) ----------------------------------------
    // Several queries (verify): half of the tile is issued here and half before the row dots,
    // so that the coefficient work does not hold all the tile registers and more waves fit on a
    // SIMD.
    constexpr int kEarlyQ = RC == 0 ? G::kQPL / 2 : G::kQPL;
    float4 hv[G::kQPL];
    const float4* tile = reinterpret_cast<const float4*>(a.ckpt) + th * (P * N / 4);
    if constexpr (RC == 0) {
        // issued in the order the row dots use them (the scheduler would otherwise reorder the
        // loads, and the first dot would wait for the whole tile): the dots then run while the
        // rest of the tile is still arriving
#pragma unroll
        for (int j = 0; j < kEarlyQ; ++j) {
            hv[j] = ld_stream(tile + (gq + G::kGrp * j) * P + row);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("" ::: "memory");  // keep every staging store below the stream issue
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. stage C and x rows in LDS; append this call's tokens to the rings ---------------
    // (every staging store is unconditional so that no load can be sunk past the stream)
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
#pragma unroll
        for (int i = 0; i < kCE; ++i) s_c[wave][j][(lane + 64 * i) % N] = to_f32<TIN>(craw[j][i]);
    }
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
        const int idx = lane + 64 * i;
        if (kXL * 64 == MAXE * kCPR || idx < MAXE * kCPR) s_x[wave][idx] = xraw[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    // appends and outputs go through write-through stores (the appends also streaming beside a
    // read copy)
    constexpr int kPol = RC == 0 ? kStoreWT : kStoreWTNT;
    const PolicyStore xring(rx + uniform64((long)head * cap * P), (uint32_t)(cap * P * sizeof(TIN)));
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
        const int idx = lane + 64 * i;
        const int e = idx / kCPR, part = idx % kCPR;
        if (e >= count && e < kmax)  // this call's token: append its x row
            xring.template bytes<kPol, 16>((uint32_t)((ring_slot(start, e, cap) * P + part * kEPC) * sizeof(TIN)),
                                           &xraw[i]);
    }
    if (lane >= count && lane < kmax) a.ring_dt[head * cap + ring_slot(start, lane, cap)] = dte;
    if (h % hpg == 0) {  // the group's first head writes the shared B entries
        const PolicyStore bring(rB + uniform64((long)bg * cap * N), (uint32_t)(cap * N * sizeof(TIN)));
#pragma unroll
        for (int i = 0; i < kBL; ++i) {
            const int e = (lane + 64 * i) / kBCE, part = lane % kBCE;
            if (e >= count && e < kmax)
                bring.template bytes<kPol, 16>((uint32_t)((ring_slot(start, e, cap) * N + part * kEPC) * sizeof(TIN)),
                                               &braw[i]);
        }
    }
    wave_sync();

    // ---- 4. replay weights w_{e,j} and checkpoint decays e^{s0_j} ---------------------------
    // Inclusive prefix sums of dt over the entries, pre(e) = sum_{m <= e} dt_m (zero past kmax):
    // the decay exponent from entry e to query j is A (pre(kq_j - 1) - pre(e)).
    float pre = dte;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(pre, o, 64);
        pre += lane >= o ? t : 0.f;
    }
    float tot[MAXQ], s0[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
        tot[j] = readlane(pre, min(count + j, 63));  // uniform index: entries 0 .. kq_j - 1
        s0[j] = j < nq ? expf(A * tot[j]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kBL; ++i) {
        if (i * (64 / kBCE) >= kmax) continue;  // uniform: no entry of this chunk is in use
        const int e = (lane + 64 * i) / kBCE, part = lane % kBCE;
        float bf[kEPC];
        Unit<TIN>::unpack(make_uint4(braw[i].x, braw[i].y, braw[i].z, braw[i].w), bf);
        const float dt_e = __shfl(dte, e & 63, 64);
        const float pre_e = __shfl(pre, e & 63, 64);
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
            if (j >= nq) break;
            const float* cj = &s_c[wave][j][part * kEPC];
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < kEPC; ++t) d += bf[t] * cj[t];
            d = group_sum<kBCE>(d);
            // sum of dt over entries e+1 .. kq-1 with kq = count + j + 1
            const float w = (e <= count + j) ? expf(A * (tot[j] - pre_e)) * dt_e * d : 0.f;
            if (part == 0 && e < MAXE) s_w[wave][e][j] = w;
        }
    }
    wave_sync();

    // ---- 5. buffered-input and skip terms (LDS only) -----------------------------------------
    float out[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) out[j] = 0.f;
    const TIN* sx = reinterpret_cast<const TIN*>(&s_x[wave][0]);
    // four entries at a time, so that the LDS reads of a group go out together; the weights of
    // entries past kmax are not written, and the select keeps them out of the sum
    for (int e0 = 0; e0 < kmax; e0 += 4) {  // uniform; MAXE is a multiple of 16
        float xe[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xe[u] = to_f32<TIN>(sx[(e0 + u) * P + row]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u;
#pragma unroll
            for (int j = 0; j < MAXQ; ++j) {
                const float t = s_w[wave][e][j] * xe[u];
                out[j] += e <= count + j ? t : 0.f;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < MAXQ; ++j)  // skip term of the query's own token
        out[j] += D * to_f32<TIN>(sx[min(count + j, MAXE - 1) * P + row]);

    if constexpr (RC == 0 && kEarlyQ < G::kQPL) {
#pragma unroll
        for (int j = kEarlyQ; j < G::kQPL; ++j) {
            hv[j] = ld_stream(tile + (gq + G::kGrp * j) * P + row);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- 6. checkpoint row dots h_c[p,:] . C_j -------------------------------------------------
    float acc[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) acc[j] = 0.f;
    if constexpr (RC == 0 && P == 64 && MAXQ >= 4) {
        // several queries: four queries per 4x4x1 MFMA (lane p = row p; query j = 4g + lane%4
        // supplies its C column), two accumulator chains per group of four
        constexpr int kG = MAXQ / 4;
        f32x4 dq[kG][2];
#pragma unroll
        for (int g = 0; g < kG; ++g) dq[g][0] = dq[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < G::kQPL; ++q) {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const float4 c4 = *reinterpret_cast<const float4*>(&s_c[wave][4 * g + (lane & 3)][4 * q]);
                f32x4& d = dq[g][q & 1];
                d = mfma4x4(c4.x, hv[q].x, d);
                d = mfma4x4(c4.y, hv[q].y, d);
                d = mfma4x4(c4.z, hv[q].z, d);
                d = mfma4x4(c4.w, hv[q].w, d);
            }
        }
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) acc[j] = dq[j / 4][0][j % 4] + dq[j / 4][1][j % 4];
    } else if constexpr (RC == 0) {
#pragma unroll
        for (int jq = 0; jq < G::kQPL; ++jq) {
            const int q = gq + G::kGrp * jq;
#pragma unroll
            for (int j = 0; j < MAXQ; ++j) {
                if (j >= nq) break;
                const float4 c4 = *reinterpret_cast<const float4*>(&s_c[wave][j][4 * q]);
                acc[j] += hv[jq].x * c4.x + hv[jq].y * c4.y + hv[jq].z * c4.z + hv[jq].w * c4.w;
            }
        }
    } else {
        RcRow<P, N, RC> rc;  // the read copy's row (news, para 4: reads from the copy)
        rc.load(RcView{a.rc_codes, a.rc_scale, a.rc_tscale}, th, row);
        rc.template dots<kCS, MAXQ>(nq, &s_c[wave][0][0], acc);
    }
    if constexpr (G::kGrp > 1) {
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) acc[j] = xor_reduce_sum<P, 32>(acc[j]);
    }
    if (gq == 0) {
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
            if (j >= nq) break;
            const PolicyStore yrow(a.y + uniform64((((long)b * nq + j) * H + h) * P), P * 4);
            const float yv = s0[j] * acc[j] + out[j];
            yrow.template bytes<kStoreWT, 4>((uint32_t)(row * 4), &yv);
        }
    }
    if constexpr (COMMIT) {
        if (lane == 0) a.ptr[kPtrInts * head + 1] = count + nq;
    }
}

// ---------------------------------------------------------------------------------------------
// Fold (flush): fold the oldest nfold committed entries into the checkpoint (news, para 3):
//   h_c <- e^{s0} h_c + sum_{e < nfold} e^{s_e} dt_e x_e B_e^T,  s_e = A sum_{m=e+1..nfold-1} dt_m
// a rank-nfold update, run on fp32 MFMA (v_mfma_f32_16x16x4f32) with the tile held in accumulator
// order: lane l owns row 16 pb + l%16 and the quad 4 nb + l/16 of every 16x16 block (pb, nb), so
// D[n][p] += sum_k B_k[n] a_k[p] with A = B-ring values and B = a_k[p] = e^{s_k} dt_k x_k[p].
// Not FUSED: nfold = L when count >= L (IF_FULL), = count (ALL), else nothing; rewrite_only
//   only rewrites the read copy (init). start += nfold, count -= nfold.
// FUSED: the L-th token of a lock-step decode (count == L-1 for every sequence): the token's own
//   inputs come from the caller and are folded with the L-1 buffered entries at once, its output
//   is y = h_new C + D x (the recurrence's own form), and the ring is left empty. This saves the
//   separate replay pass over the checkpoint on that step.
// The read copy (news, para 4) is rewritten from the new fp32 checkpoint in the same pass.
// ---------------------------------------------------------------------------------------------
template <int P, int N, typename TIN, int RC, bool FUSED>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2))) void m2_fold_kernel(M2Args a, int mode_all, int rewrite_only) {
    constexpr int kPB = P / 16, kNB = N / 16;
    constexpr int kEPC = 16 / (int)sizeof(TIN);
    constexpr int kBCR = N / kEPC;                 // 16-byte chunks per B row
    constexpr int kBL = (16 * kBCR + 63) / 64;     // B chunks per lane (16 rows)
    constexpr int kXCR = P / kEPC;                 // chunks per x row
    constexpr int kXL = (16 * kXCR + 63) / 64;
    constexpr int kBP = N + 16;                    // padded LDS row: the 4 rows an MFMA reads
    constexpr int kCE = N >= 64 ? N / 64 : 1;      //   land in disjoint banks
    __shared__ __attribute__((aligned(16))) float s_b[kHeadsPerBlock][16][kBP];
    __shared__ __attribute__((aligned(16))) u32x4_t s_x[kHeadsPerBlock][16 * kXCR];
    __shared__ __attribute__((aligned(16))) float s_c[kHeadsPerBlock][FUSED ? N : 4];

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * (int)(blockDim.x >> 6) + wave;  // one head per wave
    if (h >= a.heads) return;
    const int b = blockIdx.y;
    const int H = a.heads;
    const int head = b * H + h;
    const int grp = h / (H / a.groups);
    const int bg = b * a.groups + grp;
    const int cap = a.cap;
    const HeadPtr pt = head_ptr(a.ptr, a.hstart, a.hcount, head, b);
    const int start = pt.start;
    const int count = pt.count;
    const int slot = pt.slot;
    // copy-on-write of a shared checkpoint: a sequence that must move folds whatever it holds
    const FoldTarget ft = fold_target(a.refcnt, a.share, a.batch, b, slot);
    int nfold, nring;
    if constexpr (FUSED) {
        nfold = count + 1;  // the buffered entries and this token
        nring = count;
    } else {
        nfold = rewrite_only ? 0 : (mode_all ? count : (count >= a.window ? a.window : (ft.move ? count : 0)));
        if (nfold == 0 && !rewrite_only && !ft.move) return;
        nring = nfold;
    }
    const int li = lane & 15, lg = lane >> 4;
    const TIN* rx = static_cast<const TIN*>(a.ring_x);
    const TIN* rB = static_cast<const TIN*>(a.ring_B);
    const long tok = (long)b * H + h;  // FUSED: this token's row of the [batch][1][H] inputs

    // entry e's rows: ring slot for e < nring, the caller's token otherwise (FUSED), clamped to a
    // folded entry past nfold (those rows are zeroed in LDS)
    auto brow = [&](int e) -> const TIN* {
        if (FUSED && e >= nring)
            return static_cast<const TIN*>(a.in_B) + ((long)b * a.groups + grp) * N;
        return rB + ((long)bg * cap + ring_slot(start, min(e, max(nring - 1, 0)), cap)) * N;
    };
    auto xrow = [&](int e) -> const TIN* {
        if (FUSED && e >= nring) return static_cast<const TIN*>(a.in_x) + tok * P;
        return rx + ((long)head * cap + ring_slot(start, min(e, max(nring - 1, 0)), cap)) * P;
    };
    u32x4_t braw[kBL], xraw[kXL];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kBL; ++i) {
            const int idx = (lane + 64 * i) % (16 * kBCR);
            braw[i] = *reinterpret_cast<const u32x4_t*>(brow(c0 + idx / kBCR) + (idx % kBCR) * kEPC);
        }
#pragma unroll
        for (int i = 0; i < kXL; ++i) {
            const int idx = (lane + 64 * i) % (16 * kXCR);
            xraw[i] = *reinterpret_cast<const u32x4_t*>(xrow(c0 + idx / kXCR) + (idx % kXCR) * kEPC);
        }
    };
    float dte;
    {
        const float* src = (FUSED && lane >= nring)
                               ? a.in_dt + tok
                               : a.ring_dt + (long)head * cap + ring_slot(start, min(lane, cap - 1), cap);
        dte = *src;
        dte = lane < nfold ? dte : 0.f;
    }
    const float A = a.A[h];  // before the stream: a later load would wait for all of it
    const float D = FUSED ? a.D[h] : 0.f;
    TIN craw[kCE];
    if constexpr (FUSED) {
        const TIN* inC = static_cast<const TIN*>(a.in_C) + ((long)b * a.groups + grp) * N;
#pragma unroll
        for (int i = 0; i < kCE; ++i) craw[i] = inC[(lane + 64 * i) % N];
    }
    if (nfold > 0) fetch(0);

    f32x4 hb[kPB][kNB];
    // float4 (4 nb + lg) * P + 16 pb + li of the head's tile: read from its slot, written to the
    // fold target's
    const long th = a.share ? (long)slot * H + h : head;
    const long tw = a.share ? (long)ft.wr * H + h : head;
    const TileIO tio{reinterpret_cast<char*>(a.ckpt) + th * (P * N * 4),
                     (uint32_t)((lg * P + li) * 16)};
    const TileIO tiow{reinterpret_cast<char*>(a.ckpt) + tw * (P * N * 4), tio.lane};
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const float4 t = tio.load((uint32_t)((4 * nb * P + 16 * pb) * 16));
            hb[pb][nb] = f32x4{t.x, t.y, t.z, t.w};
        }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    if (nfold > 0) {
        float pre = dte;  // inclusive prefix sum of dt; the suffix after lane's entry is tot - pre
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float t = __shfl_up(pre, o, 64);
            pre += lane >= o ? t : 0.f;
        }
        const float tot = readlane(pre, nfold - 1);
        const float ue = expf(A * (tot - pre)) * dte;  // zero past nfold
        const float e0 = expf(A * tot);
        if constexpr (FUSED) {
#pragma unroll
            for (int i = 0; i < kCE; ++i) s_c[wave][(lane + 64 * i) % N] = to_f32<TIN>(craw[i]);
        }
        for (int c0 = 0; c0 < nfold; c0 += 16) {
            if (c0 > 0) fetch(c0);
            const int nc = min(16, nfold - c0);
#pragma unroll
            for (int i = 0; i < kBL; ++i) {
                const int idx = lane + 64 * i;
                if (idx < 16 * kBCR) {
                    const int r = idx / kBCR, part = idx % kBCR;
                    float f[kEPC];
                    Unit<TIN>::unpack(make_uint4(braw[i].x, braw[i].y, braw[i].z, braw[i].w), f);
#pragma unroll
                    for (int k = 0; k < kEPC; ++k) s_b[wave][r][part * kEPC + k] = r < nc ? f[k] : 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < kXL; ++i) {
                const int idx = lane + 64 * i;
                if (idx < 16 * kXCR) s_x[wave][idx] = xraw[i];
            }
            wave_sync();
            if (c0 == 0) {  // decay of the old checkpoint, applied once the staging is done
#pragma unroll
                for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) hb[pb][nb] *= e0;
            }
            const TIN* sx = reinterpret_cast<const TIN*>(&s_x[wave][0]);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (4 * g >= nc) break;
                const int ek = 4 * g + lg;                       // this lane's k-slot entry
                const float uk = __shfl(ue, (c0 + ek) & 63, 64);  // per-lane entry: shuffle
                float aop[kPB], bop[kNB];
#pragma unroll
                for (int pb = 0; pb < kPB; ++pb) aop[pb] = uk * to_f32<TIN>(sx[ek * P + 16 * pb + li]);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) bop[nb] = s_b[wave][ek][16 * nb + li];
#pragma unroll
                for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) hb[pb][nb] = mfma4(bop[nb], aop[pb], hb[pb][nb]);
            }
            wave_sync();
        }
    }
    if (nfold > 0 || ft.move) {
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
                tiow.store((uint32_t)((4 * nb * P + 16 * pb) * 16),
                           make_float4(hb[pb][nb][0], hb[pb][nb][1], hb[pb][nb][2], hb[pb][nb][3]));
    }
    if constexpr (FUSED) {  // output from the new state: y = h C + D x
        const TIN* xin = static_cast<const TIN*>(a.in_x) + tok * P;
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) {
            float part = 0.f;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const float4 c4 = *reinterpret_cast<const float4*>(&s_c[wave][16 * nb + 4 * lg]);
                part += hb[pb][nb][0] * c4.x + hb[pb][nb][1] * c4.y + hb[pb][nb][2] * c4.z +
                        hb[pb][nb][3] * c4.w;
            }
            part = xor_reduce_sum<16, 32>(part);
            if (lg == 0) {
                const int p = 16 * pb + li;
                a.y[tok * P + p] = part + D * to_f32<TIN>(xin[p]);
            }
        }
    }
    if constexpr (RC != 0) {
        static_assert(P == 64, "read copy needs P == 64");
        const float amax_t = RC == 2 ? xor_reduce_max<1, 32>(rc_local_amax<N>(hb)) : 0.f;
        rc_write_blocks<P, N, RC>(RcView{a.rc_codes, a.rc_scale, a.rc_tscale}, tw, 0, li, lg, hb,
                                  amax_t, lane == 0, &s_b[wave][0][0]);  // (staging is done)
    }
    if ((nfold > 0 || ft.move) && lane == 0)
        *reinterpret_cast<int4*>(a.ptr + kPtrInts * head) =
            make_int4(ring_slot(start, nfold, cap), (FUSED ? count + 1 : count) - nfold, ft.wr, 0);
}

// ---------------------------------------------------------------------------------------------
// Conventional step (the comparison point; news, para 3 -- the full state rewritten per token):
//   h <- exp(dt A) h + dt x B^T (in place), y = h C + D x.
// ---------------------------------------------------------------------------------------------
template <int P, int N, typename TIN>
__global__ __launch_bounds__(256) void m2_conv_kernel(M2ConvArgs a) {
    using G = M2Geo<P, N>;
    constexpr int kCE = N >= 64 ? N / 64 : 1;
    __shared__ __attribute__((aligned(16))) float s_bc[kHeadsPerBlock][2][N];
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * (int)(blockDim.x >> 6) + wave;  // one head per wave
    if (h >= a.heads) return;
    const int b = blockIdx.y;
    const int head = b * a.heads + h;
    const int grp = h / (a.heads / a.groups);
    const int row = lane % P, gq = lane / P;

    const TIN* inB = static_cast<const TIN*>(a.in_B) + ((long)b * a.groups + grp) * N;
    const TIN* inC = static_cast<const TIN*>(a.in_C) + ((long)b * a.groups + grp) * N;
    TIN braw[kCE], craw[kCE];
#pragma unroll
    for (int i = 0; i < kCE; ++i) {
        const int n = (lane + 64 * i) % N;
        braw[i] = inB[n];
        craw[i] = inC[n];
    }
    const float dt = a.in_dt[head];
    const TIN xraw = static_cast<const TIN*>(a.in_x)[(long)head * P + row];
    const float A = a.A[h], D = a.D[h];

    float4 hv[G::kQPL];
    // float4 (gq + kGrp j) * P + row of the head's tile
    const TileIO tio{reinterpret_cast<char*>(a.h) + (long)head * (P * N * 4),
                     (uint32_t)((gq * P + row) * 16)};
    // issued in the order the update uses them, so that it runs while the tile arrives
#pragma unroll
    for (int j = 0; j < G::kQPL; ++j) {
        hv[j] = tio.load((uint32_t)(G::kGrp * j * P * 16));
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < kCE; ++i) {
        const int n = (lane + 64 * i) % N;
        s_bc[wave][0][n] = to_f32<TIN>(braw[i]);
        s_bc[wave][1][n] = to_f32<TIN>(craw[i]);
    }
    const float decay = expf(dt * A);
    const float x = to_f32<TIN>(xraw);
    const float dx = dt * x;
    wave_sync();
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < G::kQPL; ++j) {
        const int q = gq + G::kGrp * j;
        const float4 b4 = *reinterpret_cast<const float4*>(&s_bc[wave][0][4 * q]);
        const float4 c4 = *reinterpret_cast<const float4*>(&s_bc[wave][1][4 * q]);
        hv[j].x = decay * hv[j].x + dx * b4.x;
        hv[j].y = decay * hv[j].y + dx * b4.y;
        hv[j].z = decay * hv[j].z + dx * b4.z;
        hv[j].w = decay * hv[j].w + dx * b4.w;
        acc += hv[j].x * c4.x + hv[j].y * c4.y + hv[j].z * c4.z + hv[j].w * c4.w;
        tio.store((uint32_t)(G::kGrp * j * P * 16), hv[j]);
    }
    if constexpr (G::kGrp > 1) acc = xor_reduce_sum<P, 32>(acc);
    if (gq == 0) a.y[(long)head * P + row] = acc + D * x;
}

// ---------------------------------------------------------------------------------------------
// Snapshot-based speculative step (the comparison point for the speculative verify; news, para 3
// -- per-token snapshots): the recurrence of m2_conv_kernel over ntok <= MAXQ draft tokens from
// the read-only state a.h, writing the state after each draft to its own snapshot tile
// (a.snap + (j * batch * H + head) * P * N) and y [batch][ntok][H][P].
// ---------------------------------------------------------------------------------------------
template <int P, int N, typename TIN, int MAXQ>
__global__ __launch_bounds__(256) void m2_snap_kernel(M2ConvArgs a) {
    using G = M2Geo<P, N>;
    constexpr int kCE = N >= 64 ? N / 64 : 1;
    __shared__ __attribute__((aligned(16))) float s_bc[kHeadsPerBlock][MAXQ][2][N];
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * (int)(blockDim.x >> 6) + wave;  // one head per wave
    if (h >= a.heads) return;
    const int b = blockIdx.y;
    const int H = a.heads, Gn = a.groups, nq = a.ntok;
    const int head = b * H + h;
    const int grp = h / (H / Gn);
    const int row = lane % P, gq = lane / P;

    const TIN* inB = static_cast<const TIN*>(a.in_B);
    const TIN* inC = static_cast<const TIN*>(a.in_C);
    const TIN* inx = static_cast<const TIN*>(a.in_x);
    TIN braw[MAXQ][kCE], craw[MAXQ][kCE], xraw[MAXQ];
    float dtj[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
        const long tok = (long)b * nq + (j < nq ? j : 0);  // clamped: padded drafts are unused
#pragma unroll
        for (int i = 0; i < kCE; ++i) {
            const int n = (lane + 64 * i) % N;
            braw[j][i] = inB[(tok * Gn + grp) * N + n];
            craw[j][i] = inC[(tok * Gn + grp) * N + n];
        }
        xraw[j] = inx[(tok * H + h) * P + row];
        dtj[j] = a.in_dt[tok * H + h];
    }
    const float A = a.A[h], D = a.D[h];

    float4 hv[G::kQPL];
    const uint32_t lane_off = (uint32_t)((gq * P + row) * 16);
    const TileIO tin{reinterpret_cast<char*>(a.h) + (long)head * (P * N * 4), lane_off};
#pragma unroll
    for (int j = 0; j < G::kQPL; ++j) hv[j] = tin.load((uint32_t)(G::kGrp * j * P * 16));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < MAXQ; ++j)
#pragma unroll
        for (int i = 0; i < kCE; ++i) {
            const int n = (lane + 64 * i) % N;
            s_bc[wave][j][0][n] = to_f32<TIN>(braw[j][i]);
            s_bc[wave][j][1][n] = to_f32<TIN>(craw[j][i]);
        }
    wave_sync();
    const long nheads = (long)a.batch * H;
#pragma unroll
    for (int t = 0; t < MAXQ; ++t) {
        if (t >= nq) break;
        const float decay = expf(dtj[t] * A);
        const float x = to_f32<TIN>(xraw[t]);
        const float dx = dtj[t] * x;
        const TileIO tout{reinterpret_cast<char*>(a.snap) + ((long)t * nheads + head) * (P * N * 4),
                          lane_off};
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < G::kQPL; ++j) {
            const int q = gq + G::kGrp * j;
            const float4 b4 = *reinterpret_cast<const float4*>(&s_bc[wave][t][0][4 * q]);
            const float4 c4 = *reinterpret_cast<const float4*>(&s_bc[wave][t][1][4 * q]);
            hv[j].x = decay * hv[j].x + dx * b4.x;
            hv[j].y = decay * hv[j].y + dx * b4.y;
            hv[j].z = decay * hv[j].z + dx * b4.z;
            hv[j].w = decay * hv[j].w + dx * b4.w;
            acc += hv[j].x * c4.x + hv[j].y * c4.y + hv[j].z * c4.z + hv[j].w * c4.w;
            tout.store((uint32_t)(G::kGrp * j * P * 16), hv[j]);
        }
        if constexpr (G::kGrp > 1) acc = xor_reduce_sum<P, 32>(acc);
        if (gq == 0) a.y[(((long)b * nq + t) * H + h) * P + row] = acc + D * x;
    }
}

// ---------------------------------------------------------------------------------------------
// Launch helpers shared by the instantiating translation units. One wavefront per head; four
// heads per workgroup, or one when the launch has at most two heads per CU (B * H <= 512 on 256
// CUs): then the heads spread over the CUs instead of sharing the load paths of a quarter of
// them. Grid: (ceil(H / heads per workgroup), batch).
// ---------------------------------------------------------------------------------------------
constexpr long kSmallLaunchHeads = 512;
static inline int heads_per_block(int batch, int heads) {
    return (long)batch * heads <= kSmallLaunchHeads ? 1 : kHeadsPerBlock;
}
static inline dim3 head_grid(int batch, int heads) {
    const int hpb = heads_per_block(batch, heads);
    return dim3((unsigned)((heads + hpb - 1) / hpb), (unsigned)batch);
}
static inline dim3 head_block(int batch, int heads) {
    return dim3((unsigned)(64 * heads_per_block(batch, heads)));
}

#ifdef SSM_SINGLE_SHAPE  // faster builds when inspecting the serving-shape kernels
#define SSM_M2_SHAPES(X, ...) X(64, 128, __VA_ARGS__)
#else
#define SSM_M2_SHAPES(X, ...)                                                                   \
    X(16, 16, __VA_ARGS__) X(16, 32, __VA_ARGS__) X(16, 64, __VA_ARGS__)                       \
    X(16, 128, __VA_ARGS__) X(32, 32, __VA_ARGS__) X(32, 64, __VA_ARGS__)                      \
    X(32, 128, __VA_ARGS__) X(32, 16, __VA_ARGS__) X(64, 16, __VA_ARGS__)                      \
    X(64, 32, __VA_ARGS__) X(64, 64, __VA_ARGS__) X(64, 128, __VA_ARGS__)
#endif

// Speculative verify launches (m2_verify.hip); m2_launch_replay forwards multi-token calls here.
hipError_t m2_launch_verify(const M2Args& a, int P, int N, int bf16, int rc, int maxe, hipStream_t s);

}  // namespace ssm
