// gdn_kernels.hpp -- Gated DeltaNet ReplaySSM kernel templates for gfx950 (wave64). Instantiated
// by gdn_decode.hip, gdn_verify.hip, gdn_flush.hip and gdn_conv.hip (one translation unit each).
//
// Pages: "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding" (news article, paras
// 2-3: checkpoint plus buffered inputs, outputs without a state write, fold when the buffer fills;
// the layer type is named in para 7 and in the feed excerpt). The recurrence is the published gated
// delta rule (Yang, Kautz & Hatamizadeh, 2025), per head with S in R^{dv x dk}, alpha = exp(g):
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = scale S_t q_t.
//
// Work decomposition: one workgroup of dv/64 wavefronts (two for dv = 128) per (sequence, head).
// The checkpoint uses the same quad-interleaved tile as Mamba-2 (element (p, n) at float
// ((n/4)*dv + p)*4 + n%4), so in replay and in the conventional step lane p of wave w owns row
// p = 64w + lane and every row product with a dk-vector runs inside one lane. The flush holds the
// tile in fp32 MFMA accumulator order instead (16x16 blocks: lane l owns row 16*pb + l%16 and the
// quad 4*nb + l/16), which is the same memory layout read with a different lane map.
#pragma once
#include "rc_codec.hpp"
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

constexpr int kGdnMaxWin = 32;  // most entries a replay call can see
// The flush and conventional kernels write their whole 64 KiB state tiles through write-through
// streaming stores: measured 1-2% faster for them than non-temporal ones. The snapshot kernel
// (its stores interleave with each draft's output) and the Mamba-2 kernels' 32 KiB tiles measured
// no gain and keep non-temporal stores.
constexpr int kTileStorePol = kStoreWTNT;

// ---------------------------------------------------------------------------------------------
// Replay decode / speculative verify. With entries 1..k after the checkpoint (entry k = the query's
// own token), each query's output is
//   r <- q_k, acc <- 0; for i = k..1: c_i = beta_i (k_i . r), acc += c_i v_i, r <- alpha_i (r - c_i k_i)
//   o = scale (S_c r + acc)
// which is the delta-rule recurrence unrolled k times (each step maps the query through
// alpha_i (I - beta_i k_i k_i^T) and emits beta_i (k_i . r) v_i). This call's ntok tokens are
// entries count+1 .. count+ntok (news, para 3: drafts are appended to the buffer); query j sees
// the committed entries and tokens 0..j. All queries share one read of the checkpoint rows.
// COMMIT (decode): count += ntok at the end; otherwise the tokens stay pending drafts.
// MAXW bounds the entries a call sees (count + ntok <= MAXW), MAXQ the tokens per call.
// VG (Kimi Delta Attention): alpha_i is a dk-vector (one decay per key channel), so the sweep's
// decay is elementwise: r <- alpha_i * (r - c_i k_i); g rings and inputs hold dk values per entry.
// ---------------------------------------------------------------------------------------------
template <int DV, int DK, typename TIN, int RC, int MAXW, int MAXQ, bool COMMIT, bool VG = false>
__global__ __launch_bounds__(64 * (DV >= 64 ? DV / 64 : 1))
__attribute__((amdgpu_waves_per_eu(2))) void gdn_replay_kernel(GdnArgs a) {
    static_assert(DV >= 64 && DK >= 64, "replay tile: dv, dk >= 64");
    static_assert(MAXW <= 64 && MAXW % 4 == 0, "entries per call");
    constexpr int kW = DV / 64;                   // wavefronts per head
    constexpr int kRows = 64;                     // rows per wave
    constexpr int kNQ = DK / 4;
    constexpr int kE = DK / 64;                   // key elements per lane in the sweep
    constexpr int kEPC = 16 / (int)sizeof(TIN);
    constexpr int kVC = kRows / kEPC;             // 16-byte chunks of a wave's v slice
    constexpr int kVL = (MAXW * kVC + 63) / 64;
    constexpr int kRS = DK + 4;  // r row stride: the 4 rows an MFMA operand read takes hit distinct banks
    // The waves of a head split the staging of the entries (entry e by wave e % kW) into shared
    // keys and decays. With several queries, or with a read copy, they also split the sweeps
    // (query j by wave j % kW) and share the swept r_j and coefficients: a single query is then
    // swept by wave 0 while the others wait at the barrier, which saves the repeated sweep's
    // instructions where the copy's short row stream leaves the kernel bound by instruction issue.
    // Without a copy the state stream bounds the kernel, and every wave sweeps a single query
    // itself rather than wait for another.
    static_assert(MAXW % kW == 0, "entries split over the head's waves");
    constexpr bool kSplit = kW > 1 && (MAXQ > 1 || RC != 0);
    constexpr int kQS = kSplit ? (MAXQ + kW - 1) / kW : MAXQ;  // queries this wave sweeps
    constexpr int kSW = kSplit ? 1 : kW;                       // copies of r and c
    constexpr int kEW = MAXW / kW;                             // entries this wave stages
    __shared__ __attribute__((aligned(16))) float s_r[kSW][MAXQ][kRS];
    __shared__ __attribute__((aligned(16))) u32x4_t s_v[kW][MAXW * kVC];
    __shared__ __attribute__((aligned(16))) float s_c[kSW][MAXW][MAXQ];
    __shared__ __attribute__((aligned(16))) TIN s_k[MAXW][DK];  // keys, as loaded
    __shared__ __attribute__((aligned(16))) float s_al[VG ? MAXW : 1][VG ? DK : 4];  // VG: alpha

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x, b = blockIdx.y;
    const int H = a.heads;
    const int head = b * H + h;
    const int cap = a.cap, nq = a.ntok;
    const HeadPtr pt = head_ptr(a.ptr, a.hstart, a.hcount, head, b);
    const int start = pt.start, count = pt.count;
    const long th = a.share ? (long)pt.slot * H + h : head;  // this head's checkpoint tile
    const int kmax = count + nq;
    const long rh = uniform64((long)head * cap);      // this head's first ring row
    const long t0 = uniform64((long)b * nq * H + h);  // this call's token 0 in the inputs
    // row of token j (clamped to the call's tokens) in the [batch][ntok][H] inputs
    auto tok = [&](int j) -> long { return t0 + (long)min(max(j, 0), nq - 1) * H; };
    // first element of entry e's row (wave-uniform e) in a ring or in this call's inputs, held in
    // scalar registers so that each lane adds only its own element offset
    // (offsets, not the pointers, go through uniform64: the pointers keep their global address
    // space, so the loads stay global loads with a scalar base)
    auto erow = [&](auto* ring, auto* in, int e, int w) {
        return e < count ? ring + uniform64((rh + ring_slot(start, min(e, cap - 1), cap)) * w)
                         : in + uniform64(tok(e - count) * w);
    };
    // the same for a per-lane entry e: a scalar base on each side (this head's ring rows, this
    // call's token 0) and a 32-bit element offset per lane (the host bounds heads * w * ntok)
    auto lrow = [&](auto* ring, auto* in, int e, int w) {
        const bool r = e < count;
        const unsigned o = r ? (unsigned)(ring_slot(start, min(e, cap - 1), cap) * w)
                             : (unsigned)min(max(e - count, 0), nq - 1) * (unsigned)(H * w);
        return (r ? ring + uniform64(rh * w) : in + uniform64(t0 * w)) + o;
    };
    // appends and outputs go through write-through stores (the appends also streaming beside a
    // read copy), each through a resource over this head's ring rows or one output row
    constexpr int kPol = RC == 0 ? kStoreWT : kStoreWTNT;
    const PolicyStore kring(static_cast<TIN*>(a.ring_k) + uniform64(rh * DK), (uint32_t)(cap * DK * sizeof(TIN)));
    const PolicyStore gring(a.ring_g + uniform64(rh * (VG ? DK : 1)), (uint32_t)(cap * (VG ? DK : 1) * 4));
    const TIN* rk = static_cast<const TIN*>(a.ring_k);
    const TIN* rv = static_cast<const TIN*>(a.ring_v);
    const TIN* inq = static_cast<const TIN*>(a.in_q);
    const TIN* ink = static_cast<const TIN*>(a.in_k);
    const TIN* inv = static_cast<const TIN*>(a.in_v);
    const int row = wave * kRows + lane;

    // ---- small loads first (in-order memory counter; branch-free, masked later) ---------------
    const int el = lane;  // lane's key elements: [el*kE, el*kE + kE)
    float be = 0.f, ge = 0.f;  // beta, g of entry e = lane
    {
        be = *lrow(a.ring_beta, a.in_beta, lane, 1);
        be = lane < kmax ? be : 0.f;
        if constexpr (!VG) {
            ge = *lrow(a.ring_g, a.in_g, lane, 1);
            ge = lane < kmax ? ge : 0.f;
        }
    }
    // keys of this wave's entries e = ee kW + wave (entries >= count are this call's tokens)
    TIN kraw[kEW][kE];
#pragma unroll
    for (int ee = 0; ee < kEW; ++ee) {
        const int e = ee * kW + wave;
        load_raw<TIN, kE>(erow(rk, ink, e, DK) + el * kE, kraw[ee]);
    }
    float graw[VG ? kEW : 1][kE];  // VG: the lane's log-decays of this wave's entries
    // (issued before the state stream for up to 16 entries; after it for more, where holding
    // them across the stream would exceed the register budget)
    constexpr bool kLateG = VG && MAXW > 16;
    auto load_g = [&]() {
#pragma unroll
        for (int ee = 0; ee < kEW; ++ee) {
            const int e = ee * kW + wave;
            load_raw<float, kE>(erow(a.ring_g, a.in_g, e, DK) + el * kE, graw[ee]);
        }
    };
    if constexpr (VG && !kLateG) load_g();
    auto qidx = [&](int jj) { return kSplit ? jj * kW + wave : jj; };  // query of sweep slot jj
    TIN qraw[kQS][kE];
#pragma unroll
    for (int jj = 0; jj < kQS; ++jj)
        load_raw<TIN, kE>(inq + uniform64(tok(qidx(jj)) * DK) + el * kE, qraw[jj]);
    u32x4_t vraw[kVL];
#pragma unroll
    for (int i = 0; i < kVL; ++i) {
        const int idx = (lane + 64 * i) % (MAXW * kVC);
        const int e = idx / kVC, part = idx % kVC;
        vraw[i] = *reinterpret_cast<const u32x4_t*>(lrow(rv, inv, e, DV) + wave * kRows + part * kEPC);
    }

    // ---- the checkpoint rows of this wave ------------------------------------------------------
    // Half of the row is issued here and half after the sweeps, so that the sweeps do not hold
    // all 128 row registers and more waves fit on a SIMD. Loads are issued in the order the row
    // products use them.
    constexpr int kEarlyQ = RC == 0 ? kNQ / 2 : kNQ;
    float4 hv[kNQ];  // the fp32 rows (no read copy)
    RcRow<DV, DK, RC> rc;  // or the read copy's row, issued at the same point (news, para 4)
    const float4* tile = reinterpret_cast<const float4*>(a.ckpt) + th * (DV * DK / 4);
    if constexpr (RC == 0) {
#pragma unroll
        for (int q = 0; q < kEarlyQ; ++q) {
            hv[q] = ld_stream(tile + q * DV + row);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        rc.load(RcView{a.rc_codes, a.rc_scale, a.rc_tscale}, th, row);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage keys and v rows, append this call's tokens to the rings ------------------------
#pragma unroll
    for (int ee = 0; ee < kEW; ++ee)
#pragma unroll
        for (int i = 0; i < kE; ++i) s_k[ee * kW + wave][el * kE + i] = kraw[ee][i];
    if constexpr (VG && !kLateG) {
#pragma unroll
        for (int ee = 0; ee < kEW; ++ee)
#pragma unroll
            for (int i = 0; i < kE; ++i) s_al[ee * kW + wave][el * kE + i] = __expf(graw[ee][i]);
    } else if constexpr (VG) {  // up to eight entries at a time: few registers live beside the rows
        constexpr int kGB = kEW % 8 == 0 ? 8 : kEW % 6 == 0 ? 6 : kEW % 4 == 0 ? 4 : kEW % 2 == 0 ? 2 : 1;
#pragma unroll
        for (int e0 = 0; e0 < kEW; e0 += kGB) {
            float gb[kGB][kE];
#pragma unroll
            for (int u = 0; u < kGB; ++u) {
                const int e = (e0 + u) * kW + wave;
                load_raw<float, kE>(erow(a.ring_g, a.in_g, e, DK) + el * kE, gb[u]);
            }
#pragma unroll
            for (int u = 0; u < kGB; ++u) {
                const int e = (e0 + u) * kW + wave;
#pragma unroll
                for (int i = 0; i < kE; ++i) s_al[e][el * kE + i] = __expf(gb[u][i]);
                if (e >= count && e < kmax)  // this call's tokens: append g
                    gring.template bytes<kPol, kE * 4>((uint32_t)((ring_slot(start, e, cap) * DK + el * kE) * 4),
                                                       gb[u]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kVL; ++i) {
        const int idx = lane + 64 * i;
        if (idx < MAXW * kVC) s_v[wave][idx] = vraw[i];
    }
    {
        const PolicyStore vring(static_cast<TIN*>(a.ring_v) + uniform64(rh * DV), (uint32_t)(cap * DV * sizeof(TIN)));
#pragma unroll
        for (int i = 0; i < kVL; ++i) {
            const int idx = lane + 64 * i;
            const int e = idx / kVC, part = idx % kVC;
            if (e >= count && e < kmax && idx < MAXW * kVC)
                vring.template bytes<kPol, 16>(
                    (uint32_t)((ring_slot(start, e, cap) * DV + wave * kRows + part * kEPC) * sizeof(TIN)), &vraw[i]);
        }
        // each wave appends the keys (and decays) it staged
#pragma unroll
        for (int ee = 0; ee < kEW; ++ee) {
            const int e = ee * kW + wave;
            if (e >= count && e < kmax) {
                const uint32_t ro = (uint32_t)(ring_slot(start, e, cap) * DK + el * kE);
                kring.template bytes<kPol, kE * (int)sizeof(TIN)>(ro * (uint32_t)sizeof(TIN), kraw[ee]);
                if constexpr (VG && !kLateG) gring.template bytes<kPol, kE * 4>(ro * 4u, graw[ee]);
            }
        }
        if (wave == 0 && lane >= count && lane < kmax) {
            const unsigned rs = ring_slot(start, lane, cap);
            a.ring_beta[rh + rs] = be;
            if constexpr (!VG) a.ring_g[rh + rs] = ge;
        }
    }

    // ---- backward sweeps of this wave's queries over the entries they see -----------------------
    const int sw = kSplit ? 0 : wave;  // this wave's copy of r and c
    float r[kQS][kE];
#pragma unroll
    for (int jj = 0; jj < kQS; ++jj)
#pragma unroll
        for (int i = 0; i < kE; ++i) r[jj][i] = to_f32<TIN>(qraw[jj][i]);
    if constexpr (kW > 1) __syncthreads();  // every wave's entries are staged
    else wave_sync();
    const bool sweeps = qidx(0) < nq;  // uniform: a wave left without a query skips the sweep
    const float ae = VG ? 0.f : expf(ge);  // GDN: the decay of entry e = lane, one exp per lane
    // The sweep is a serial chain through r. Entry e - 1's key (and decays) are read from LDS
    // while entry e is processed, the lane sums stay in vector registers, and coefficient c_e
    // is kept by lane e (cv) and stored once after the sweep.
    float cv[kQS];
#pragma unroll
    for (int jj = 0; jj < kQS; ++jj) cv[jj] = 0.f;
    float kn[kE], an[VG ? kE : 1];
    auto fetch = [&](int e) {
#pragma unroll
        for (int i = 0; i < kE; ++i) kn[i] = to_f32<TIN>(s_k[e][el * kE + i]);
        if constexpr (VG) {
#pragma unroll
            for (int i = 0; i < kE; ++i) an[i] = s_al[e][el * kE + i];
        }
    };
    fetch(max(kmax - 1, 0));
    for (int e = sweeps ? kmax - 1 : -1; e >= 0; --e) {  // uniform trip count
        float kv[kE], al[kE];  // entry e's key and the decay of the lane's key elements
#pragma unroll
        for (int i = 0; i < kE; ++i) kv[i] = kn[i];
        if constexpr (VG) {
#pragma unroll
            for (int i = 0; i < kE; ++i) al[i] = an[i];
        } else {
            const float as = readlane(ae, e);
#pragma unroll
            for (int i = 0; i < kE; ++i) al[i] = as;
        }
        fetch(max(e - 1, 0));
        const float bt = readlane(be, e);
        const bool mine = lane == e;
        if constexpr (kQS == 1) {
            const int j = qidx(0);
            if (j < nq && e <= count + j) {  // (entries after query j's own token: uniform skip)
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < kE; ++i) d += kv[i] * r[0][i];
                const float c = bt * group_sum<64>(d);
#pragma unroll
                for (int i = 0; i < kE; ++i) r[0][i] = al[i] * (r[0][i] - c * kv[i]);
                cv[0] = mine ? c : cv[0];
            }
        } else {
            // several queries: their reductions are independent chains, so the loop body has no
            // branch and they interleave; a query that does not see entry e (e after its own
            // token, or a padding query) keeps its r, and its coefficient slot is never read
            float d[kQS];
#pragma unroll
            for (int jj = 0; jj < kQS; ++jj) {
                d[jj] = 0.f;
#pragma unroll
                for (int i = 0; i < kE; ++i) d[jj] += kv[i] * r[jj][i];
            }
#pragma unroll
            for (int jj = 0; jj < kQS; ++jj) d[jj] = bt * group_sum<64>(d[jj]);
#pragma unroll
            for (int jj = 0; jj < kQS; ++jj) {
                const int j = qidx(jj);
                const bool sees = j < nq && e <= count + j;
#pragma unroll
                for (int i = 0; i < kE; ++i)
                    r[jj][i] = sees ? al[i] * (r[jj][i] - d[jj] * kv[i]) : r[jj][i];
                cv[jj] = mine && sees ? d[jj] : cv[jj];  // 0 for an entry the query does not see
            }
        }
    }
    // coefficients c_e of the entries each query sees (0 for the others, so a later draft's
    // inputs, finite or not, never reach an earlier draft's output)
#pragma unroll
    for (int jj = 0; jj < kQS; ++jj) {
        const int j = qidx(jj);
        if (j < MAXQ && lane < MAXW) s_c[sw][lane][j] = cv[jj];
    }
    if constexpr (RC == 0 && kEarlyQ < kNQ) {
#pragma unroll
        for (int q = kEarlyQ; q < kNQ; ++q) {
            hv[q] = ld_stream(tile + q * DV + row);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int jj = 0; jj < kQS; ++jj) {
        const int j = qidx(jj);
        if (j >= MAXQ) break;
#pragma unroll
        for (int i = 0; i < kE; ++i) s_r[sw][j][el * kE + i] = r[jj][i];
    }
    if constexpr (kSplit) __syncthreads();  // the other waves' r and c
    else wave_sync();

    // ---- value terms and the checkpoint row products --------------------------------------------
    const TIN* sv = reinterpret_cast<const TIN*>(&s_v[wave][0]);
    float acc[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) acc[j] = 0.f;
    // value terms four entries at a time, so that the LDS reads of a group go out together. Every
    // slot e < MAXW of s_v holds a staged row (entries past the call's last token repeat it) and
    // s_c holds 0 for the entries a query does not see; the select keeps a non-finite v of such
    // an entry out of the sum.
    for (int e0 = 0; e0 < kmax; e0 += 4) {  // uniform; MAXW is a multiple of 4
        float ve[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ve[u] = to_f32<TIN>(sv[(e0 + u) * kRows + lane]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u;
#pragma unroll
            for (int j = 0; j < MAXQ; ++j) {
                acc[j] = fmaf(s_c[sw][e][j], e <= count + j ? ve[u] : 0.f, acc[j]);
            }
        }
    }
    float dot[MAXQ];
    if constexpr (RC != 0) {  // the decoded copy's rows against every r_j (news, para 4)
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) dot[j] = 0.f;
        rc.template dots<kRS, MAXQ>(nq, &s_r[sw][0][0], dot);
    } else if constexpr (MAXQ >= 4) {
        // four queries per 4x4x1 MFMA (lane = row; query 4g + lane%4 supplies its r column),
        // two accumulator chains per group of four
        constexpr int kG = MAXQ / 4;
        f32x4 dq[kG][2];
#pragma unroll
        for (int g = 0; g < kG; ++g) dq[g][0] = dq[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const float4 r4 = *reinterpret_cast<const float4*>(&s_r[sw][4 * g + (lane & 3)][4 * q]);
                f32x4& d = dq[g][q & 1];
                d = mfma4x4(r4.x, hv[q].x, d);
                d = mfma4x4(r4.y, hv[q].y, d);
                d = mfma4x4(r4.z, hv[q].z, d);
                d = mfma4x4(r4.w, hv[q].w, d);
            }
        }
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) dot[j] = dq[j / 4][0][j % 4] + dq[j / 4][1][j % 4];
    } else {
#pragma unroll
        for (int j = 0; j < MAXQ; ++j) {
            dot[j] = 0.f;
#pragma unroll
            for (int q = 0; q < kNQ; ++q) {
                const float4 r4 = *reinterpret_cast<const float4*>(&s_r[sw][j][4 * q]);
                dot[j] += hv[q].x * r4.x + hv[q].y * r4.y + hv[q].z * r4.z + hv[q].w * r4.w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
        if (j >= nq) break;
        const PolicyStore orow(a.o + uniform64(tok(j) * DV), DV * 4);
        const float ov = a.scale * (dot[j] + acc[j]);
        orow.template bytes<kStoreWT, 4>((uint32_t)(row * 4), &ov);
    }
    if constexpr (COMMIT) {
        if constexpr (kW > 1) __builtin_amdgcn_s_barrier();  // every wave has read the pointers
        if (wave == 0 && lane == 0) a.ptr[kPtrInts * head + 1] = count + nq;
    }
}

// ---------------------------------------------------------------------------------------------
// Conventional step (comparison point; the full state rewritten every token):
//   S <- alpha S + beta (v - alpha S k) k^T (in place),  o = scale S q.
// VG (Kimi Delta Attention): alpha is a dk-vector and scales the state's columns.
// ---------------------------------------------------------------------------------------------
template <int DV, int DK, typename TIN, bool VG = false>
__global__ __launch_bounds__(64 * (DV >= 64 ? DV / 64 : 1))
__attribute__((amdgpu_waves_per_eu(2))) void gdn_conv_kernel(GdnConvArgs a) {
    constexpr int kW = DV >= 64 ? DV / 64 : 1;
    constexpr int kRows = DV >= 64 ? 64 : DV;
    constexpr int kNQ = DK / 4;
    constexpr int kCE = DK >= 64 ? DK / 64 : 1;
    __shared__ __attribute__((aligned(16))) float s_kq[kW][VG ? 3 : 2][DK];  // k, q (, alpha)
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x, b = blockIdx.y;
    const long head = (long)b * a.heads + h;
    const int row = wave * kRows + (lane % kRows);
    const TIN* ink = static_cast<const TIN*>(a.in_k) + head * DK;
    const TIN* inq = static_cast<const TIN*>(a.in_q) + head * DK;
    TIN kraw[kCE], qraw[kCE];
    float graw[kCE];
#pragma unroll
    for (int i = 0; i < kCE; ++i) {
        const int n = (lane + 64 * i) % DK;
        kraw[i] = ink[n];
        qraw[i] = inq[n];
        if constexpr (VG) graw[i] = a.in_g[head * DK + n];
    }
    const float v = to_f32<TIN>(static_cast<const TIN*>(a.in_v)[head * DV + row]);
    const float beta = a.in_beta[head];
    const float alpha = VG ? 1.f : expf(a.in_g[head]);
    float4 hv[kNQ];
    // float4 q * DV + row of the head's tile
    const TileIO tio{reinterpret_cast<char*>(a.S) + (long)head * (DV * DK * 4), (uint32_t)(row * 16)};
    // issued in the order the row dot uses them, so that it runs while the row arrives
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
        hv[q] = tio.load((uint32_t)(q * DV * 16));
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kCE; ++i) {
        const int n = (lane + 64 * i) % DK;
        s_kq[wave][0][n] = to_f32<TIN>(kraw[i]);
        s_kq[wave][1][n] = to_f32<TIN>(qraw[i]);
        if constexpr (VG) s_kq[wave][2][n] = expf(graw[i]);
    }
    wave_sync();
    float sk = 0.f;  // (S k) for a scalar decay; (S diag(alpha) k) with VG
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
        float4 k4 = *reinterpret_cast<const float4*>(&s_kq[wave][0][4 * q]);
        if constexpr (VG) {
            const float4 a4 = *reinterpret_cast<const float4*>(&s_kq[wave][2][4 * q]);
            k4 = make_float4(k4.x * a4.x, k4.y * a4.y, k4.z * a4.z, k4.w * a4.w);
        }
        sk += hv[q].x * k4.x + hv[q].y * k4.y + hv[q].z * k4.z + hv[q].w * k4.w;
    }
    const float u = beta * (v - alpha * sk);
    asm volatile("" ::: "memory");  // re-read k below rather than keeping 32 quads of it live
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
        const float4 k4 = *reinterpret_cast<const float4*>(&s_kq[wave][0][4 * q]);
        const float4 q4 = *reinterpret_cast<const float4*>(&s_kq[wave][1][4 * q]);
        float4 a4 = make_float4(alpha, alpha, alpha, alpha);
        if constexpr (VG) a4 = *reinterpret_cast<const float4*>(&s_kq[wave][2][4 * q]);
        hv[q].x = a4.x * hv[q].x + u * k4.x;
        hv[q].y = a4.y * hv[q].y + u * k4.y;
        hv[q].z = a4.z * hv[q].z + u * k4.z;
        hv[q].w = a4.w * hv[q].w + u * k4.w;
        o += hv[q].x * q4.x + hv[q].y * q4.y + hv[q].z * q4.z + hv[q].w * q4.w;
        tio.template store<kTileStorePol>((uint32_t)(q * DV * 16), hv[q]);
    }
    if (lane < kRows) a.o[head * DV + row] = a.scale * o;
}

// ---------------------------------------------------------------------------------------------
// Snapshot-based speculative step (the comparison point for the speculative verify; news para 3:
// conventional speculation keeps per-token state snapshots; explainer, "Usage examples": snapshot
// and restore): the recurrence of gdn_conv_kernel over ntok <= MAXQ draft tokens from the
// read-only state a.S, writing the state after each draft j to its own snapshot tile
// a.snap + (j * batch * H + head) * DV * DK and o [batch][ntok][H][DV].
// ---------------------------------------------------------------------------------------------
template <int DV, int DK, typename TIN, int MAXQ, bool VG = false>
__global__ __launch_bounds__(DV)
__attribute__((amdgpu_waves_per_eu(2))) void gdn_snap_kernel(GdnConvArgs a) {
    static_assert(DV % 64 == 0 && DK % 64 == 0, "snapshot tile shape");
    constexpr int kW = DV / 64;
    constexpr int kNQ = DK / 4;
    constexpr int kCE = DK / 64;
    __shared__ __attribute__((aligned(16))) float s_kq[kW][MAXQ][VG ? 3 : 2][DK];  // k, q (, alpha)
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x, b = blockIdx.y;
    const int H = a.heads, nq = a.ntok;
    const long head = (long)b * H + h;
    const int row = wave * 64 + lane;
    const TIN* ink = static_cast<const TIN*>(a.in_k);
    const TIN* inq = static_cast<const TIN*>(a.in_q);
    const TIN* inv = static_cast<const TIN*>(a.in_v);
    // every draft's inputs, issued before the state stream (rows past ntok repeat the last one)
    TIN kraw[MAXQ][kCE], qraw[MAXQ][kCE], vraw[MAXQ];
    float graw[VG ? MAXQ : 1][kCE], betaj[MAXQ], gj[MAXQ];
#pragma unroll
    for (int j = 0; j < MAXQ; ++j) {
        const long tok = ((long)b * nq + min(j, nq - 1)) * H + h;
#pragma unroll
        for (int i = 0; i < kCE; ++i) {
            const int n = lane + 64 * i;
            kraw[j][i] = ink[tok * DK + n];
            qraw[j][i] = inq[tok * DK + n];
            if constexpr (VG) graw[j][i] = a.in_g[tok * DK + n];
        }
        vraw[j] = inv[tok * DV + row];
        betaj[j] = a.in_beta[tok];
        gj[j] = VG ? 0.f : a.in_g[tok];
    }
    float4 hv[kNQ];
    const uint32_t lane_off = (uint32_t)(row * 16);
    const TileIO tin{reinterpret_cast<char*>(a.S) + head * (DV * DK * 4), lane_off};
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
        hv[q] = tin.load((uint32_t)(q * DV * 16));
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < MAXQ; ++j)
#pragma unroll
        for (int i = 0; i < kCE; ++i) {
            const int n = lane + 64 * i;
            s_kq[wave][j][0][n] = to_f32<TIN>(kraw[j][i]);
            s_kq[wave][j][1][n] = to_f32<TIN>(qraw[j][i]);
            if constexpr (VG) s_kq[wave][j][2][n] = expf(graw[j][i]);
        }
    wave_sync();
    const long nheads = (long)a.batch * H;
#pragma unroll
    for (int t = 0; t < MAXQ; ++t) {
        if (t >= nq) break;
        const float alpha = VG ? 1.f : expf(gj[t]);
        float sk = 0.f;  // (S k) for a scalar decay; (S diag(alpha) k) with VG
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
            float4 k4 = *reinterpret_cast<const float4*>(&s_kq[wave][t][0][4 * q]);
            if constexpr (VG) {
                const float4 a4 = *reinterpret_cast<const float4*>(&s_kq[wave][t][2][4 * q]);
                k4 = make_float4(k4.x * a4.x, k4.y * a4.y, k4.z * a4.z, k4.w * a4.w);
            }
            sk += hv[q].x * k4.x + hv[q].y * k4.y + hv[q].z * k4.z + hv[q].w * k4.w;
        }
        const float u = betaj[t] * (to_f32<TIN>(vraw[t]) - alpha * sk);
        asm volatile("" ::: "memory");  // re-read k below rather than keeping 32 quads of it live
        const TileIO tout{reinterpret_cast<char*>(a.snap) + ((long)t * nheads + head) * (DV * DK * 4),
                          lane_off};
        float o = 0.f;
#pragma unroll
        for (int q = 0; q < kNQ; ++q) {
            const float4 k4 = *reinterpret_cast<const float4*>(&s_kq[wave][t][0][4 * q]);
            const float4 q4 = *reinterpret_cast<const float4*>(&s_kq[wave][t][1][4 * q]);
            float4 a4 = make_float4(alpha, alpha, alpha, alpha);
            if constexpr (VG) a4 = *reinterpret_cast<const float4*>(&s_kq[wave][t][2][4 * q]);
            hv[q].x = a4.x * hv[q].x + u * k4.x;
            hv[q].y = a4.y * hv[q].y + u * k4.y;
            hv[q].z = a4.z * hv[q].z + u * k4.z;
            hv[q].w = a4.w * hv[q].w + u * k4.w;
            o += hv[q].x * q4.x + hv[q].y * q4.y + hv[q].z * q4.z + hv[q].w * q4.w;
            tout.store((uint32_t)(q * DV * 16), hv[q]);
        }
        a.o[(((long)b * nq + t) * H + h) * DV + row] = a.scale * o;
    }
}

// ---------------------------------------------------------------------------------------------
// Flush in UT/WY form (news para 3: fold the buffer into the checkpoint in one pass). For a chunk
// of (up to) 16 entries, with G_t the running sum of g (log of the cumulative decay gamma_t):
//   Lm[t][i] = beta_t exp(G_t - G_i) (k_t . k_i)   (i < t; decay as a partial sum of g)
//   W_t = beta_t gamma_t k_t - sum_{i<t} Lm[t][i] W_i       (forward substitution, dk-vectors)
//   U_t = beta_t v_t     - sum_{i<t} Lm[t][i] U_i       (forward substitution, dv-vectors)
//   Delta_t = U_t - S W_t,   S <- gamma_L S + sum_t (gamma_L / gamma_t) Delta_t k_t^T
// The Gram matrix K K^T and the two dv x dk x 16 contractions run on fp32 MFMA
// (v_mfma_f32_16x16x4f32): A[m][k] from lane l = (m = l%16, k = l/16), B[k][c] from lane l =
// (k = l/16, c = l%16), D[m][c] in lane l at register r = (m = 4(l/16) + r, c = l%16).
// Entries past the fold count are zero rows (beta = g = 0, k = v = 0), which leave S unchanged.
// FUSED: the L-th token of a lock-step decode (count == L-1 for every sequence) is folded with
// the L-1 buffered entries straight from the caller's inputs, and its output is taken from the
// new state, o = scale S_L q_L (the recurrence's own form); the ring is left empty.
// Requires DV % 64 == 0 (one wave per 64 rows) and DK % 64 == 0.
// VG (Kimi Delta Attention): the decay is a dk-vector per entry. With G_t[n] the within-chunk
// cumulative log-decay of key channel n, the same UT/WY steps hold with
//   Lm[t][i] = beta_t sum_n k_t[n] k_i[n] exp(G_t[n] - G_i[n])   (a gated Gram matrix, on MFMA
//     as four products over a binary split of the chunk, every exponent <= 0: see below),
//   W_t = beta_t (exp(G_t) * k_t) - sum_{i<t} Lm[t][i] W_i,
//   S <- S diag(exp(G_L)) + sum_t Delta_t (k_t * exp(G_L - G_t))^T.
// ---------------------------------------------------------------------------------------------
template <int DV, int DK, typename TIN, int RC, bool FUSED, bool VG = false>
__global__ __launch_bounds__(DV)
__attribute__((amdgpu_waves_per_eu(2))) void gdn_flush_kernel(GdnArgs a, int mode_all,
                                                              int rewrite_only) {
    static_assert(DV % 64 == 0 && DK % 64 == 0, "flush tile shape");
    constexpr int kW = DV / 64;
    constexpr int kPB = 4;            // 16-row blocks per wave
    constexpr int kNB = DK / 16;      // 16-column blocks
    constexpr int kKP = DK + 4;       // padded LDS row strides (bank spread)
    constexpr int kVP = 64 + 4;
    constexpr int kEPC = 16 / (int)sizeof(TIN);
    constexpr int kKC = DK / kEPC, kVC = 64 / kEPC;   // 16-byte chunks per k row / per v slice
    // the waves of a head split the staging of the chunk's keys (and VG log-decays)
    constexpr int kKL = (16 * kKC / kW + 63) / 64, kVL = (16 * kVC + 63) / 64;
    constexpr int kGC = DK / 4, kGL = (16 * kGC / kW + 63) / 64;  // VG: 16-byte pieces of g rows
    constexpr int kWE = DK / 64;      // columns n = lane + 64 j, j < kWE, of the substitution
    // Shared by the head's waves (the keys, W and Lm do not depend on the state rows):
    __shared__ __attribute__((aligned(16))) float s_k[16][kKP];   // K chunk (fp32); VG: then K~
    __shared__ __attribute__((aligned(16))) float s_w[16][kKP];   // VG: G first; then -W
    __shared__ __attribute__((aligned(16))) float s_l[16][17];    // Lm
    __shared__ __attribute__((aligned(16))) float s_q[FUSED ? DK : 4];   // FUSED: the token's q
    __shared__ __attribute__((aligned(16))) float s_gl[VG ? DK : 4];     // VG: exp(G_L) per column
    // Per wave: its v slice, then U ([t][p]); after step A the same floats hold Delta' as [p][t]
    // (64 x 17 == 16 x 68), the transpose buffer
    __shared__ __attribute__((aligned(16))) float s_v[kW][16][kVP];
    __shared__ float s_amax[kW];  // fp4 read copy: the waves' largest magnitudes
    static_assert(16 * kVP == 64 * 17, "transpose buffer aliases the v slice");

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x, b = blockIdx.y;
    const int head = b * a.heads + h;
    const int cap = a.cap;
    const HeadPtr pt = head_ptr(a.ptr, a.hstart, a.hcount, head, b);
    const int start = pt.start, count = pt.count, slot = pt.slot;
    // copy-on-write of a shared checkpoint: a sequence that must move folds whatever it holds
    const FoldTarget ft = fold_target(a.refcnt, a.share, a.batch, b, slot);
    // FUSED: the buffered entries and this token; otherwise the oldest L (or all) entries
    const int nfold = FUSED ? count + 1
                            : (rewrite_only ? 0 : (mode_all ? count : (count >= a.window ? a.window : (ft.move ? count : 0))));
    const int nring = FUSED ? count : nfold;  // entries that come from the ring
    // uniform over the workgroup: no barrier is skipped
    if (nfold == 0 && !rewrite_only && !ft.move) return;
    const long th = a.share ? (long)slot * a.heads + h : head;   // tile read
    const long tw = a.share ? (long)ft.wr * a.heads + h : head;  // tile written
    const long rh = uniform64((long)head * cap);                  // this head's first ring row
    const TIN* rk = static_cast<const TIN*>(a.ring_k);
    const TIN* rv = static_cast<const TIN*>(a.ring_v);
    const int li = lane & 15, lg = lane >> 4;
    const int p_base = wave * 64;
    float (*s_d)[17] = reinterpret_cast<float (*)[17]>(&s_v[wave][0][0]);

    // entry e (already clamped to a folded entry): ring slot, or the caller's token (FUSED)
    auto krow = [&](int e) -> const TIN* {
        if (FUSED && e >= nring) return static_cast<const TIN*>(a.in_k) + (long)head * DK;
        return rk + (rh + ring_slot(start, e, cap)) * DK;
    };
    auto vrow = [&](int e) -> const TIN* {
        if (FUSED && e >= nring) return static_cast<const TIN*>(a.in_v) + (long)head * DV;
        return rv + (rh + ring_slot(start, e, cap)) * DV;
    };
    auto grow = [&](int e) -> const float* {  // VG: the entry's dk log-decays
        if (FUSED && e >= nring) return a.in_g + (long)head * DK;
        return a.ring_g + (rh + ring_slot(start, e, cap)) * DK;
    };
    // chunk loader (branch-free: entries past nfold read the last folded entry, zeroed later);
    // wave w loads key pieces w * 16 kKC / kW .. of the chunk
    u32x4_t kraw[kKL], vraw[kVL];
    float be = 0.f, ge = 0.f;
    auto fetch = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kKL; ++i) {
            const int idx = (wave * (16 * kKC / kW) + lane + 64 * i) % (16 * kKC);
            const int e = min(c0 + idx / kKC, max(nfold - 1, 0)), part = idx % kKC;
            kraw[i] = *reinterpret_cast<const u32x4_t*>(krow(e) + part * kEPC);
        }
#pragma unroll
        for (int i = 0; i < kVL; ++i) {
            const int idx = (lane + 64 * i) % (16 * kVC);
            const int e = min(c0 + idx / kVC, max(nfold - 1, 0)), part = idx % kVC;
            vraw[i] = *reinterpret_cast<const u32x4_t*>(vrow(e) + p_base + part * kEPC);
        }
        const int e = min(c0 + li, max(nfold - 1, 0));
        const long s = rh + ring_slot(start, min(e, cap - 1), cap);
        const bool tok = FUSED && e >= nring;
        be = tok ? a.in_beta[head] : a.ring_beta[s];
        be = (c0 + li < nfold) ? be : 0.f;  // lanes 16..63 mirror lanes 0..15
        if constexpr (!VG) {
            ge = tok ? a.in_g[head] : a.ring_g[s];
            ge = (c0 + li < nfold) ? ge : 0.f;
        }
    };
    fetch(0);  // entries clamped to >= 0: in bounds also when nothing is folded (rewrite only)
    constexpr int kQE = DK / 64;  // FUSED: q elements per lane
    TIN qraw[FUSED ? kQE : 1];
    if constexpr (FUSED) {
        const TIN* inq = static_cast<const TIN*>(a.in_q) + (long)head * DK;
#pragma unroll
        for (int i = 0; i < kQE; ++i) qraw[i] = inq[lane + 64 * i];
    }

    // the tile in accumulator order: block (pb, nb) of lane l = row p_base + 16pb + l%16,
    // columns 16nb + 4(l/16) .. +3
    f32x4 S[kPB][kNB];
    // float4 (4 nb + lg) * DV + p_base + 16 pb + li of the head's tile
    const TileIO tio{reinterpret_cast<char*>(a.ckpt) + th * (DV * DK * 4),
                     (uint32_t)((lg * DV + p_base + li) * 16)};
    const TileIO tiow{reinterpret_cast<char*>(a.ckpt) + tw * (DV * DK * 4), tio.lane};
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const float4 t = tio.load((uint32_t)((4 * nb * DV + 16 * pb) * 16));
            S[pb][nb] = f32x4{t.x, t.y, t.z, t.w};
        }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    float opart[kPB] = {};  // FUSED: partial dot products of the new state's rows with q
    if constexpr (FUSED) {
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < kQE; ++i) s_q[lane + 64 * i] = to_f32<TIN>(qraw[i]);
        }
    }
    for (int c0 = 0; c0 < nfold; c0 += 16) {
        if (c0 > 0) fetch(c0);
        const int nc = min(16, nfold - c0);
        // ---- stage this wave's share of K, its own V slice (entries >= nc as zeros) ----------
#pragma unroll
        for (int i = 0; i < kKL; ++i) {
            const int idx = wave * (16 * kKC / kW) + lane + 64 * i;
            if (lane + 64 * i < 16 * kKC / kW) {
                const int e = idx / kKC, part = idx % kKC;
                float f[kEPC];
                Unit<TIN>::unpack(make_uint4(kraw[i].x, kraw[i].y, kraw[i].z, kraw[i].w), f);
#pragma unroll
                for (int j = 0; j < kEPC; ++j) s_k[e][part * kEPC + j] = e < nc ? f[j] : 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < kVL; ++i) {
            const int idx = lane + 64 * i;
            if (idx < 16 * kVC) {
                const int e = idx / kVC, part = idx % kVC;
                float f[kEPC];
                Unit<TIN>::unpack(make_uint4(vraw[i].x, vraw[i].y, vraw[i].z, vraw[i].w), f);
#pragma unroll
                for (int j = 0; j < kEPC; ++j) s_v[wave][e][part * kEPC + j] = e < nc ? f[j] : 0.f;
            }
        }
        float glog[VG ? kWE : 1];  // VG: G_L of the lane's own columns
        if constexpr (VG) {
            // g rows -> s_w (this wave's share, loaded here after the state stream, four 16-byte
            // pieces at a time: held across the stream they would spill)
#pragma unroll
            for (int i0 = 0; i0 < kGL; i0 += 4) {
                u32x4_t graw[4];
#pragma unroll
                for (int i = i0; i < i0 + 4 && i < kGL; ++i) {
                    const int idx = (wave * (16 * kGC / kW) + lane + 64 * i) % (16 * kGC);
                    const int e = min(c0 + idx / kGC, max(nfold - 1, 0)), part = idx % kGC;
                    graw[i - i0] = *reinterpret_cast<const u32x4_t*>(grow(e) + part * 4);
                }
#pragma unroll
                for (int i = i0; i < i0 + 4 && i < kGL; ++i) {
                    if (lane + 64 * i < 16 * kGC / kW) {
                        const int idx = wave * (16 * kGC / kW) + lane + 64 * i;
                        const int e = idx / kGC, part = idx % kGC;
                        const u32x4_t u = graw[i - i0];
                        const float f[4] = {__uint_as_float(u.x), __uint_as_float(u.y),
                                            __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
                        for (int j = 0; j < 4; ++j) s_w[e][part * 4 + j] = e < nc ? f[j] : 0.f;
                    }
                }
            }
            __syncthreads();
            // the within-chunk cumulative G of the columns this lane owns, in place
#pragma unroll
            for (int j = 0; j < kWE; ++j) {
                if (j % kW != wave) continue;  // the waves split the columns
                const int n = lane + 64 * j;
                float Gc = 0.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    Gc += s_w[t][n];
                    s_w[t][n] = Gc;
                }
                glog[j] = Gc;
                s_gl[n] = __expf(Gc);
            }
        }
        __syncthreads();

        // ---- Gram matrix and Lm (once per head, by wave 0) ------------------------------------
        // G_t = sum_{m <= t} g_m within the chunk (inclusive scan over each 16-lane row; the four
        // rows hold the same entries, so every lane l has G at entry l%16)
        float G = ge;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const float t = __shfl_up(G, o, 16);
            G += li >= o ? t : 0.f;
        }
        // The flush's decay factors use the hardware exponential (__expf: the exponent scaled by
        // log2 e, then v_exp_f32): relative error about 1e-7 |x| for exp(x), far inside the fp32
        // metric, at a fraction of the instructions of the correctly rounded expf (KDA takes
        // about a hundred per lane per chunk). With log-decays g <= 0 no exponent here is positive.
        if constexpr (VG) {
            // Gated Gram matrix sum_n k_t[n] k_i[n] exp(G_t[n] - G_i[n]) for i < t, over a binary
            // split of the chunk: the pair (t, i) belongs to level b, the highest bit in which t and
            // i differ, and there both lie in one aligned block of 2^(b+1) entries with i in its
            // lower half and t in its upper half. With c the last entry of the lower half,
            // exp(G_t - G_i) = exp(G_t - G_c) exp(G_c - G_i) and both factors are <= 1 (G only
            // falls), so neither overflows however fast a channel decays; a factor that underflows
            // bounds the true product below it. Each level is one Gram product on MFMA: lane l
            // supplies row l%16 scaled by its factor as the left operand if it lies in the upper
            // half of its block, as the right one if in the lower half (the other operand 0).
            // The head's waves split the four levels (level b on wave b % kW).
            constexpr int kLv = 4 / kW;  // levels of this wave
#pragma unroll
            for (int v = 0; v < kLv; ++v) {
                __builtin_amdgcn_sched_barrier(0);  // one level's operands live at a time
                const int lev = v * kW + wave;
                const int half = 1 << lev;
                const int cut = (li & ~(2 * half - 1)) | (half - 1);
                const bool upper = (li & half) != 0;
                f32x4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int n0 = 0; n0 < DK; n0 += 4) {
                    const float kk = s_k[li][n0 + lg];
                    const float Gr = s_w[li][n0 + lg], Gc = s_w[cut][n0 + lg];
                    const float x = kk * __expf(upper ? Gr - Gc : Gc - Gr);
                    gram = mfma4(upper ? x : 0.f, upper ? 0.f : x, gram);
                }
                // Lm[t][i] = beta_t Gram[t][i] for t = 4lg + r, i = li, for the pairs of this level
                // (t and i differ first in bit lev); wave 0 also writes the zeros of i >= t
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * lg + r, i = li;
                    const float bt = __shfl(be, t, 64);
                    if (i < t && 31 - __clz(t ^ i) == lev) s_l[t][i] = bt * gram[r];
                    if (v == 0 && wave == 0 && i >= t) s_l[t][i] = 0.f;
                }
            }
        } else if (wave == 0) {
            // K K^T on MFMA: lane l supplies K[l%16][n0 + l/16] as both operands
            f32x4 gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int n0 = 0; n0 < DK; n0 += 4) {
                const float kk = s_k[li][n0 + lg];
                gram = mfma4(kk, kk, gram);
            }
            // Lm[t][i] for t = 4lg + r, i = li (t varies across lanes: per-lane shuffles);
            // the decay from entry i to t is exp(G_t - G_i) <= 1 (only taken where i < t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * lg + r, i = li;
                const float bt = __shfl(be, t, 64);
                const float Gt = __shfl(G, t, 64);
                s_l[t][i] = (i < t) ? bt * __expf(Gt - G) * gram[r] : 0.f;
            }
        }
        __syncthreads();

        // ---- forward substitution, in place in LDS ---------------------------------------------
        // W: lane owns the columns n = lane + 64 j (the waves split them); U: lane owns row
        // p_base + lane. Every value a lane reads back it wrote itself. W is kept negated
        // (s_w[t] = -W_t) for the MFMA below; U overwrites V in s_v ([t][p]).
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const float bt = readlane(be, t);
            const float bg = bt * (VG ? 1.f : __expf(readlane(G, t)));
            float lrow[16];
#pragma unroll
            for (int i = 0; i < t; ++i) lrow[i] = s_l[t][i];
#pragma unroll
            for (int j = 0; j < kWE; ++j) {
                if (j % kW != wave) continue;
                const int n = lane + 64 * j;
                const float kt = s_k[t][n];
                float sw;
                if constexpr (VG) {  // row t of s_w still holds G_t here
                    const float Gt = s_w[t][n];
                    sw = -bg * __expf(Gt) * kt;
                    s_k[t][n] = kt * __expf(glog[j] - Gt);  // K~ for the update below
                } else {
                    sw = -bg * kt;
                }
#pragma unroll
                for (int i = 0; i < t; ++i) sw -= lrow[i] * s_w[i][n];
                s_w[t][n] = sw;
            }
            float su = bt * s_v[wave][t][lane];
#pragma unroll
            for (int i = 0; i < t; ++i) su -= lrow[i] * s_v[wave][i][lane];
            s_v[wave][t][lane] = su;
            asm volatile("" ::: "memory");  // one row of Lm live at a time
        }
        const float gL = readlane(G, 15);  // log gamma_L (zero-padded entries add nothing)
        __syncthreads();  // W and K~ complete for every column

        asm volatile("" ::: "memory");
        // ---- Delta^T[p][t] = U^T[p][t] - sum_n S[p][n] W[t][n]   (D layout: p = 4lg + r, t = li)
        const float dscale = VG ? 1.f : __expf(gL - G);  // gamma_L / gamma_t for t = li (VG: in K~)
        f32x4 delta[kPB];
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) delta[pb][r] = s_v[wave][li][16 * pb + 4 * lg + r];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            // B operand: -W[t = li][16nb + 4lg + r]
            const f32x4 wop = *reinterpret_cast<const f32x4*>(&s_w[li][16 * nb + 4 * lg]);
#pragma unroll
            for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) delta[pb] = mfma4(S[pb][nb][r], wop[r], delta[pb]);
        }
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) delta[pb] *= dscale;  // Delta' = (gamma_L/gamma_t) Delta
        wave_sync();  // every lane of the wave has read U: its floats become the transpose buffer
        // transpose Delta' through LDS ([p][t])
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_d[16 * pb + 4 * lg + r][li] = delta[pb][r];
        wave_sync();

        asm volatile("" ::: "memory");
        // ---- S <- gamma_L S + sum_t K^T[n][t] Delta'^T[t][p]   (D rows = n, columns = p) -----
        const float gammaL = __expf(gL);
        if constexpr (VG) {  // column n = 16 nb + 4 lg + r scaled by exp(G_L[n]), one block at a time
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                const f32x4 gc = *reinterpret_cast<const f32x4*>(&s_gl[16 * nb + 4 * lg]);
#pragma unroll
                for (int pb = 0; pb < kPB; ++pb) S[pb][nb] *= gc;
            }
        }
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) {
            opart[pb] = 0.f;
            float dop[4];  // B operand: Delta'[p = 16pb + li][t = 4tg + lg]
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) dop[tg] = s_d[16 * pb + li][4 * tg + lg];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                f32x4 acc = VG ? S[pb][nb] : S[pb][nb] * gammaL;  // (VG: scaled above)
#pragma unroll
                for (int tg = 0; tg < 4; ++tg)
                    acc = mfma4(s_k[4 * tg + lg][16 * nb + li], dop[tg], acc);
                S[pb][nb] = acc;
                if constexpr (FUSED) {  // the token's output row partials, o = scale S q
                    // (every chunk recomputes them; the last chunk's are the new state's)
                    const float4 q4 = *reinterpret_cast<const float4*>(&s_q[16 * nb + 4 * lg]);
                    opart[pb] += acc[0] * q4.x + acc[1] * q4.y + acc[2] * q4.z + acc[3] * q4.w;
                }
            }
        }
        __syncthreads();  // the next chunk overwrites the shared K, W and Lm
    }

#pragma unroll
    for (int pb = 0; pb < kPB; ++pb)  // (a rewrite-only pass stores the tile unchanged)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
            tiow.template store<kTileStorePol>((uint32_t)((4 * nb * DV + 16 * pb) * 16),
                       make_float4(S[pb][nb][0], S[pb][nb][1], S[pb][nb][2], S[pb][nb][3]));
    if constexpr (FUSED) {
        // row p_base + 16 pb + li is spread over lanes li + 16 lg: sum the four partials through
        // the wave's (now free) transpose buffer, then lane p writes row p_base + p
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) s_d[16 * pb + li][lg] = opart[pb];
        wave_sync();
        const float* r = s_d[lane];
        a.o[(long)head * DV + p_base + lane] = a.scale * ((r[0] + r[1]) + (r[2] + r[3]));
    }
    // (the copy's encoding stays below this point: scheduled up with the fused output it took
    // more than 256 registers)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RC != 0) {  // rewrite the read copy from the new fp32 tile (news, para 4)
        float amax_t = 0.f;
        if constexpr (RC == 2) {
            const float wmax = xor_reduce_max<1, 32>(rc_local_amax<DK>(S));
            if constexpr (kW > 1) {
                if (lane == 0) s_amax[wave] = wmax;
                __syncthreads();
#pragma unroll
                for (int w = 0; w < kW; ++w) amax_t = fmaxf(amax_t, s_amax[w]);
            } else {
                amax_t = wmax;
            }
        }
        rc_write_blocks<DV, DK, RC>(RcView{a.rc_codes, a.rc_scale, a.rc_tscale}, tw, p_base, li, lg,
                                    S, amax_t, wave == 0 && lane == 0, &s_v[wave][0][0]);
    }
    if constexpr (kW > 1) __builtin_amdgcn_s_barrier();  // every wave has read the pointers
    if ((nfold > 0 || ft.move) && wave == 0 && lane == 0)
        *reinterpret_cast<int4*>(a.ptr + kPtrInts * head) =
            make_int4(ring_slot(start, nfold, cap), (FUSED ? count + 1 : count) - nfold, ft.wr, 0);
}

// ---------------------------------------------------------------------------------------------
// Launch helpers shared by the instantiating translation units: grid (H, batch), one workgroup of
// dv/64 wavefronts per head.
// ---------------------------------------------------------------------------------------------
#define SSM_GDN_SHAPES(X, T) X(64, 64, T) X(64, 128, T) X(128, 64, T) X(128, 128, T)

// Speculative verify launches (gdn_verify.hip); gdn_launch_replay forwards multi-token calls here.
// Snapshot-based speculation (gdn_conv.hip) is declared with the other launchers.
hipError_t gdn_launch_verify(const GdnArgs& a, int dv, int dk, int bf16, int rc, int maxe,
                             hipStream_t s);

}  // namespace ssm
