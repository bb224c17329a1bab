// Sanitizer driver for the host half of the C ABI (ssm_api.hip built host-only with AddressSanitizer
// and UndefinedBehaviorSanitizer, linked with the launcher stand-ins of abi_host_stubs.cpp). It runs
// without a GPU: every device address is a fake, unmapped one, and the stand-ins check that each
// region a launch would touch lies inside the state. Covered: the layout arithmetic for small and
// very large states (offsets past 4 GiB), lock-step decode with its fused folds and the host's ring
// start, speculation and its capacity checks, restore, fork (region slicing with 64-bit offsets),
// flush, export, the conventional and snapshot comparison points, and argument validation.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/ssm_replay.h"
#include "abi_host_stubs.h"

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            exit(1);                                                                 \
        }                                                                            \
    } while (0)

// fake device addresses (256-byte aligned, never mapped)
static const uintptr_t kMem = 0x7F0000000000ull, kIn = 0x7E0000000000ull;
static const uintptr_t kOut = 0x7D0000000000ull, kAux = 0x7C0000000000ull;

static ssm_config make(int kind, int B, int H, int G, int P, int N, int L, int S, int bf16, int rc,
                       int share) {
    ssm_config c;
    memset(&c, 0, sizeof(c));
    c.kind = kind; c.batch = B; c.heads = H; c.groups = G; c.dim_p = P; c.dim_n = N;
    c.window = L; c.max_draft = S; c.in_dtype = bf16 ? SSM_IN_BF16 : SSM_IN_F32;
    c.readcopy = rc; c.gdn_scale = 1.0f; c.share_ckpt = share;
    return c;
}

static void check_layout(const ssm_config& c, const ssm_layout& L) {
    const uint64_t B = c.batch, H = c.heads, G = c.groups, P = c.dim_p, N = c.dim_n;
    const uint64_t cap = L.ring_cap, esz = c.in_dtype == SSM_IN_BF16 ? 2 : 4;
    const uint64_t S = L.ckpt_slots;
    CHECK(cap == (uint64_t)(c.window + c.max_draft - 1));
    CHECK(S == (c.share_ckpt ? 2 * B : B));
    struct R { uint64_t off, bytes; } r[14];
    int n = 0;
    r[n++] = {L.off_ckpt, S * H * P * N * 4};
    if (c.readcopy == SSM_RC_FP8_ROW) {
        r[n++] = {L.off_rc_codes, S * H * P * N};
        r[n++] = {L.off_rc_scale, S * H * P * 4};
    } else if (c.readcopy == SSM_RC_FP4_B16) {
        r[n++] = {L.off_rc_codes, S * H * P * N / 2};
        r[n++] = {L.off_rc_scale, S * H * P * (N / 16)};
        r[n++] = {L.off_rc_tscale, S * H * 4};
    }
    if (c.kind == SSM_MAMBA2) {
        r[n++] = {L.off_ring[0], B * H * cap * P * esz};
        r[n++] = {L.off_ring[1], B * G * cap * N * esz};
        r[n++] = {L.off_ring[2], 0};  // C is not buffered
        r[n++] = {L.off_ring[3], B * H * cap * 4};
    } else {
        r[n++] = {L.off_ring[0], 0};  // q is not buffered
        r[n++] = {L.off_ring[1], B * H * cap * N * esz};
        r[n++] = {L.off_ring[2], B * H * cap * P * esz};
        r[n++] = {L.off_ring[3], B * H * cap * 4};
        r[n++] = {L.off_ring[4], B * H * cap * (c.kind == SSM_KDA ? N : 1) * 4};
    }
    r[n++] = {L.off_ptr, B * H * 16};
    r[n++] = {L.off_flags, 4};
    r[n++] = {L.off_refcnt, S * 4};
    for (int i = 0; i < n; ++i) {
        CHECK(r[i].off % 256 == 0);
        CHECK(r[i].off + r[i].bytes <= L.total_bytes);
        if (i + 1 < n) CHECK(r[i].off + r[i].bytes <= r[i + 1].off);  // in order, disjoint
    }
}

static void register_state(const ssm_config& c, const ssm_layout& L) {
    g_world.mem = kMem;
    g_world.total = L.total_bytes;
    g_world.slots = L.ckpt_slots;
    g_world.P = c.dim_p;
    g_world.N = c.dim_n;
    g_world.esz = c.in_dtype == SSM_IN_BF16 ? 2 : 4;
    g_world.batch = c.batch;
    g_world.rc = c.readcopy;
}

static void drive(const ssm_config& c) {
    fprintf(stderr, "config: kind %d batch %d heads %d tile %dx%d window %d drafts %d copy %d share %d\n",
            c.kind, c.batch, c.heads, c.dim_p, c.dim_n, c.window, c.max_draft, c.readcopy,
            c.share_ckpt);
    ssm_layout L;
    CHECK(ssm_layout_query(&c, &L) == SSM_OK);
    check_layout(c, L);
    register_state(c, L);
    const bool m2 = c.kind == SSM_MAMBA2;
    const float* A = m2 ? (const float*)kAux : nullptr;
    const float* D = m2 ? (const float*)(kAux + 4096) : nullptr;
    ssm_state st;
    memset(&st, 0, sizeof(st));
    CHECK(ssm_ckpt_init(&st, &c, (void*)kMem, L.total_bytes - 1, nullptr, A, D, nullptr) == SSM_E_ARG);
    CHECK(ssm_ckpt_init(&st, &c, (void*)(kMem + 16), L.total_bytes, nullptr, A, D, nullptr) == SSM_E_ALIGN);
    CHECK(ssm_ckpt_init(&st, &c, (void*)kMem, L.total_bytes, (const float*)kIn, A, D, nullptr) == SSM_OK);
    ssm_m2_in mi = {(const void*)kIn, (const void*)(kIn + (1 << 24)), (const void*)(kIn + (2 << 24)),
                    (const float*)(kIn + (3 << 24))};
    ssm_gdn_in gi = {(const void*)kIn, (const void*)(kIn + (1 << 24)), (const void*)(kIn + (2 << 24)),
                     (const float*)(kIn + (3 << 24)), (const float*)(kIn + (4 << 24))};
    const void* in = m2 ? (const void*)&mi : (const void*)&gi;
    float* y = (float*)kOut;
    const int Lw = c.window;

    // lock-step decode: two whole windows and three more tokens
    const long fused0 = g_world.calls[kFused], fold0 = g_world.calls[kFold];
    const int ntok = 2 * Lw + 3, nwin = ntok / Lw, rest = ntok % Lw;
    for (int t = 0; t < ntok; ++t) CHECK(ssm_replay_decode(&st, in, y, nullptr) == SSM_OK);
    if (c.share_ckpt) {
        // a fold launch may move a sequence that shared its slot, folding whatever it held, so
        // the host keeps only bounds: [0, count] and folds are device predicates from there on
        CHECK(g_world.calls[kFused] + g_world.calls[kFold] - fused0 - fold0 >= (c.batch > 0 ? nwin : 0));
        CHECK(st.count_lo <= rest && rest <= st.count_hi && st.count_hi <= L.ring_cap);
    } else {
        if (c.batch > 0) {
            CHECK(g_world.calls[kFused] - fused0 == nwin);  // every window closes in one pass
            CHECK(g_world.calls[kFold] - fold0 == 0);
        }
        CHECK(st.count_lo == rest && st.count_hi == rest);
        CHECK(st.ring_start == (nwin * Lw) % L.ring_cap);
    }

    // speculation: drafts pending block decode; capacity is checked against the host bounds
    if (c.max_draft > 1) {
        CHECK(ssm_spec_append(&st, c.max_draft + 1, in, y, nullptr) == SSM_E_CAPACITY);
        CHECK(ssm_spec_append(&st, c.max_draft, in, y, nullptr) == SSM_OK);
        CHECK(st.pending == c.max_draft);
        CHECK(ssm_replay_decode(&st, in, y, nullptr) == SSM_E_STATE);
        CHECK(ssm_spec_append(&st, 1, in, y, nullptr) == SSM_E_STATE);
        CHECK(ssm_spec_rollback(&st, (const int32_t*)(kAux + 2), nullptr) == SSM_E_ALIGN);
        CHECK(ssm_spec_rollback(&st, (const int32_t*)kAux, nullptr) == SSM_OK);
        CHECK(st.pending == 0 && st.ring_start == -1 && st.count_lo <= st.count_hi);
        CHECK(st.count_hi < Lw + c.max_draft);
        for (int r = 0; r < 3 * Lw; ++r) {  // rounds never overflow the ring
            const ssm_status s = ssm_spec_append(&st, c.max_draft, in, y, nullptr);
            CHECK(s == SSM_OK);
            CHECK(ssm_spec_rollback(&st, (const int32_t*)kAux, nullptr) == SSM_OK);
            CHECK(st.count_hi <= L.ring_cap);
        }
    }
    CHECK(ssm_restore(&st, (const int32_t*)kAux, nullptr) == SSM_OK);
    CHECK(st.count_lo == 0);

    // fork: the first half of the sequences into the second half, and validation
    if (c.batch >= 2) {
        int src[64], dst[64], n = 0;
        for (int b = 0; b + c.batch / 2 < c.batch && n < 64; ++b, ++n) {
            src[n] = b;
            dst[n] = c.batch - 1 - b;
            if (dst[n] <= src[n]) break;
        }
        CHECK(ssm_fork(&st, src, dst, n, nullptr) == SSM_OK);
        int s2[2] = {0, 0}, d2[2] = {1, 1};
        CHECK(ssm_fork(&st, s2, d2, 2, nullptr) == SSM_E_ARG);  // one source per destination
        int s3[2] = {0, 1}, d3[2] = {1, 2};
        CHECK(ssm_fork(&st, s3, d3, 2, nullptr) == SSM_E_ARG);  // no chains within a call
        int s4[1] = {c.batch}, d4[1] = {0};
        CHECK(ssm_fork(&st, s4, d4, 1, nullptr) == SSM_E_ARG);  // out of range
        CHECK(ssm_fork(&st, src, dst, 0, nullptr) == SSM_OK);
    }
    CHECK(ssm_flush(&st, SSM_FLUSH_ALL, nullptr) == SSM_OK);
    CHECK(ssm_flush(&st, 7, nullptr) == SSM_E_ARG);
    CHECK(ssm_ckpt_export(&st, (float*)kOut, nullptr) == SSM_OK);
    CHECK(ssm_ckpt_export(&st, (float*)(kOut + 4), nullptr) == SSM_E_ALIGN);

    // the comparison points
    CHECK(ssm_conventional_step(&c, (float*)kAux, in, A, D, y, nullptr) == SSM_OK);
    if (c.batch > 0 && c.max_draft > 1) {
        CHECK(ssm_conventional_spec_snapshot(&c, (const float*)kAux, (float*)(kAux + (1ull << 36)),
                                             c.max_draft, in, A, D, y, nullptr) == SSM_OK);
        CHECK(ssm_conventional_spec_select(&c, (float*)kAux, (const float*)(kAux + (1ull << 36)),
                                           c.max_draft, (const int32_t*)kIn, nullptr) == SSM_OK);
    }
}

int main() {
    // the supported shape set, every layer type and read copy, with and without shared slots
    const int kinds[3] = {SSM_MAMBA2, SSM_GDN, SSM_KDA};
    int n = 0;
    for (int kind : kinds)
        for (int rc = 0; rc <= 2; ++rc)
            for (int share = 0; share <= 1; ++share)
                for (int S : {1, 4}) {
                    const bool m2 = kind == SSM_MAMBA2;
                    const int P = m2 ? 64 : 128, N = 128, H = m2 ? 8 : 3, G = m2 ? 4 : H;
                    drive(make(kind, 5, H, G, P, N, 16, S, 1, rc, share));
                    drive(make(kind, 3, H, G, P, 64, 4, S > 4 ? 4 : S, 0, rc, share));
                    n += 2;
                }
    // small tiles and windows at the edges of the supported set
    drive(make(SSM_MAMBA2, 2, 4, 4, 16, 16, 1, 1, 0, 0, 0));
    drive(make(SSM_MAMBA2, 2, 6, 3, 32, 16 * 2, 32, 8, 1, 0, 1));
    drive(make(SSM_GDN, 2, 2, 2, 64, 64, 25, 8, 1, 0, 0));
    drive(make(SSM_MAMBA2, 0, 128, 128, 64, 128, 16, 4, 1, 1, 1));  // no sequences: every call a no-op
    // serving layers and far larger batches: offsets past 4 GiB, fork slices near the top
    drive(make(SSM_MAMBA2, 256, 128, 128, 64, 128, 16, 4, 1, 2, 1));
    drive(make(SSM_MAMBA2, 4096, 128, 128, 64, 128, 16, 4, 1, 1, 1));
    drive(make(SSM_GDN, 8192, 32, 32, 128, 128, 16, 4, 1, 2, 0));
    drive(make(SSM_KDA, 8192, 32, 32, 128, 128, 16, 4, 1, 0, 1));
    n += 8;
    // configurations the layout must reject
    ssm_layout L;
    ssm_config bad = make(SSM_MAMBA2, 1 << 20, 2048, 2048, 64, 128, 16, 1, 1, 0, 0);
    CHECK(ssm_layout_query(&bad, &L) == SSM_E_SHAPE);  // batch * heads > 2^30
    bad = make(SSM_GDN, 2, 4, 4, 128, 128, 32, 2, 1, 0, 0);
    CHECK(ssm_layout_query(&bad, &L) == SSM_E_UNSUPPORTED);  // a call could see 33 entries
    bad = make(SSM_MAMBA2, 2, 4, 3, 64, 128, 16, 1, 1, 0, 0);
    CHECK(ssm_layout_query(&bad, &L) == SSM_E_SHAPE);  // H % G != 0
    printf("host ABI sanitizer run: %d configurations, replay %ld, verify %ld, fold %ld, fused %ld, "
           "fork %ld\n", n, g_world.calls[kReplay], g_world.calls[kVerify], g_world.calls[kFold],
           g_world.calls[kFused], g_world.calls[kFork]);
    return 0;
}
