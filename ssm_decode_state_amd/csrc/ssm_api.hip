// ssm_api.hip -- the C ABI (include/ssm_replay.h): validation, state layout, host-side pointer
// bounds, and kernel launches. All checks run on the host before anything is enqueued.
#include "../../include/ssm_replay.h"

#include <math.h>
#include <string.h>

#include "ssm_kernels.hpp"

namespace {

constexpr uint32_t kMagic = 0x524d5353u;  // "SSMR"
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool is_pow2_dim(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

ssm_status check_config(const ssm_config* c) {
    if (!c) return SSM_E_ARG;
    if (c->kind != SSM_MAMBA2 && c->kind != SSM_GDN && c->kind != SSM_KDA) return SSM_E_ARG;
    if (c->in_dtype != SSM_IN_F32 && c->in_dtype != SSM_IN_BF16) return SSM_E_ARG;
    if (c->readcopy < SSM_RC_NONE || c->readcopy > SSM_RC_FP4_B16) return SSM_E_ARG;
    if (c->share_ckpt != 0 && c->share_ckpt != 1) return SSM_E_ARG;
    if (c->batch < 0 || c->heads < 1 || c->groups < 1) return SSM_E_SHAPE;
    if ((int64_t)c->batch * c->heads > (int64_t)1 << 30) return SSM_E_SHAPE;
    // the kernels reach a call's token j of a sequence by a 32-bit element offset j * H * width
    const int64_t width = c->dim_p > c->dim_n ? c->dim_p : c->dim_n;
    if ((int64_t)c->heads * width * (c->max_draft > 1 ? c->max_draft : 1) >= (int64_t)1 << 31)
        return SSM_E_SHAPE;
    if (c->heads % c->groups != 0) return SSM_E_SHAPE;
    if (c->window < 1 || c->window > 32) return SSM_E_SHAPE;
    if (c->max_draft < 1 || c->max_draft > 8 || c->max_draft > c->window) return SSM_E_SHAPE;
    if (!is_pow2_dim(c->dim_p) || !is_pow2_dim(c->dim_n)) return SSM_E_SHAPE;
    if (c->kind == SSM_MAMBA2) {
        if (c->dim_p > 64) return SSM_E_SHAPE;           // one wavefront per head tile
        if (c->dim_n < 64 / c->dim_p * 4) return SSM_E_SHAPE;  // every lane group owns a quad
        // read copies: lane p owns row p, N in {64, 128}
        if (c->readcopy != SSM_RC_NONE && (c->dim_p != 64 || c->dim_n < 64)) return SSM_E_UNSUPPORTED;
    } else {
        if (c->groups != c->heads) return SSM_E_SHAPE;
        if (c->dim_p < 64 || c->dim_n < 64) return SSM_E_SHAPE;  // dv, dk in {64, 128}
        if (!isfinite(c->gdn_scale)) return SSM_E_ARG;
        // a call sees at most 32 entries (the replay kernel's sweep bound)
        if (c->window + c->max_draft - 1 > 32) return SSM_E_UNSUPPORTED;
    }
    return SSM_OK;
}

void compute_layout(const ssm_config* c, ssm_layout* L) {
    memset(L, 0, sizeof(*L));
    const uint64_t B = (uint64_t)c->batch, H = (uint64_t)c->heads, G = (uint64_t)c->groups;
    const uint64_t P = (uint64_t)c->dim_p, N = (uint64_t)c->dim_n;
    const uint64_t cap = (uint64_t)(c->window + c->max_draft - 1);
    const uint64_t esz = c->in_dtype == SSM_IN_BF16 ? 2 : 4;
    const uint64_t S = c->share_ckpt ? 2 * B : B;  // checkpoint slots (tile sets of H heads)
    L->ring_cap = (int32_t)cap;
    L->ckpt_slots = (int32_t)S;
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) { const uint64_t o = off; off = align_up(off + bytes); return o; };
    L->off_ckpt = take(S * H * P * N * 4);
    if (c->readcopy == SSM_RC_FP8_ROW) {
        L->off_rc_codes = take(S * H * P * N);
        L->off_rc_scale = take(S * H * P * 4);
        L->off_rc_tscale = take(0);
    } else if (c->readcopy == SSM_RC_FP4_B16) {
        L->off_rc_codes = take(S * H * P * N / 2);
        L->off_rc_scale = take(S * H * P * (N / 16));
        L->off_rc_tscale = take(S * H * 4);
    } else {
        L->off_rc_codes = L->off_rc_scale = L->off_rc_tscale = take(0);
    }
    if (c->kind == SSM_MAMBA2) {
        L->off_ring[0] = take(B * H * cap * P * esz);  // x
        L->off_ring[1] = take(B * G * cap * N * esz);  // B
        L->off_ring[2] = take(0);  // C is not buffered: it enters only its own token's output
        L->off_ring[3] = take(B * H * cap * 4);        // dt
        L->off_ring[4] = take(0);
    } else {
        L->off_ring[0] = take(0);  // q is not buffered: it enters only its own token's output
        L->off_ring[1] = take(B * H * cap * N * esz);  // k  (dk)
        L->off_ring[2] = take(B * H * cap * P * esz);  // v  (dv)
        L->off_ring[3] = take(B * H * cap * 4);        // beta
        L->off_ring[4] = take(B * H * cap * (c->kind == SSM_KDA ? N : 1) * 4);  // g (KDA: dk)
    }
    L->off_ptr = take(B * H * ssm::kPtrInts * 4);
    L->off_flags = take(4);
    L->off_refcnt = take(S * 4);
    L->total_bytes = off;
}

ssm_status check_state(const ssm_state* st) {
    if (!st || st->magic != kMagic || !st->mem) return SSM_E_STATE;
    return SSM_OK;
}

ssm_status hip_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_E_HIP; }

template <typename T> T* at(const ssm_state* st, uint64_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(st->mem) + off);
}

// Start and count of every sequence's ring when the host knows them (see ssm_state.ring_start):
// the kernels then skip their dependent read of the pointer entries. hstart = -1 otherwise.
void known_ptr(const ssm_state* st, int* hstart, int* hcount) {
    const bool known = !st->cfg.share_ckpt && st->ring_start >= 0 && st->count_lo == st->count_hi;
    *hstart = known ? st->ring_start : -1;
    *hcount = known ? st->count_lo : 0;
}

// The host's copy of the ring start after a fold of nfold entries from every sequence.
void advance_start(ssm_state* st, int nfold) {
    if (st->ring_start >= 0 && st->count_lo == st->count_hi)
        st->ring_start = (st->ring_start + nfold) % st->lay.ring_cap;
    else
        st->ring_start = -1;
}

ssm::M2Args m2_args(const ssm_state* st) {
    ssm::M2Args a;
    memset(&a, 0, sizeof(a));
    const ssm_layout& L = st->lay;
    a.ckpt = at<float>(st, L.off_ckpt);
    a.rc_codes = at<uint8_t>(st, L.off_rc_codes);
    a.rc_scale = at<void>(st, L.off_rc_scale);
    a.rc_tscale = at<float>(st, L.off_rc_tscale);
    a.ring_x = at<void>(st, L.off_ring[0]);
    a.ring_B = at<void>(st, L.off_ring[1]);
    a.ring_dt = at<float>(st, L.off_ring[3]);
    a.ptr = at<int>(st, L.off_ptr);
    a.refcnt = at<int>(st, L.off_refcnt);
    a.share = st->cfg.share_ckpt;
    a.A = st->A;
    a.D = st->D;
    a.batch = st->cfg.batch;
    a.heads = st->cfg.heads;
    a.groups = st->cfg.groups;
    a.cap = L.ring_cap;
    a.window = st->cfg.window;
    known_ptr(st, &a.hstart, &a.hcount);
    return a;
}

ssm::GdnArgs gdn_args(const ssm_state* st) {
    ssm::GdnArgs a;
    memset(&a, 0, sizeof(a));
    const ssm_layout& L = st->lay;
    a.ckpt = at<float>(st, L.off_ckpt);
    a.rc_codes = at<uint8_t>(st, L.off_rc_codes);
    a.rc_scale = at<void>(st, L.off_rc_scale);
    a.rc_tscale = at<float>(st, L.off_rc_tscale);
    a.ring_k = at<void>(st, L.off_ring[1]);
    a.ring_v = at<void>(st, L.off_ring[2]);
    a.ring_beta = at<float>(st, L.off_ring[3]);
    a.ring_g = at<float>(st, L.off_ring[4]);
    a.ptr = at<int>(st, L.off_ptr);
    a.refcnt = at<int>(st, L.off_refcnt);
    a.share = st->cfg.share_ckpt;
    a.scale = st->cfg.gdn_scale;
    a.batch = st->cfg.batch;
    a.heads = st->cfg.heads;
    a.cap = L.ring_cap;
    a.window = st->cfg.window;
    a.kda = st->cfg.kind == SSM_KDA;
    known_ptr(st, &a.hstart, &a.hcount);
    return a;
}

ssm_status check_inputs(const ssm_config& c, const void* in) {
    if (!in) return SSM_E_ARG;
    if (c.kind == SSM_MAMBA2) {
        const ssm_m2_in* m = static_cast<const ssm_m2_in*>(in);
        if (!m->x || !m->B || !m->C || !m->dt) return SSM_E_ARG;
        if (!aligned16(m->x) || !aligned16(m->B) || !aligned16(m->C) || !aligned16(m->dt))
            return SSM_E_ALIGN;
    } else {
        const ssm_gdn_in* g = static_cast<const ssm_gdn_in*>(in);
        if (!g->q || !g->k || !g->v || !g->beta || !g->g) return SSM_E_ARG;
        if (!aligned16(g->q) || !aligned16(g->k) || !aligned16(g->v) || !aligned16(g->beta) ||
            !aligned16(g->g))
            return SSM_E_ALIGN;
    }
    return SSM_OK;
}

// Host bounds on the committed counts after a fold of L entries from every sequence with
// count >= L (the device predicate of SSM_FLUSH_IF_FULL).
void fold_bounds(ssm_state* st) {
    const int L = st->cfg.window;
    if (st->count_hi < L) return;
    if (st->count_lo >= L) {
        st->count_lo -= L;
        st->count_hi -= L;
    } else {
        st->count_lo = 0;
        st->count_hi = (st->count_hi - L > L - 1) ? st->count_hi - L : L - 1;
    }
}

// Shared checkpoints: recount every slot's readers after a launch that can move sequences
// between slots (a fold or a fork), so that the next fold launch sees who still shares.
hipError_t recount(ssm_state* st, hipStream_t s) {
    if (!st->cfg.share_ckpt) return hipSuccess;
    return ssm::launch_recount(at<int>(st, st->lay.off_refcnt), at<int>(st, st->lay.off_ptr),
                               st->cfg.batch, st->cfg.heads, st->lay.ckpt_slots, s);
}

ssm_status launch_flush(ssm_state* st, int mode_all, hipStream_t s) {
    // lock step: every sequence folds all its entries (ALL) or the oldest L when full (IF_FULL)
    const int nfold = mode_all ? st->count_lo : (st->count_lo >= st->cfg.window ? st->cfg.window : 0);
    if (st->cfg.batch == 0) {
        advance_start(st, nfold);
        return SSM_OK;
    }
    hipError_t e;
    if (st->cfg.kind == SSM_MAMBA2) {
        ssm::M2Args a = m2_args(st);
        e = ssm::m2_launch_flush(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype, st->cfg.readcopy,
                                 mode_all, 0, s);
    } else {
        ssm::GdnArgs a = gdn_args(st);
        e = ssm::gdn_launch_flush(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                  st->cfg.readcopy, mode_all, 0, s);
    }
    if (e == hipErrorNotSupported) return SSM_E_UNSUPPORTED;
    if (e != hipSuccess) return SSM_E_HIP;
    advance_start(st, nfold);
    // a sequence that shared its checkpoint folded everything it held: its count may now be 0
    if (st->cfg.share_ckpt) st->count_lo = 0;
    return hip_status(recount(st, s));
}

}  // namespace

extern "C" {

int32_t ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(ssm_status s) {
    switch (s) {
        case SSM_OK: return "ok";
        case SSM_E_ARG: return "invalid argument";
        case SSM_E_SHAPE: return "unsupported or inconsistent shape";
        case SSM_E_ALIGN: return "device pointer not 16-byte aligned";
        case SSM_E_STATE: return "invalid state for this call";
        case SSM_E_CAPACITY: return "ring capacity exceeded";
        case SSM_E_UNSUPPORTED: return "not supported by this build";
        case SSM_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

ssm_status ssm_layout_query(const ssm_config* cfg, ssm_layout* out) {
    if (!out) return SSM_E_ARG;
    const ssm_status s = check_config(cfg);
    if (s != SSM_OK) return s;
    compute_layout(cfg, out);
    return SSM_OK;
}

ssm_status ssm_ckpt_init(ssm_state* st, const ssm_config* cfg, void* mem, uint64_t mem_bytes,
                         const float* h0, const float* A, const float* D, void* stream) {
    if (!st) return SSM_E_ARG;
    ssm_status s = check_config(cfg);
    if (s != SSM_OK) return s;
    ssm_layout lay;
    compute_layout(cfg, &lay);
    if (!mem || mem_bytes < lay.total_bytes) return SSM_E_ARG;
    if (((uintptr_t)mem & (kAlign - 1)) != 0) return SSM_E_ALIGN;
    if (h0 && !aligned16(h0)) return SSM_E_ALIGN;
    if (cfg->kind == SSM_MAMBA2) {
        if (!A || !D) return SSM_E_ARG;
        if (!aligned16(A) || !aligned16(D)) return SSM_E_ALIGN;
    }
    memset(st, 0, sizeof(*st));
    st->ring_start = cfg->share_ckpt ? -1 : 0;  // every pointer entry starts at {0, 0}
    st->cfg = *cfg;
    st->lay = lay;
    st->mem = mem;
    st->A = cfg->kind == SSM_MAMBA2 ? A : nullptr;
    st->D = cfg->kind == SSM_MAMBA2 ? D : nullptr;
    st->magic = kMagic;
    const hipStream_t hs = as_stream(stream);
    const long nheads = (long)cfg->batch * cfg->heads;
    if (nheads == 0) return SSM_OK;
    float* ck = at<float>(st, lay.off_ckpt);
    hipError_t e;
    if (h0) {  // sequence b starts in its own slot b: tile index = head index
        e = ssm::launch_pack(h0, ck, nheads, cfg->dim_p, cfg->dim_n, 0, nullptr, 0, hs);
    } else {
        e = ssm::launch_fill_i32(reinterpret_cast<int*>(ck), 0, nheads * cfg->dim_p * cfg->dim_n, hs);
    }
    if (e != hipSuccess) return SSM_E_HIP;
    e = ssm::launch_ptr_init(at<int>(st, lay.off_ptr), cfg->batch, cfg->heads, hs);
    if (e != hipSuccess) return SSM_E_HIP;
    e = recount(st, hs);
    if (e != hipSuccess) return SSM_E_HIP;
    e = ssm::launch_fill_i32(at<int>(st, lay.off_flags), 0, 1, hs);
    if (e != hipSuccess) return SSM_E_HIP;
    if (cfg->readcopy != SSM_RC_NONE) {  // the copy of the initial checkpoint
        if (cfg->kind == SSM_MAMBA2) {
            ssm::M2Args a = m2_args(st);
            e = ssm::m2_launch_flush(a, cfg->dim_p, cfg->dim_n, cfg->in_dtype, cfg->readcopy, 0, 1, hs);
        } else {
            ssm::GdnArgs a = gdn_args(st);
            e = ssm::gdn_launch_flush(a, cfg->dim_p, cfg->dim_n, cfg->in_dtype, cfg->readcopy, 0, 1, hs);
        }
        if (e != hipSuccess) return SSM_E_HIP;
    }
    return SSM_OK;
}

ssm_status ssm_replay_decode(ssm_state* st, const void* in, float* y, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (st->pending) return SSM_E_STATE;
    if (!y) return SSM_E_ARG;
    if (!aligned16(y)) return SSM_E_ALIGN;
    s = check_inputs(st->cfg, in);
    if (s != SSM_OK) return s;
    if (st->count_hi + 1 > st->lay.ring_cap) return SSM_E_CAPACITY;
    const hipStream_t hs = as_stream(stream);
    hipError_t e = hipSuccess;
    if (st->cfg.batch == 0) {
        // no sequences: nothing to launch, the host bounds still advance
    } else if (st->cfg.kind == SSM_MAMBA2) {
        ssm::M2Args a = m2_args(st);
        const ssm_m2_in* m = static_cast<const ssm_m2_in*>(in);
        a.in_x = m->x; a.in_B = m->B; a.in_C = m->C; a.in_dt = m->dt;
        a.y = y;
        a.ntok = 1;
        const int L = st->cfg.window;
        if (st->count_lo == L - 1 && st->count_hi == L - 1) {
            // lock step and this token completes every window: one pass folds the window and
            // emits the output from the new checkpoint (no replay pass, no ring append)
            e = ssm::m2_launch_flush(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                     st->cfg.readcopy, 2, 0, hs);
            if (e == hipSuccess) e = recount(st, hs);
            if (e != hipSuccess) return SSM_E_HIP;
            advance_start(st, L);  // the L - 1 buffered entries and this token
            st->count_lo = st->count_hi = 0;
            return SSM_OK;
        }
        e = ssm::m2_launch_replay(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                  st->cfg.readcopy, false, st->count_hi + 1, hs);
    } else {
        ssm::GdnArgs a = gdn_args(st);
        const ssm_gdn_in* g = static_cast<const ssm_gdn_in*>(in);
        a.in_q = g->q; a.in_k = g->k; a.in_v = g->v; a.in_beta = g->beta; a.in_g = g->g;
        a.o = y;
        a.ntok = 1;
        const int L = st->cfg.window;
        if (st->count_lo == L - 1 && st->count_hi == L - 1) {
            // as for Mamba-2 above (with a read copy, the same pass rewrites the copy)
            e = ssm::gdn_launch_flush(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                      st->cfg.readcopy, 2, 0, hs);
            if (e == hipSuccess) e = recount(st, hs);
            if (e != hipSuccess) return SSM_E_HIP;
            advance_start(st, L);  // the L - 1 buffered entries and this token
            st->count_lo = st->count_hi = 0;
            return SSM_OK;
        }
        e = ssm::gdn_launch_replay(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                   st->cfg.readcopy, false,
                                   st->count_hi + 1, hs);
    }
    if (e == hipErrorNotSupported) return SSM_E_UNSUPPORTED;
    if (e != hipSuccess) return SSM_E_HIP;
    st->count_lo += 1;
    st->count_hi += 1;
    if (st->count_hi >= st->cfg.window) {
        s = launch_flush(st, 0, hs);
        if (s != SSM_OK) return s;
        fold_bounds(st);
    }
    return SSM_OK;
}

ssm_status ssm_flush(ssm_state* st, int32_t mode, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (mode != SSM_FLUSH_IF_FULL && mode != SSM_FLUSH_ALL) return SSM_E_ARG;
    if (st->pending) return SSM_E_STATE;
    const hipStream_t hs = as_stream(stream);
    if (mode == SSM_FLUSH_IF_FULL) {
        if (st->count_hi < st->cfg.window) return SSM_OK;  // no sequence can be full
        s = launch_flush(st, 0, hs);
        if (s == SSM_OK) fold_bounds(st);
        return s;
    }
    if (st->count_hi == 0) return SSM_OK;
    s = launch_flush(st, 1, hs);
    if (s == SSM_OK) st->count_lo = st->count_hi = 0;
    return s;
}

ssm_status ssm_spec_append(ssm_state* st, int32_t ndraft, const void* in, float* y, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (st->pending) return SSM_E_STATE;
    if (ndraft < 1) return SSM_E_ARG;
    if (ndraft > st->cfg.max_draft) return SSM_E_CAPACITY;
    if (!y) return SSM_E_ARG;
    if (!aligned16(y)) return SSM_E_ALIGN;
    s = check_inputs(st->cfg, in);
    if (s != SSM_OK) return s;
    if (st->count_hi + ndraft > st->lay.ring_cap) return SSM_E_CAPACITY;
    if (st->cfg.batch > 0) {
        hipError_t e;
        if (st->cfg.kind == SSM_MAMBA2) {
            ssm::M2Args a = m2_args(st);
            const ssm_m2_in* m = static_cast<const ssm_m2_in*>(in);
            a.in_x = m->x; a.in_B = m->B; a.in_C = m->C; a.in_dt = m->dt;
            a.y = y;
            a.ntok = ndraft;
            e = ssm::m2_launch_replay(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                      st->cfg.readcopy, true, st->count_hi + ndraft,
                                      as_stream(stream));
        } else {
            ssm::GdnArgs a = gdn_args(st);
            const ssm_gdn_in* g = static_cast<const ssm_gdn_in*>(in);
            a.in_q = g->q; a.in_k = g->k; a.in_v = g->v; a.in_beta = g->beta; a.in_g = g->g;
            a.o = y;
            a.ntok = ndraft;
            e = ssm::gdn_launch_replay(a, st->cfg.dim_p, st->cfg.dim_n, st->cfg.in_dtype,
                                       st->cfg.readcopy, true,
                                       st->count_hi + ndraft, as_stream(stream));
        }
        if (e != hipSuccess) return SSM_E_HIP;
    }
    st->pending = ndraft;
    return SSM_OK;
}

ssm_status ssm_spec_rollback(ssm_state* st, const int32_t* n_accept, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (!st->pending) return SSM_E_STATE;
    if (!n_accept) return SSM_E_ARG;
    if (((uintptr_t)n_accept & 3u) != 0) return SSM_E_ALIGN;
    const hipStream_t hs = as_stream(stream);
    const hipError_t e = ssm::launch_commit(at<int>(st, st->lay.off_ptr), n_accept, st->cfg.batch,
                                            st->cfg.heads, st->pending, at<int>(st, st->lay.off_flags),
                                            hs);
    if (e != hipSuccess) return SSM_E_HIP;
    st->ring_start = -1;  // the accepted counts are known only on the device
    st->count_hi += st->pending;
    st->pending = 0;
    // a flush fires whenever a sequence's committed count reaches L
    if (st->count_hi >= st->cfg.window) {
        s = launch_flush(st, 0, hs);
        if (s != SSM_OK) return s;
        fold_bounds(st);
    }
    return SSM_OK;
}

ssm_status ssm_restore(ssm_state* st, const int32_t* n_back, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (st->pending) return SSM_E_STATE;
    if (!n_back) return SSM_E_ARG;
    if (((uintptr_t)n_back & 3u) != 0) return SSM_E_ALIGN;
    const hipError_t e = ssm::launch_restore(at<int>(st, st->lay.off_ptr), n_back, st->cfg.batch,
                                             st->cfg.heads, as_stream(stream));
    if (e != hipSuccess) return SSM_E_HIP;
    st->count_lo = 0;  // the rewound counts are known only on the device
    st->ring_start = -1;
    return SSM_OK;
}

ssm_status ssm_fork(ssm_state* st, const int32_t* src, const int32_t* dst, int32_t n, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (st->pending) return SSM_E_STATE;
    if (n < 0 || (n > 0 && (!src || !dst))) return SSM_E_ARG;
    const int B = st->cfg.batch;
    for (int i = 0; i < n; ++i) {
        if (src[i] < 0 || src[i] >= B || dst[i] < 0 || dst[i] >= B) return SSM_E_ARG;
        for (int j = 0; j < n; ++j) {
            if (j != i && dst[j] == dst[i]) return SSM_E_ARG;  // one source per destination
            if (dst[i] == src[j]) return SSM_E_ARG;            // no chains within one call
        }
    }
    if (n == 0) return SSM_OK;
    // every region's per-sequence slice (the layout's regions are all [batch][...]); with shared
    // checkpoints the copies point at the source's checkpoint slot instead of copying its tiles
    const ssm_config& c = st->cfg;
    const ssm_layout& L = st->lay;
    const uint64_t H = c.heads, G = c.groups, P = c.dim_p, N = c.dim_n, cap = L.ring_cap;
    const uint64_t esz = c.in_dtype == SSM_IN_BF16 ? 2 : 4;
    ssm::ForkRegions r;
    memset(&r, 0, sizeof(r));
    auto add = [&](uint64_t off, uint64_t slice) {
        if (slice) { r.off[r.n] = off; r.slice[r.n] = slice; ++r.n; }
    };
    if (!c.share_ckpt) {
        add(L.off_ckpt, H * P * N * 4);
        if (c.readcopy == SSM_RC_FP8_ROW) {
            add(L.off_rc_codes, H * P * N);
            add(L.off_rc_scale, H * P * 4);
        } else if (c.readcopy == SSM_RC_FP4_B16) {
            add(L.off_rc_codes, H * P * N / 2);
            add(L.off_rc_scale, H * P * (N / 16));
            add(L.off_rc_tscale, H * 4);
        }
    }
    if (c.kind == SSM_MAMBA2) {
        add(L.off_ring[0], H * cap * P * esz);
        add(L.off_ring[1], G * cap * N * esz);
        add(L.off_ring[3], H * cap * 4);
    } else {
        add(L.off_ring[1], H * cap * N * esz);
        add(L.off_ring[2], H * cap * P * esz);
        add(L.off_ring[3], H * cap * 4);
        add(L.off_ring[4], H * cap * (c.kind == SSM_KDA ? N : 1) * 4);
    }
    add(L.off_ptr, H * ssm::kPtrInts * 4);  // start, count and checkpoint slot
    const hipStream_t hs = as_stream(stream);
    for (int i0 = 0; i0 < n; i0 += ssm::kMaxForkPairs) {
        ssm::ForkPairs p;
        memset(&p, 0, sizeof(p));
        p.n = n - i0 < ssm::kMaxForkPairs ? n - i0 : ssm::kMaxForkPairs;
        for (int i = 0; i < p.n; ++i) {
            p.src[i] = src[i0 + i];
            p.dst[i] = dst[i0 + i];
        }
        const hipError_t e = ssm::launch_fork_copy(static_cast<char*>(st->mem), r, p, hs);
        if (e != hipSuccess) return SSM_E_HIP;
    }
    if (recount(st, hs) != hipSuccess) return SSM_E_HIP;
    // the copies' pointers are their sources': the host bounds (and a start that every
    // sequence shares) still hold
    return SSM_OK;
}

ssm_status ssm_ckpt_export(const ssm_state* st, float* h_out, void* stream) {
    ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (!h_out) return SSM_E_ARG;
    if (!aligned16(h_out)) return SSM_E_ALIGN;
    const long nheads = (long)st->cfg.batch * st->cfg.heads;
    return hip_status(ssm::launch_pack(at<float>(st, st->lay.off_ckpt), h_out, nheads,
                                       st->cfg.dim_p, st->cfg.dim_n, 1,
                                       st->cfg.share_ckpt ? at<int>(st, st->lay.off_ptr) : nullptr,
                                       st->cfg.heads, as_stream(stream)));
}

ssm_status ssm_conventional_step(const ssm_config* cfg, float* h, const void* in, const float* A,
                                 const float* D, float* y, void* stream) {
    ssm_config c;
    if (!cfg) return SSM_E_ARG;
    c = *cfg;
    c.readcopy = SSM_RC_NONE;  // the conventional step reads and writes the fp32 state itself
    ssm_status s = check_config(&c);
    if (s != SSM_OK) return s;
    if (!h || !y) return SSM_E_ARG;
    if (!aligned16(h) || !aligned16(y)) return SSM_E_ALIGN;
    s = check_inputs(c, in);
    if (s != SSM_OK) return s;
    if (c.batch == 0) return SSM_OK;
    hipError_t e;
    if (c.kind == SSM_MAMBA2) {
        if (!A || !D) return SSM_E_ARG;
        if (!aligned16(A) || !aligned16(D)) return SSM_E_ALIGN;
        const ssm_m2_in* m = static_cast<const ssm_m2_in*>(in);
        ssm::M2ConvArgs a{h, m->x, m->B, m->C, m->dt, A, D, y, c.batch, c.heads, c.groups};
        e = ssm::m2_launch_conv(a, c.dim_p, c.dim_n, c.in_dtype, as_stream(stream));
    } else {
        const ssm_gdn_in* g = static_cast<const ssm_gdn_in*>(in);
        ssm::GdnConvArgs a{h, g->q, g->k, g->v, g->beta, g->g, y, c.gdn_scale, c.batch, c.heads,
                           c.kind == SSM_KDA};
        e = ssm::gdn_launch_conv(a, c.dim_p, c.dim_n, c.in_dtype, as_stream(stream));
    }
    if (e == hipErrorNotSupported) return SSM_E_UNSUPPORTED;
    return hip_status(e);
}

static ssm_status check_spec_baseline(const ssm_config* cfg, ssm_config* c, int32_t ndraft) {
    if (!cfg) return SSM_E_ARG;
    *c = *cfg;
    c->readcopy = SSM_RC_NONE;
    const ssm_status s = check_config(c);
    if (s != SSM_OK) return s;
    if (ndraft < 1 || ndraft > 8) return SSM_E_CAPACITY;
    return SSM_OK;
}

ssm_status ssm_conventional_spec_snapshot(const ssm_config* cfg, const float* h, float* h_snap,
                                          int32_t ndraft, const void* in, const float* A,
                                          const float* D, float* y, void* stream) {
    ssm_config c;
    ssm_status s = check_spec_baseline(cfg, &c, ndraft);
    if (s != SSM_OK) return s;
    if (!h || !h_snap || !y) return SSM_E_ARG;
    if (!aligned16(h) || !aligned16(h_snap) || !aligned16(y)) return SSM_E_ALIGN;
    if (c.kind == SSM_MAMBA2) {
        if (!A || !D) return SSM_E_ARG;
        if (!aligned16(A) || !aligned16(D)) return SSM_E_ALIGN;
    }
    s = check_inputs(c, in);
    if (s != SSM_OK) return s;
    if (c.batch == 0) return SSM_OK;
    hipError_t e;
    if (c.kind == SSM_MAMBA2) {
        const ssm_m2_in* m = static_cast<const ssm_m2_in*>(in);
        ssm::M2ConvArgs a{const_cast<float*>(h), m->x, m->B, m->C, m->dt, A, D, y,
                          c.batch, c.heads, c.groups, h_snap, ndraft};
        e = ssm::m2_launch_snapshot(a, c.dim_p, c.dim_n, c.in_dtype, as_stream(stream));
    } else {
        const ssm_gdn_in* g = static_cast<const ssm_gdn_in*>(in);
        ssm::GdnConvArgs a{const_cast<float*>(h), g->q, g->k, g->v, g->beta, g->g, y,
                           c.gdn_scale, c.batch, c.heads, c.kind == SSM_KDA, h_snap, ndraft};
        e = ssm::gdn_launch_snapshot(a, c.dim_p, c.dim_n, c.in_dtype, as_stream(stream));
    }
    if (e == hipErrorNotSupported) return SSM_E_UNSUPPORTED;
    return hip_status(e);
}

ssm_status ssm_conventional_spec_select(const ssm_config* cfg, float* h, const float* h_snap,
                                        int32_t ndraft, const int32_t* n_accept, void* stream) {
    ssm_config c;
    const ssm_status s = check_spec_baseline(cfg, &c, ndraft);
    if (s != SSM_OK) return s;
    if (!h || !h_snap || !n_accept) return SSM_E_ARG;
    if (!aligned16(h) || !aligned16(h_snap) || ((uintptr_t)n_accept & 3u) != 0) return SSM_E_ALIGN;
    if (c.batch == 0) return SSM_OK;
    return hip_status(ssm::launch_snap_select(h, h_snap, n_accept, c.batch,
                                              (long)c.heads * c.dim_p * c.dim_n, ndraft,
                                              as_stream(stream)));
}

ssm_status ssm_debug_flags(const ssm_state* st, int32_t* host_flags, int32_t clear, void* stream) {
    const ssm_status s = check_state(st);
    if (s != SSM_OK) return s;
    if (!host_flags) return SSM_E_ARG;
    const hipStream_t hs = as_stream(stream);
    int* dflags = reinterpret_cast<int*>(static_cast<char*>(st->mem) + st->lay.off_flags);
    hipError_t e = hipMemcpyAsync(host_flags, dflags, sizeof(int32_t), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e == hipSuccess && clear) e = ssm::launch_fill_i32(dflags, 0, 1, hs);
    return hip_status(e);
}

static ssm_status pack_common(const ssm_config* cfg, const float* src, float* dst, int unpack,
                              void* stream) {
    ssm_config c;
    if (!cfg) return SSM_E_ARG;
    c = *cfg;
    c.readcopy = SSM_RC_NONE;
    const ssm_status s = check_config(&c);
    if (s != SSM_OK) return s;
    if (!src || !dst) return SSM_E_ARG;
    if (!aligned16(src) || !aligned16(dst)) return SSM_E_ALIGN;
    return hip_status(ssm::launch_pack(src, dst, (long)c.batch * c.heads, c.dim_p, c.dim_n, unpack,
                                       nullptr, 0, as_stream(stream)));
}

ssm_status ssm_tiles_pack(const ssm_config* cfg, const float* natural, float* tiles, void* stream) {
    return pack_common(cfg, natural, tiles, 0, stream);
}

ssm_status ssm_tiles_unpack(const ssm_config* cfg, const float* tiles, float* natural,
                            void* stream) {
    return pack_common(cfg, tiles, natural, 1, stream);
}

ssm_status ssm_debug_codec(int32_t op, const void* in, void* out, int64_t n, void* stream) {
    if (op < 0 || op > 11 || n < 0) return SSM_E_ARG;
    if (n > 0 && (!in || !out)) return SSM_E_ARG;
    return hip_status(ssm::launch_codec(op, in, out, (long)n, as_stream(stream)));
}

ssm_status ssm_debug_stream_read(const void* src, uint64_t bytes, uint32_t* out, int32_t blocks,
                                 void* stream) {
    if (blocks < 1 || blocks > (1 << 20) || (bytes % 16) != 0) return SSM_E_ARG;
    if (bytes > 0 && (!src || !out)) return SSM_E_ARG;
    if (!aligned16(src) || ((uintptr_t)out & 3u) != 0) return SSM_E_ALIGN;
    return hip_status(ssm::launch_stream_read(src, (long)bytes, out, blocks, as_stream(stream)));
}

}  // extern "C"
