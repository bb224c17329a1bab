/*
 * ssm_replay.h -- C ABI of the ReplaySSM decode library for MI355X (gfx950).
 *
 * What the library computes. The pages this follows ("ReplaySSM: Rethinking State Storage for
 * Faster Hybrid-Model Decoding": the deskofai.com news article, paragraphs counted from the first
 * body paragraph, and the nexus-ai-blog.com explainer, cited by section heading) describe the SSM
 * layer's decode state kept as a high-precision checkpoint plus a buffer of the most recent inputs
 * (news, para 2). Each token's output is computed from the checkpoint and the buffered inputs
 * without writing the state; the buffer is folded into the checkpoint when it fills, and
 * speculative drafts are appended to the buffer and rejected by moving a pointer, with no
 * per-token snapshots (news, para 3). An optional low-precision copy of the checkpoint serves the
 * reads while the recurrence stays in high precision (news, para 4). The window L is a parameter;
 * 16 is the value the news article reports as the default (news, para 6).
 *
 * The two layer types (both named as SSM layers in the news article, para 7) follow their
 * published definitions:
 *   Mamba-2 (per head, state h in R^{P x N}, scalar A < 0 and D per head, B/C shared by a group):
 *     h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T,      y_t = h_t C_t + D x_t
 *   Gated DeltaNet (per head, state S in R^{dv x dk}, alpha_t = exp(g_t)):
 *     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = scale S_t q_t
 *   Kimi Delta Attention (named beside them in the feed excerpt and news para 7): the same with
 *   one decay per key channel, D_t = diag(exp(g_t)), g_t in R^{dk}:
 *     S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) k_t^T,           o_t = scale S_t q_t
 * Replay computes exactly these outputs (up to fp32 rounding) from the checkpoint h_c at token
 * position c and the buffered entries c+1..c+k:
 *   Mamba-2: y_k = e^{s_0} h_c C_k + sum_{i<=k} e^{s_i} dt_i (B_i . C_k) x_i + D x_k,
 *            s_i = A * sum_{m=i+1..k} dt_m
 *   GDN:     backward sweep r <- q_k; for i = k..1: c_i = beta_i (k_i . r), acc += c_i v_i,
 *            r <- alpha_i (r - c_i k_i); o = scale (S_c r + acc)   (KDA: alpha_i elementwise)
 *
 * Conventions shared by every entry point
 * - All device pointers are plain device addresses (hipMalloc / torch CUDA tensors) and must be
 *   16-byte aligned. `stream` is a hipStream_t (NULL = the null stream); all work is enqueued
 *   asynchronously on it and the call returns without synchronizing.
 * - The library allocates no device memory. The caller allocates `ssm_layout.total_bytes` of device
 *   memory for a state and keeps it alive while work on it is in flight.
 * - `ssm_state` is a plain host struct owned by the caller; it holds host-side mirrors (pending
 *   drafts, bounds on the committed count) that the entry points update. One state must be used by
 *   one host thread and one stream at a time; distinct states are independent.
 * - Every call validates its arguments on the host first and returns a negative status BEFORE
 *   enqueueing anything when they are wrong. SSM_E_HIP reports a failed launch; device faults
 *   surface at the caller's next synchronization, as usual in HIP.
 * - Input tensors (natural layouts, last index fastest; ntok = 1 for decode, ndraft for drafts):
 *     Mamba-2: x [batch][ntok][H][P], B and C [batch][ntok][G][N] in the input dtype,
 *              dt [batch][ntok][H] fp32 (already positive: the caller applies softplus/bias)
 *     GDN:     q, k [batch][ntok][H][dk], v [batch][ntok][H][dv] in the input dtype,
 *              beta [batch][ntok][H], g [batch][ntok][H] fp32 (g is the log of the decay)
 *     KDA:     as GDN (ssm_gdn_in) with g [batch][ntok][H][dk] fp32, one log-decay per channel
 *   Outputs y are fp32 [batch][ntok][H][P] (GDN: [batch][ntok][H][dv]).
 * - Supported shapes: Mamba-2 P in {16, 32, 64} and N in {16, 32, 64, 128} with N >= 4 * 64 / P
 *   (P = 64 takes every N); GDN dv and dk in {64, 128}; window L in [1, 32]; max_draft in
 *   [1, min(L, 8)], and for GDN / KDA L + max_draft - 1 <= 32 (SSM_E_UNSUPPORTED otherwise).
 *   KDA takes the GDN shapes. The read copies need N (dk) in {64, 128}, and P = 64 for Mamba-2.
 *   batch * heads <= 2^30 and heads * max(P, N) * max_draft < 2^31 (SSM_E_SHAPE otherwise: the
 *   kernels address a call's token rows with 32-bit offsets from each sequence's first token).
 */
#ifndef SSM_REPLAY_H
#define SSM_REPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 5

typedef int32_t ssm_status;
enum {
    SSM_OK = 0,
    SSM_E_ARG = -1,         /* null pointer, bad enum value, bad flag */
    SSM_E_SHAPE = -2,       /* dimension out of the supported set, H % G != 0, ... */
    SSM_E_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
    SSM_E_STATE = -4,       /* bad magic, decode/flush with drafts pending, rollback w/o drafts */
    SSM_E_CAPACITY = -5,    /* the ring could overflow (ndraft too large for the free slots) */
    SSM_E_UNSUPPORTED = -6, /* valid request this build does not implement */
    SSM_E_HIP = -7          /* a HIP launch failed */
};

enum { SSM_MAMBA2 = 0, SSM_GDN = 1, SSM_KDA = 2 };
enum { SSM_IN_F32 = 0, SSM_IN_BF16 = 1 };
enum { SSM_RC_NONE = 0, SSM_RC_FP8_ROW = 1, SSM_RC_FP4_B16 = 2 };
enum { SSM_FLUSH_IF_FULL = 0, SSM_FLUSH_ALL = 1 };
/* Bits of a state's device flag word (see ssm_debug_flags). */
enum { SSM_FLAG_ACCEPT_CLAMPED = 1 /* an n_accept value outside [0, pending] was clamped */ };

/* Layer shape and options. */
typedef struct ssm_config {
    int32_t kind;      /* SSM_MAMBA2, SSM_GDN or SSM_KDA */
    int32_t batch;     /* sequences B (0 allowed: every call is then a no-op) */
    int32_t heads;     /* H */
    int32_t groups;    /* Mamba-2: B/C groups G, H % G == 0 (head h uses group h / (H/G)); GDN/KDA: H */
    int32_t dim_p;     /* Mamba-2 head dim P; GDN value dim dv (rows of a state tile) */
    int32_t dim_n;     /* Mamba-2 state dim N; GDN key dim dk (columns of a state tile) */
    int32_t window;    /* L: the buffer is folded into the checkpoint when L entries are committed */
    int32_t max_draft; /* most drafts per ssm_spec_append (1 = no speculation) */
    int32_t in_dtype;  /* SSM_IN_F32 or SSM_IN_BF16 for x/B/C (q/k/v); dt/beta/g are always fp32 */
    int32_t readcopy;  /* SSM_RC_*: low-precision copy read by the output path */
    float gdn_scale;   /* GDN / KDA output scale (1.0 = none); ignored for Mamba-2 */
    int32_t share_ckpt; /* 1: ssm_fork shares checkpoints (2 batch checkpoint slots); 0: it copies */
} ssm_config;

/* Byte offsets of the regions inside one state's device memory (each 256-byte aligned).
 * Checkpoint slots: the checkpoint region holds ckpt_slots sets of H tiles (batch, or 2 batch
 * with share_ckpt). Without share_ckpt sequence b always uses slot b (its pointers' slot field
 * is not read); with it, sequence b reads the slot s recorded in its pointers: b, batch + b, or
 * a fork source's slot. t = s*H + h is the tile index of head (b, h). Checkpoint tile layout ("quad-interleaved"): tile t starts at float
 * offset t*P*N and element (p, n) sits at float ((n/4)*P + p)*4 + n%4, i.e. groups of four
 * consecutive n of one row are 16-byte units and consecutive rows' units are adjacent. The read
 * copy follows the tiles' slots and uses the same idea with wider units: fp8 codes of tile t at
 * byte t*P*N + ((n/16)*P + p)*16 + n%16, row scales fp32 [t][P]; fp4 codes (two per byte, low
 * nibble = even n) at byte t*P*N/2 + ((n/32)*P + p)*16 + (n%32)/2, block-scale E4M3 codes
 * [t][P][N/16], tile scale fp32 [t].
 * Rings (slot s of cap) hold the inputs the state update consumes: Mamba-2 x [b][h][s][P],
 * B [b][g][s][N] (input dtype), dt [b][h][s] fp32; GDN k [b][h][s][dk], v [b][h][s][dv] (input
 * dtype), beta, g [b][h][s]; KDA as GDN with g [b][h][s][dk]. C (GDN: q) enters only its own
 * token's output and is not buffered: its off_ring entry (Mamba-2 [2], GDN [0]) names an empty
 * region.
 * Pointers: int32 [b][h][4] = {start slot, committed count, checkpoint slot, 0}. Flags: one int32
 * word of SSM_FLAG_* bits set by device-side checks. Reader counts: int32 [ckpt_slots], the
 * number of sequences reading each checkpoint slot (kept by the library). */
typedef struct ssm_layout {
    uint64_t total_bytes;
    int32_t ring_cap;       /* slots per ring = L + max_draft - 1 */
    int32_t ckpt_slots;     /* checkpoint slots: batch, or 2 batch with share_ckpt */
    uint64_t off_ckpt;      /* fp32 checkpoint tiles */
    uint64_t off_rc_codes;  /* read-copy codes (0 bytes when readcopy == SSM_RC_NONE) */
    uint64_t off_rc_scale;  /* fp8: row scales fp32; fp4: block-scale codes u8 */
    uint64_t off_rc_tscale; /* fp4: tile scales fp32 */
    uint64_t off_ring[5];   /* Mamba-2: x, B, (empty), dt, (empty); GDN: (empty), k, v, beta, g */
    uint64_t off_ptr;       /* int32 [batch][heads][4] */
    uint64_t off_flags;     /* int32 flag word */
    uint64_t off_refcnt;    /* int32 [ckpt_slots] reader counts */
} ssm_layout;

/* Host handle of one layer's state. Plain data: copyable only while no work is in flight. */
typedef struct ssm_state {
    uint32_t magic;
    int32_t pending;          /* drafts appended by the last ssm_spec_append, not yet resolved */
    int32_t count_lo;         /* bounds on every sequence's committed count (host mirror) */
    int32_t count_hi;
    ssm_config cfg;
    ssm_layout lay;
    void *mem;                /* device memory of lay.total_bytes, owned by the caller */
    const float *A;           /* Mamba-2: device [H] (A < 0), borrowed; NULL for GDN */
    const float *D;           /* Mamba-2: device [H], borrowed; NULL for GDN */
    int32_t ring_start;       /* every sequence's ring start while all sequences sit at one start
                                 and one count (lock-step decoding, checkpoints not shared), else
                                 -1. The replay and fold launches then take start and count as
                                 arguments instead of reading them from the device. */
} ssm_state;

/* Mamba-2 token inputs (device pointers, layouts above). */
typedef struct ssm_m2_in {
    const void *x;
    const void *B;
    const void *C;
    const float *dt;
} ssm_m2_in;

/* Gated DeltaNet and Kimi Delta Attention token inputs (device pointers, layouts above). */
typedef struct ssm_gdn_in {
    const void *q;
    const void *k;
    const void *v;
    const float *beta;
    const float *g;
} ssm_gdn_in;

/* Version of this ABI (SSM_ABI_VERSION). */
int32_t ssm_abi_version(void);

/* Static text for a status code. */
const char *ssm_status_string(ssm_status s);

/* Sizes and offsets of a state for `cfg` (host only, no GPU work). Validates the config. */
ssm_status ssm_layout_query(const ssm_config *cfg, ssm_layout *out);

/* Initialise a state in `mem` (device, mem_bytes >= layout total_bytes): the checkpoint is set to
 * h0 (device fp32 [batch][H][P][N] natural layout, N fastest; NULL = zeros), every ring is empty
 * (start = count = 0) and the read copy, if configured, is written from the checkpoint.
 * A, D: Mamba-2 per-head device fp32 [H], borrowed for the state's lifetime; NULL for GDN.
 * Checkpoint = the state after the prefilled tokens (news, para 2). */
ssm_status ssm_ckpt_init(ssm_state *st, const ssm_config *cfg, void *mem, uint64_t mem_bytes,
                         const float *h0, const float *A, const float *D, void *stream);

/* One decode token for every sequence (news, paras 2-3): append the token's inputs (`in` points
 * to an ssm_m2_in or ssm_gdn_in with ntok = 1) to each ring, compute y [batch][H][P] fp32 from the
 * checkpoint (or its read copy) and the buffered inputs with no state write, and commit the token.
 * When a sequence's committed count reaches L the buffer is folded into the checkpoint (the same
 * work as ssm_flush(SSM_FLUSH_IF_FULL)) before the call returns. In lock step (every sequence at
 * count L - 1) that token is handled by the fold pass itself: its output comes from the new fp32
 * checkpoint, and the read copy, if configured, is rewritten in the same pass.
 * Errors: SSM_E_STATE if drafts are pending; SSM_E_CAPACITY if a ring could overflow. */
ssm_status ssm_replay_decode(ssm_state *st, const void *in, float *y, void *stream);

/* Fold buffered entries into the checkpoint (news, para 3) and rewrite the read copy.
 * SSM_FLUSH_IF_FULL: every sequence whose committed count is >= L folds its oldest L entries
 * (a device-side predicate per sequence). SSM_FLUSH_ALL: fold every committed entry (export).
 * With share_ckpt every fold launch (here, and the ones decode and rollback make) also moves each
 * sequence that shares a checkpoint slot to a slot of its own, folding what it holds (ssm_fork).
 * Errors: SSM_E_STATE if drafts are pending. */
ssm_status ssm_flush(ssm_state *st, int32_t mode, void *stream);

/* Speculative append (news, para 3; explainer, "Usage examples", example 3): write `ndraft`
 * draft tokens (`in` with ntok = ndraft) after each sequence's committed entries, marked pending,
 * and compute all their outputs y [batch][ndraft][H][P] in one pass over the checkpoint. Draft j's
 * output is the output the layer would give after the committed tokens and drafts 1..j.
 * Both layer types (GDN: o [batch][ndraft][H][dv]).
 * Errors: SSM_E_STATE if drafts are already pending; SSM_E_CAPACITY if ndraft > max_draft or the
 * ring could overflow. */
ssm_status ssm_spec_append(ssm_state *st, int32_t ndraft, const void *in, float *y, void *stream);

/* Resolve the pending drafts by moving pointers only (news, para 3): sequence b commits its
 * first n_accept[b] drafts (device int32 [batch], each in [0, pending]; values outside are clamped)
 * and the rest are dropped. No state bytes move for the rollback itself; afterwards every sequence
 * whose committed count reached L folds its oldest L entries (as ssm_flush(SSM_FLUSH_IF_FULL)).
 * Errors: SSM_E_STATE if no drafts are pending. */
ssm_status ssm_spec_rollback(ssm_state *st, const int32_t *n_accept, void *stream);

/* Restore to an earlier position (explainer, "What a Replay-First Design Implies": restore state
 * to position p): sequence b drops its newest min(n_back[b], committed count) entries (device
 * int32 [batch]; negative values count as 0). Positions back to the checkpoint are reached by
 * moving a pointer, since replay rebuilds the output at any of them; earlier positions are not
 * kept. Errors: SSM_E_STATE if drafts are pending. */
ssm_status ssm_restore(ssm_state *st, const int32_t *n_back, void *stream);

/* Fork (explainer, "The State-Storage Bottleneck in Branching Workloads": beam search and
 * best-of-n branch one prefix into several continuations): for k < n, sequence dst[k] continues
 * from sequence src[k]'s position. With share_ckpt the destination gets src's pointers and
 * buffered entries and reads src's checkpoint slot: no checkpoint bytes move. A sequence whose
 * slot is shared, or that reads another's, folds everything it holds into one of its own slots
 * (b or batch + b) at the next fold launch (copy-on-write), whatever its count. Without
 * share_ckpt the checkpoint tiles and read copy are copied too. src and dst are HOST arrays of n
 * sequence indices in [0, batch); destinations must be distinct and none may also be a source in
 * the same call (SSM_E_ARG otherwise). Errors: SSM_E_STATE if drafts are pending. */
ssm_status ssm_fork(ssm_state *st, const int32_t *src, const int32_t *dst, int32_t n,
                    void *stream);

/* Checkpoint of every head in the natural layout, h_out device fp32 [batch][H][P][N]. Only the
 * folded tokens are in it: call ssm_flush(SSM_FLUSH_ALL) first to include the buffered ones. */
ssm_status ssm_ckpt_export(const ssm_state *st, float *h_out, void *stream);

/* Conventional decode step, the comparison point (news, para 3: the full state rewritten every
 * token): h <- exp(dt A) h + dt x B^T, y = h C + D x, read-modify-write of h in place.
 * h: device fp32 [batch][H] tiles in the checkpoint tile layout (see ssm_layout; use
 * ssm_tiles_pack to convert). `in` has ntok = 1. GDN: S <- alpha S + beta (v - alpha S k) k^T,
 * o = scale S q (A, D ignored). */
ssm_status ssm_conventional_step(const ssm_config *cfg, float *h, const void *in, const float *A,
                                 const float *D, float *y, void *stream);

/* Conventional speculative decoding, the comparison point for ssm_spec_append (news, para 3:
 * per-token snapshots; explainer, "Usage examples", example 3: snapshot and restore). Runs the
 * recurrence of ssm_conventional_step over `ndraft` draft tokens (`in` with ntok = ndraft,
 * 1 <= ndraft <= 8, SSM_E_CAPACITY otherwise) starting from h, which is only read, and writes the
 * state after each draft j = 0..ndraft-1 to h_snap [ndraft][batch][H] tiles (tile layout of
 * ssm_layout) and the outputs y [batch][ndraft][H][P] (GDN / KDA: [batch][ndraft][H][dv], `in`
 * an ssm_gdn_in, A and D ignored and may be NULL). All three layer types. h and h_snap must not
 * overlap. */
ssm_status ssm_conventional_spec_snapshot(const ssm_config *cfg, const float *h, float *h_snap,
                                          int32_t ndraft, const void *in, const float *A,
                                          const float *D, float *y, void *stream);

/* The restore half of the snapshot scheme: sequence b takes the state after its n_accept[b]-th
 * draft, h[b] <- h_snap[n_accept[b] - 1][b] (device int32 [batch], clamped to [0, ndraft]; 0
 * keeps h[b]). Moves one state per sequence that accepted a draft. All three layer types. */
ssm_status ssm_conventional_spec_select(const ssm_config *cfg, float *h, const float *h_snap,
                                        int32_t ndraft, const int32_t *n_accept, void *stream);

/* Natural [batch][H][P][N] <-> tile layout conversion of fp32 states (out-of-place). */
ssm_status ssm_tiles_pack(const ssm_config *cfg, const float *natural, float *tiles, void *stream);
ssm_status ssm_tiles_unpack(const ssm_config *cfg, const float *tiles, float *natural,
                            void *stream);

/* Test hook: run the device's OCP codecs over n elements (op 0: fp32 -> E4M3 code, 1: E4M3 code
 * -> fp32, 2: fp32 -> E2M1 code, 3: E2M1 code -> fp32; codes are one per byte; ops 4..7: the same
 * four through the gfx950 conversion instructions; ops 8..11: packed 32-bit words, n = words:
 * 8 E4M3 word -> 4 fp32, 9 E2M1 word -> 8 fp32, 10 4 fp32 -> E4M3 word, 11 8 fp32 -> E2M1 word,
 * element i in byte i / nibble i, low nibble first). n counts work items (values, codes or words
 * as listed); `in` and `out` must hold n items each -- they are not checked. Lets tests check the
 * read-copy codecs bit for bit against the format definitions. */
ssm_status ssm_debug_codec(int32_t op, const void *in, void *out, int64_t n, void *stream);

/* Measurement hook: one pass of plain streaming reads over `bytes` of device memory at src (a
 * multiple of 16; 16-byte aligned) by `blocks` workgroups of 256 threads: each wavefront reads
 * contiguous 32 KiB chunks with 32 16-byte non-temporal loads in flight per lane, the way the
 * decode kernels stream a state tile; the practical read ceiling that the decode kernels' achieved
 * bandwidth is compared with. out: device uint32 [blocks * 4] (one word per wavefront, derived from the data
 * so that no read is dead; its value means nothing). SSM_E_ARG for blocks outside [1, 2^20], a
 * size not a multiple of 16, or a null pointer with bytes > 0. */
ssm_status ssm_debug_stream_read(const void *src, uint64_t bytes, uint32_t *out, int32_t blocks,
                                 void *stream);

/* Test hook: read the state's flag word (SSM_FLAG_* bits) into *host_flags, clearing it on the
 * device when `clear` is non-zero. Synchronizes `stream`. */
ssm_status ssm_debug_flags(const ssm_state *st, int32_t *host_flags, int32_t clear, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_REPLAY_H */
