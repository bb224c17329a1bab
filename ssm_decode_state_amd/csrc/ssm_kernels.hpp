// ssm_kernels.hpp -- kernel argument blocks and launcher entry points (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Pointer entry of one head: {start slot, committed count, checkpoint slot, 0}.
constexpr int kPtrInts = 4;

// Where a fold writes a head's new checkpoint. Without shared checkpoints a sequence reads and
// writes its own slot b. With them (a fork points its copies at the source's slot), sequence b
// owns slots b and batch + b: it folds in place when it reads one of them and no other sequence
// reads it; otherwise it must fold at this launch (copy-on-write) into whichever of its two slots
// nobody reads. At most one of a sequence's slots is read by anyone: every sequence that shares
// a slot moves at the next fold launch, so a slot it left is free again by the one after.
struct FoldTarget {
    int wr;
    bool move;
};
__device__ __forceinline__ FoldTarget fold_target(const int* refcnt, int share, int batch, int b,
                                                  int slot) {
    if (!share) return {slot, false};
    const int own0 = b, own1 = batch + b;
    if ((slot == own0 || slot == own1) && refcnt[slot] == 1) return {slot, false};
    return {refcnt[own0] == 0 ? own0 : own1, true};
}

// Ring pointers of one head. When the host knows them (every sequence at the same start and
// count, checkpoints not shared, so slot == sequence) they come in as kernel arguments and the
// wave starts its loads without a dependent round trip to the pointer entry; hstart < 0 means
// read the entry.
struct HeadPtr {
    int start, count, slot;
};
__device__ __forceinline__ HeadPtr head_ptr(const int* ptr, int hstart, int hcount, long head, int b) {
    if (hstart >= 0) return {hstart, hcount, b};
    const int4 pt = *reinterpret_cast<const int4*>(ptr + kPtrInts * head);
    return {__builtin_amdgcn_readfirstlane(pt.x), __builtin_amdgcn_readfirstlane(pt.y),
            __builtin_amdgcn_readfirstlane(pt.z)};
}

// Everything a Mamba-2 replay / verify / flush launch touches. Device pointers into one state's
// memory (see the layout in ssm_replay.h) plus this call's inputs and outputs.
struct M2Args {
    float* ckpt;        // fp32 checkpoint tiles
    uint8_t* rc_codes;  // read-copy codes
    void* rc_scale;     // fp8: fp32 row scales; fp4: E4M3 block-scale codes
    float* rc_tscale;   // fp4: fp32 tile scales
    void* ring_x;       // buffered inputs: x, B and dt (C enters only its own token's output)
    void* ring_B;
    float* ring_dt;
    int* ptr;           // int32 [batch][heads][4] = {start, count, checkpoint slot, 0}
    const int* refcnt;  // shared checkpoints: readers of each slot [2 batch]
    const void* in_x;   // this call's tokens, [batch][ntok][...]
    const void* in_B;
    const void* in_C;
    const float* in_dt;
    const float* A;
    const float* D;
    float* y;           // [batch][ntok][H][P]
    int batch, heads, groups, cap, ntok, window;
    int share;          // shared checkpoints enabled (slots 0 .. 2 batch - 1)
    int hstart, hcount; // every head's {start, count} when known on the host, else hstart = -1
};

struct M2ConvArgs {
    float* h;  // tiles, updated in place
    const void* in_x;
    const void* in_B;
    const void* in_C;
    const float* in_dt;
    const float* A;
    const float* D;
    float* y;
    int batch, heads, groups;
    float* snap = nullptr;  // speculative snapshots [ntok][batch * heads] tiles (h read only)
    int ntok = 1;
};

// Gated DeltaNet launches.
struct GdnArgs {
    float* ckpt;
    uint8_t* rc_codes;  // read-copy codes (null without a read copy)
    void* rc_scale;     // fp8: fp32 row scales; fp4: E4M3 block-scale codes
    float* rc_tscale;   // fp4: fp32 tile scales
    void* ring_k;       // buffered inputs: k, v, beta and g (q enters only its own token's output)
    void* ring_v;
    float* ring_beta;
    float* ring_g;
    int* ptr;           // as M2Args
    const int* refcnt;
    const void* in_q;
    const void* in_k;
    const void* in_v;
    const float* in_beta;
    const float* in_g;
    float* o;
    float scale;
    int batch, heads, cap, ntok, window;
    int kda;  // Kimi Delta Attention: g holds dk decays per entry (per-channel gate)
    int share;
    int hstart, hcount;  // as M2Args
};

struct GdnConvArgs {
    float* S;
    const void* in_q;
    const void* in_k;
    const void* in_v;
    const float* in_beta;
    const float* in_g;
    float* o;
    float scale;
    int batch, heads;
    int kda;  // per-channel gate (g [batch][H][dk])
    float* snap = nullptr;  // speculative snapshots [ntok][batch * heads] tiles (S read only)
    int ntok = 1;
};

// maxe: upper bound on count + ntok over all sequences (<= 64).
hipError_t m2_launch_replay(const M2Args& a, int P, int N, int bf16, int rc, bool spec, int maxe,
                            hipStream_t s);
// mode_all: 0 = fold L entries where count >= L, 1 = fold every committed entry, 2 = fused
// decode + fold of the L-th lock-step token (inputs and y in `a`, ntok = 1).
hipError_t m2_launch_flush(const M2Args& a, int P, int N, int bf16, int rc, int mode_all,
                           int rewrite_only, hipStream_t s);
hipError_t m2_launch_conv(const M2ConvArgs& a, int P, int N, int bf16, hipStream_t s);
hipError_t m2_launch_snapshot(const M2ConvArgs& a, int P, int N, int bf16, hipStream_t s);

hipError_t gdn_launch_replay(const GdnArgs& a, int dv, int dk, int bf16, int rc, bool spec,
                             int maxe, hipStream_t s);
hipError_t gdn_launch_flush(const GdnArgs& a, int dv, int dk, int bf16, int rc, int mode_all,
                            int rewrite_only, hipStream_t s);
hipError_t gdn_launch_conv(const GdnConvArgs& a, int dv, int dk, int bf16, hipStream_t s);
hipError_t gdn_launch_snapshot(const GdnConvArgs& a, int dv, int dk, int bf16, hipStream_t s);

// Pointer commit after a speculative round: count += min(n_accept[b], pending) for every head.
hipError_t launch_snap_select(float* h, const float* snap, const int32_t* n_accept, int batch,
                              long seq_floats, int ndraft, hipStream_t s);
hipError_t launch_commit(int* ptr, const int32_t* n_accept, int batch, int heads, int pending,
                         int* flags, hipStream_t s);
hipError_t launch_fill_i32(int* p, int value, long n, hipStream_t s);

// Per-sequence slices of a state's regions, for copying whole sequences (fork).
constexpr int kMaxForkRegions = 12, kMaxForkPairs = 64;
struct ForkRegions {
    uint64_t off[kMaxForkRegions];    // region byte offset in the state memory
    uint64_t slice[kMaxForkRegions];  // bytes per sequence (a multiple of 4)
    int n;
};
struct ForkPairs {
    int src[kMaxForkPairs];
    int dst[kMaxForkPairs];
    int n;
};
hipError_t launch_fork_copy(char* mem, const ForkRegions& r, const ForkPairs& p, hipStream_t s);
hipError_t launch_restore(int* ptr, const int32_t* n_back, int batch, int heads, hipStream_t s);
// Natural [heads][P][N] -> quad-interleaved tiles (unpack = 0) or back (unpack = 1). With ptr
// (a state's pointer array, `heads` per sequence) the tiles of head (b, h) are those of its
// checkpoint slot, tile index slot * heads + h; without it tile index = head index.
hipError_t launch_pack(const float* src, float* dst, long nheads, int P, int N, int unpack,
                       const int* ptr, int heads, hipStream_t s);
// Pointer entries {0, 0, b, 0} for every head of sequence b.
hipError_t launch_ptr_init(int* ptr, int batch, int heads, hipStream_t s);
// refcnt[s] = number of sequences whose checkpoint slot is s, for s < nslot.
hipError_t launch_recount(int* refcnt, const int* ptr, int batch, int heads, int nslot,
                          hipStream_t s);
hipError_t launch_codec(int op, const void* in, void* out, long n, hipStream_t s);
// One pass of streaming 16-byte reads over `bytes` (a multiple of 16); out: 4 words per block.
hipError_t launch_stream_read(const void* src, long bytes, uint32_t* out, int blocks, hipStream_t s);

}  // namespace ssm
