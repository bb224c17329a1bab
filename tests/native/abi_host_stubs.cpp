// Host-only stand-ins for the library's kernel launchers, for a sanitizer build of the ABI's host
// half (ssm_api.hip) that runs without a GPU. Each stand-in checks that every device pointer it is
// handed lies, with the extent the real kernel would touch, inside the state memory the driver
// registered (or is one of the driver's input / output addresses), records the call, and returns
// hipSuccess. Nothing is dereferenced: the driver passes fake, unmapped device addresses, so host
// code that touched device memory would fault.
#include <stdio.h>
#include <stdlib.h>

#include "../../ssm_decode_state_amd/csrc/ssm_kernels.hpp"
#include "abi_host_stubs.h"

StubWorld g_world;

static void fail(const char* what, const char* fn) {
    fprintf(stderr, "stub %s: %s\n", fn, what);
    abort();
}

// [p, p + bytes) inside the registered state memory
static void in_state(const void* p, uint64_t bytes, const char* fn, const char* what) {
    const uintptr_t a = (uintptr_t)p, lo = g_world.mem, hi = g_world.mem + g_world.total;
    if (a < lo || a > hi || bytes > hi - a) {
        fprintf(stderr, "stub %s: %s [%#lx, +%llu) outside the state [%#lx, +%llu)\n", fn, what,
                (unsigned long)a, (unsigned long long)bytes, (unsigned long)lo,
                (unsigned long long)g_world.total);
        abort();
    }
}
static void not_null(const void* p, const char* fn, const char* what) {
    if (!p) fail(what, fn);
}

static void check_m2(const ssm::M2Args& a, const char* fn) {
    const uint64_t S = g_world.slots, B = a.batch, H = a.heads, G = a.groups;
    const uint64_t P = g_world.P, N = g_world.N, cap = a.cap, esz = g_world.esz;
    in_state(a.ckpt, S * H * P * N * 4, fn, "checkpoint");
    in_state(a.ring_x, B * H * cap * P * esz, fn, "x ring");
    in_state(a.ring_B, B * G * cap * N * esz, fn, "B ring");
    in_state(a.ring_dt, B * H * cap * 4, fn, "dt ring");
    in_state(a.ptr, B * H * 16, fn, "pointers");
    if (a.share) in_state(a.refcnt, S * 4, fn, "reader counts");
    if (g_world.rc == 1) {
        in_state(a.rc_codes, S * H * P * N, fn, "fp8 codes");
        in_state(a.rc_scale, S * H * P * 4, fn, "fp8 scales");
    } else if (g_world.rc == 2) {
        in_state(a.rc_codes, S * H * P * N / 2, fn, "fp4 codes");
        in_state(a.rc_scale, S * H * P * (N / 16), fn, "fp4 block scales");
        in_state(a.rc_tscale, S * H * 4, fn, "fp4 tile scales");
    }
    if (a.window < 1 || a.cap < a.window) fail("window / capacity", fn);
    if (a.hstart >= a.cap || a.hcount > a.cap) fail("host-known pointers out of range", fn);
}

static void check_gdn(const ssm::GdnArgs& a, const char* fn) {
    const uint64_t S = g_world.slots, B = a.batch, H = a.heads;
    const uint64_t dv = g_world.P, dk = g_world.N, cap = a.cap, esz = g_world.esz;
    in_state(a.ckpt, S * H * dv * dk * 4, fn, "checkpoint");
    in_state(a.ring_k, B * H * cap * dk * esz, fn, "k ring");
    in_state(a.ring_v, B * H * cap * dv * esz, fn, "v ring");
    in_state(a.ring_beta, B * H * cap * 4, fn, "beta ring");
    in_state(a.ring_g, B * H * cap * (a.kda ? dk : 1) * 4, fn, "g ring");
    in_state(a.ptr, B * H * 16, fn, "pointers");
    if (a.share) in_state(a.refcnt, S * 4, fn, "reader counts");
    if (g_world.rc == 2) in_state(a.rc_tscale, S * H * 4, fn, "fp4 tile scales");
    if (g_world.rc != 0) in_state(a.rc_codes, S * H * dv * dk / (g_world.rc == 2 ? 2 : 1), fn, "codes");
    if (a.hstart >= a.cap || a.hcount > a.cap) fail("host-known pointers out of range", fn);
}

namespace ssm {

hipError_t m2_launch_replay(const M2Args& a, int, int, int, int, bool spec, int maxe, hipStream_t) {
    check_m2(a, "m2_launch_replay");
    if (maxe < a.ntok || maxe > a.cap || a.ntok < 1) fail("entries per call", "m2_launch_replay");
    not_null(a.in_x, "m2_launch_replay", "inputs");
    not_null(a.y, "m2_launch_replay", "outputs");
    g_world.calls[spec ? kVerify : kReplay]++;
    return hipSuccess;
}
hipError_t m2_launch_flush(const M2Args& a, int, int, int, int, int mode_all, int rewrite_only,
                           hipStream_t) {
    check_m2(a, "m2_launch_flush");
    g_world.calls[rewrite_only ? kRewrite : (mode_all == 2 ? kFused : kFold)]++;
    return hipSuccess;
}
hipError_t m2_launch_conv(const M2ConvArgs& a, int, int, int, hipStream_t) {
    not_null(a.h, "m2_launch_conv", "state");
    g_world.calls[kConv]++;
    return hipSuccess;
}
hipError_t m2_launch_snapshot(const M2ConvArgs& a, int, int, int, hipStream_t) {
    if (a.ntok < 1 || a.ntok > 8 || !a.snap) fail("snapshot arguments", "m2_launch_snapshot");
    g_world.calls[kSnap]++;
    return hipSuccess;
}
hipError_t gdn_launch_replay(const GdnArgs& a, int, int, int, int, bool spec, int maxe, hipStream_t) {
    check_gdn(a, "gdn_launch_replay");
    if (maxe < a.ntok || maxe > 32) fail("entries per call", "gdn_launch_replay");
    g_world.calls[spec ? kVerify : kReplay]++;
    return hipSuccess;
}
hipError_t gdn_launch_flush(const GdnArgs& a, int, int, int, int, int mode_all, int rewrite_only,
                            hipStream_t) {
    check_gdn(a, "gdn_launch_flush");
    g_world.calls[rewrite_only ? kRewrite : (mode_all == 2 ? kFused : kFold)]++;
    return hipSuccess;
}
hipError_t gdn_launch_conv(const GdnConvArgs& a, int, int, int, hipStream_t) {
    not_null(a.S, "gdn_launch_conv", "state");
    g_world.calls[kConv]++;
    return hipSuccess;
}
hipError_t gdn_launch_snapshot(const GdnConvArgs& a, int, int, int, hipStream_t) {
    if (a.ntok < 1 || a.ntok > 8 || !a.snap) fail("snapshot arguments", "gdn_launch_snapshot");
    g_world.calls[kSnap]++;
    return hipSuccess;
}
hipError_t launch_snap_select(float* h, const float* snap, const int32_t* n_accept, int batch,
                              long seq_floats, int ndraft, hipStream_t) {
    if (batch == 0 || seq_floats == 0) return hipSuccess;  // (the real launcher: nothing to do)
    if (!h || !snap || !n_accept || batch < 0 || seq_floats < 0 || ndraft < 1)
        fail("select arguments", "launch_snap_select");
    return hipSuccess;
}
hipError_t launch_commit(int* ptr, const int32_t* n_accept, int batch, int heads, int pending,
                         int* flags, hipStream_t) {
    in_state(ptr, (uint64_t)batch * heads * 16, "launch_commit", "pointers");
    in_state(flags, 4, "launch_commit", "flags");
    if (!n_accept || pending < 1) fail("commit arguments", "launch_commit");
    g_world.calls[kCommit]++;
    return hipSuccess;
}
hipError_t launch_fill_i32(int* p, int, long n, hipStream_t) {
    in_state(p, (uint64_t)n * 4, "launch_fill_i32", "filled words");
    return hipSuccess;
}
hipError_t launch_fork_copy(char* mem, const ForkRegions& r, const ForkPairs& p, hipStream_t) {
    if ((uintptr_t)mem != g_world.mem) fail("state base", "launch_fork_copy");
    if (r.n < 1 || r.n > kMaxForkRegions || p.n < 1 || p.n > kMaxForkPairs)
        fail("region / pair counts", "launch_fork_copy");
    for (int g = 0; g < r.n; ++g) {
        if (r.slice[g] % 4) fail("slice not a multiple of 4", "launch_fork_copy");
        for (int k = 0; k < p.n; ++k) {
            if (p.src[k] < 0 || p.src[k] >= g_world.batch || p.dst[k] < 0 || p.dst[k] >= g_world.batch)
                fail("sequence index", "launch_fork_copy");
            in_state(mem + r.off[g] + (uint64_t)p.src[k] * r.slice[g], r.slice[g], "launch_fork_copy", "source slice");
            in_state(mem + r.off[g] + (uint64_t)p.dst[k] * r.slice[g], r.slice[g], "launch_fork_copy", "destination slice");
        }
    }
    g_world.calls[kFork]++;
    return hipSuccess;
}
hipError_t launch_restore(int* ptr, const int32_t* n_back, int batch, int heads, hipStream_t) {
    in_state(ptr, (uint64_t)batch * heads * 16, "launch_restore", "pointers");
    if (!n_back) fail("n_back", "launch_restore");
    return hipSuccess;
}
hipError_t launch_pack(const float* src, float* dst, long nheads, int P, int N, int, const int* ptr,
                       int heads, hipStream_t) {
    if (nheads == 0) return hipSuccess;  // (the real launcher: nothing to do)
    if (!src || !dst || nheads < 0 || P < 1 || N < 1) fail("pack arguments", "launch_pack");
    if (ptr) in_state(ptr, (uint64_t)nheads * 16, "launch_pack", "pointers");
    (void)heads;
    return hipSuccess;
}
hipError_t launch_ptr_init(int* ptr, int batch, int heads, hipStream_t) {
    in_state(ptr, (uint64_t)batch * heads * 16, "launch_ptr_init", "pointers");
    return hipSuccess;
}
hipError_t launch_recount(int* refcnt, const int* ptr, int batch, int heads, int nslot, hipStream_t) {
    in_state(refcnt, (uint64_t)nslot * 4, "launch_recount", "reader counts");
    in_state(ptr, (uint64_t)batch * heads * 16, "launch_recount", "pointers");
    return hipSuccess;
}
hipError_t launch_codec(int, const void*, void*, long, hipStream_t) { return hipSuccess; }
hipError_t launch_stream_read(const void*, long, uint32_t*, int, hipStream_t) { return hipSuccess; }

}  // namespace ssm
