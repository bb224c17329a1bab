#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--skip-conv] [--copy-ref MB]

Workload (the headline): a Mamba-2 SSM layer decoding at serving batch -- B = 256 sequences,
H = 128 heads, head dim P = 64, state dim N = 128 (fp32 checkpoint, 4 MiB per sequence), window
L = 16, bf16 x/B/C and fp32 dt. One step = one decode token for every sequence through the whole
replay path: append to the ring, replay output from the checkpoint, and (every L-th step) the
flush that folds the window into the checkpoint. After W warm-up steps, the K steps run launched
back to back from Python behind a GPU pre-roll (about 2 ms of unrelated streaming reads, so the
host's launches get ahead of the GPU), synchronized before and after; `value` is B * K over the
GPU time from the first step's start to the last step's end, bracketed by HIP events, for the
median of three such passes in a row, and HIP events between runs of one kernel (a window's
replays, the fold) give the per-kernel figures over all three passes. The
same K steps then run once more with an event pair around each launch (per-count figures) and
as one HIP graph (reported beside the headline). The window-amortized step ((L - 1) replays +
the fused fold) / L is reported too, so a K that is not a multiple of L neither flatters nor
penalizes the fold's share.

Reported: tokens/s per layer, the in-house conventional read-modify-write step on the same shapes
and inputs (timed the same way), the replay kernel's achieved HBM bandwidth from those HIP events
against the algorithmic bytes (also against a streaming-read ceiling measured at the same bytes
per launch), and the
fp64 CPU oracle timed on a bounded sample of the same workload on this host.

Inputs are seeded synthetic draws made on the device (ssm_decode_state_amd.synth) and resident in
HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
REPS = 3  # timed passes of the K headline steps; the median is reported


# Sources the one-token replay kernel is compiled from; the counter profile records their hash.
DECODE_SOURCES = ("m2_kernels.hpp", "m2_decode.hip", "ssm_device.hpp", "ssm_kernels.hpp")


def sources_sha(files=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "ssm_decode_state_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic():
    """HBM bytes per launch of the replay kernel from the committed counter profile
    (profiles/hbm_traffic_pmc_b256.md), or None when the kernel sources changed since."""
    prof = os.path.join(ROOT, "profiles", "hbm_traffic_pmc_b256.md")
    try:
        line = [l for l in open(prof) if l.startswith("traffic-json:")][0]
        rec = json.loads(line.split(":", 1)[1])
        sha = sources_sha()
    except (OSError, IndexError, ValueError):
        return None
    return rec["bytes_per_launch"] if rec.get("sha") == sha else None


def m2_replay_bytes_per_head(P, N, k, esz=2):
    """Algorithmic bytes of one replay launch for one head at committed count k (after append):
    checkpoint read + the k-1 older ring entries read (x, B, dt) + the token's inputs read (x, B,
    C, dt) + its x, B and dt appended + y written + the count written (lock-step launches take
    start and count from the host; a launch that reads the pointer entry adds 16 bytes)."""
    entry = P * esz + N * esz + 4
    token = P * esz + 2 * N * esz + 4
    return P * N * 4 + (k - 1) * entry + token + entry + P * 4 + 4


def m2_flush_bytes_per_head(P, N, L, esz=2):
    """Checkpoint read + write and the L folded entries read (x, B, dt) + pointers."""
    return 2 * P * N * 4 + L * (P * esz + N * esz + 4) + 16


def rc_copy_bytes_per_head(rows, cols, rc):
    """One head's read copy: fp8 codes and an fp32 scale per row, or fp4 codes, an E4M3 scale per
    16 elements and the fp32 tile scale."""
    if rc == 0:
        return 0
    return rows * cols + rows * 4 if rc == 1 else rows * cols // 2 + rows * cols // 16 + 4


def m2_fused_step_bytes_per_head(P, N, L, rc=0, esz=2):
    """The window-closing step (one fused pass): checkpoint read + written, the L-1 buffered
    entries (x, B, dt), the token read (x, B, C, dt), y, the pointer entry; with a read copy, the
    copy rewritten."""
    entry = P * esz + N * esz + 4
    token = P * esz + 2 * N * esz + 4
    return 2 * P * N * 4 + (L - 1) * entry + token + P * 4 + 16 + rc_copy_bytes_per_head(P, N, rc)


def m2_conv_bytes_per_head(P, N, esz=2):
    """State read + write, the token's inputs read, y written."""
    return 2 * P * N * 4 + P * esz + 2 * N * esz + 4 + P * 4


def m2_verify_bytes_per_head(P, N, kc, S, esz=2):
    """One speculative verify launch for one head: checkpoint read once, kc committed entries
    (x, B, dt), S drafts read (x, B, C, dt) and appended (x, B, dt), S outputs, pointers."""
    entry = P * esz + N * esz + 4
    token = P * esz + 2 * N * esz + 4
    return P * N * 4 + kc * entry + S * (token + entry) + S * P * 4 + 8


def m2_snapshot_bytes_per_head(P, N, S, esz=2):
    """Snapshot-based speculation for one head: state read once, S snapshot states written, the
    S drafts' inputs read, S outputs written."""
    return P * N * 4 + S * P * N * 4 + S * (P * esz + 2 * N * esz + 4) + S * P * 4


def m2_rc_replay_bytes_per_head(P, N, k, rc, esz=2):
    """Replay launch reading the low-precision copy instead of the fp32 checkpoint."""
    return m2_replay_bytes_per_head(P, N, k, esz) - P * N * 4 + rc_copy_bytes_per_head(P, N, rc)


def gdn_replay_bytes_per_head(dv, dk, k, esz=2, gsz=4):
    """GDN replay for one head at count k: state read + k-1 older entries (k, v, beta, g) + this
    token read (q, k, v, beta, g) and appended (k, v, beta, g) + o written + the count written
    (as for Mamba-2). gsz: bytes of g per entry (4; Kimi Delta Attention: 4 dk)."""
    entry = dk * esz + dv * esz + 4 + gsz
    token = 2 * dk * esz + dv * esz + 4 + gsz
    return dv * dk * 4 + (k - 1) * entry + token + entry + dv * 4 + 4


def gdn_verify_bytes_per_head(dv, dk, kc, S, esz=2, gsz=4):
    """GDN (KDA: gsz = 4 dk) speculative verify for one head: state read once, kc committed
    entries (k, v, beta, g), S drafts read (q, k, v, beta, g) and appended (k, v, beta, g), S
    outputs, pointers."""
    entry = dk * esz + dv * esz + 4 + gsz
    token = 2 * dk * esz + dv * esz + 4 + gsz
    return dv * dk * 4 + kc * entry + S * (token + entry) + S * dv * 4 + 8


def gdn_snapshot_bytes_per_head(dv, dk, S, esz=2, gsz=4):
    """Snapshot-based GDN / KDA speculation: read the state once, write it after each of S drafts,
    read the drafts' inputs, write their outputs."""
    return 4 * dv * dk * (1 + S) + S * (2 * dk * esz + dv * esz + 4 + gsz) + 4 * S * dv


def gdn_fused_step_bytes_per_head(dv, dk, L, rc=0, esz=2, gsz=4):
    """GDN / KDA window-closing step: state read + written, the L-1 buffered entries (k, v, beta,
    g), the token read (q, k, v, beta, g), o, the pointer entry; with a read copy, the copy
    rewritten."""
    entry = dk * esz + dv * esz + 4 + gsz
    token = 2 * dk * esz + dv * esz + 4 + gsz
    return 2 * dv * dk * 4 + (L - 1) * entry + token + dv * 4 + 16 + rc_copy_bytes_per_head(dv, dk, rc)


def fold_step_rate(nbytes, ms_list):
    """Achieved GB/s and fraction of the HBM peak of the timed window-closing steps (nbytes each)."""
    if not ms_list:
        return {}
    gbs = nbytes / (sum(ms_list) / len(ms_list) * 1e-3) / 1e9
    return {"fold_step_achieved_gbs": gbs, "fold_step_frac": gbs / HBM_PEAK_GBS}


def gdn_conv_bytes_per_head(dv, dk, esz=2, gsz=4):
    return 2 * dv * dk * 4 + 2 * dk * esz + dv * esz + 4 + gsz + dv * 4


_PREROLL = {}


def gpu_preroll(launches=12):
    """Queue about 2 ms of unrelated streaming reads on the current stream, so that the host's
    launches that follow get ahead of the GPU: then each HIP-event pair around a launch brackets
    the kernel alone, not the gap while the GPU waited for the host to submit it."""
    import torch
    from ssm_decode_state_amd import binding as bd
    if "buf" not in _PREROLL:
        _PREROLL["buf"] = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        _PREROLL["out"] = torch.empty(4 * 2048, dtype=torch.int32, device="cuda")
    for _ in range(launches):
        bd.ssm_debug_stream_read(_PREROLL["buf"], _PREROLL["out"], 2048)


def timed_calls(n, fn, kind=None):
    """Run fn(i) for i < n on the current stream behind a GPU pre-roll (see gpu_preroll).
    Without `kind`, a HIP-event pair brackets each call. With kind(i), a label per call (say
    replay or fold), events mark only the boundaries between runs of calls of one kind and each
    call of a run is charged the run's span over its length: the launches of a run go back to
    back with no event between them, as a serving loop issues them, and no per-launch event
    overhead lands on short kernels. Returns (seconds of GPU time from the first call's start to
    the last call's end, per-call milliseconds)."""
    import torch
    torch.cuda.synchronize()
    if kind is None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        gpu_preroll()
        for i in range(n):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return ev[0][0].elapsed_time(ev[-1][1]) * 1e-3, [a.elapsed_time(b) for a, b in ev]
    starts = [0] + [i for i in range(1, n) if kind(i) != kind(i - 1)]
    ends = starts[1:] + [n]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(starts) + 1)]
    gpu_preroll()
    r = 0
    for i in range(n):
        if r < len(starts) and i == starts[r]:
            ev[r].record()
            r += 1
        fn(i)
    ev[-1].record()
    torch.cuda.synchronize()
    ms = []
    for j, (a, b) in enumerate(zip(starts, ends)):
        ms += [ev[j].elapsed_time(ev[j + 1]) / (b - a)] * (b - a)
    return ev[0].elapsed_time(ev[-1]) * 1e-3, ms


CEILING_SIZES_MIB = (64, 128, 256, 512, 1024)


def bench_read_ceiling(dev, sizes_mib=CEILING_SIZES_MIB, launches=12, pool_bytes=2 << 30):
    """The practical read ceiling against bytes per launch: one pass of plain streaming reads
    (16-byte non-temporal loads, ssm_debug_stream_read) over S bytes for S from 64 MiB to 1 GiB,
    each launch on the next S-byte slice of a 2 GiB pool (eight times the last-level cache), so
    that every launch reads HBM. Timed like the decode kernels' per-launch figures: launches back
    to back behind a GPU pre-roll, their span over their number. Per size, the better of two grid
    shapes (one
    or four 32 KiB chunks per wavefront). A short launch pays the grid's ramp-up and drain, so a
    kernel is compared with this curve at its own bytes per launch (ceiling_at)."""
    import torch
    from ssm_decode_state_amd import binding as bd
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    out = torch.empty(4 * (pool_bytes >> 15), dtype=torch.int32, device=dev)
    by_size = {}
    for mib in sizes_mib:
        nb = mib << 20
        nsl = pool_bytes // nb
        chunks = nb >> 15
        best = None
        for per_wave in (1, 4):
            blocks = max(1, chunks // (4 * per_wave))

            def fn(i, nb=nb, nsl=nsl, blocks=blocks):
                j = (i + 2) % nsl  # slices 0 and 1 take the untimed first launches
                bd.ssm_debug_stream_read(pool[j * nb:(j + 1) * nb], out, blocks)

            for i in (-2, -1):
                fn(i)
            _, ms = timed_calls(launches, fn, kind=lambda i: 0)  # back to back, like the workloads
            us = sum(ms) / len(ms) * 1e3
            r = {"avg_us": us, "gbs": nb / (us * 1e-6) / 1e9, "workgroups": blocks}
            if best is None or r["gbs"] > best["gbs"]:
                best = r
        by_size[str(nb)] = best
    del pool, out
    top = by_size[str(max(sizes_mib) << 20)]
    return {"kernel": "stream_read_kernel", "by_bytes": by_size,
            "best_gbs": top["gbs"], "best_frac_of_peak": top["gbs"] / HBM_PEAK_GBS,
            "note": "best_gbs: one pass over 1 GiB; by_bytes: the curve ceiling_at interpolates"}


def ceiling_at(rc, nbytes):
    """The read ceiling (GB/s) at nbytes per launch: log-linear between the measured sizes, the
    smallest size's figure below them and the largest's above."""
    import math
    pts = sorted((int(b), r["gbs"]) for b, r in rc["by_bytes"].items())
    if nbytes <= pts[0][0]:
        return pts[0][1]
    for (b0, g0), (b1, g1) in zip(pts, pts[1:]):
        if nbytes <= b1:
            t = (math.log2(nbytes) - math.log2(b0)) / (math.log2(b1) - math.log2(b0))
            return g0 + t * (g1 - g0)
    return pts[-1][1]


def annotate_ceiling(node, rc):
    """Add `<x>frac_of_read_ceiling` beside every `<x>achieved_gbs` that has a per-launch time
    (`<x>avg_us` or `<x>avg_launch_us`): achieved rate over the read ceiling at the launch's own
    bytes (achieved rate x time)."""
    if isinstance(node, list):
        for v in node:
            annotate_ceiling(v, rc)
        return
    if not isinstance(node, dict):
        return
    for key in list(node):
        v = node[key]
        if isinstance(v, (dict, list)):
            annotate_ceiling(v, rc)
        elif key.endswith("achieved_gbs") and isinstance(v, float):
            pre = key[:-len("achieved_gbs")]
            us = node.get(pre + "avg_us", node.get(pre + "avg_launch_us"))
            if isinstance(us, float) and us > 0:
                node[pre + "frac_of_read_ceiling"] = v / ceiling_at(rc, v * 1e9 * us * 1e-6)


def bench_spec(dev, rounds=64, warm=16, pool=16):
    """Speculative decoding on the serving shapes: each round appends 4 drafts per sequence and
    verifies them in one replay call, then accepts U{0..4} per sequence and rolls back by moving
    pointers (a fold fires whenever a sequence reaches L)."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["m2_b256_spec"]
    shape = w["shape"]
    Bn, H, P, N, L, S = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window, w["ndraft"]
    A, D = synth.head_constants(shape, w["seed"])
    h0 = synth.initial_state_device(shape, w["seed"], w["h0_std"])
    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, shape.groups, P, N, L, S, bd.SSM_IN_BF16)
    st = bd.State(cfg, h0, A.to(dev), D.to(dev))
    del h0
    drafts = [synth.token_inputs_device(shape, w["seed"], "bench-draft", i, ntok=S)
              for i in range(pool)]
    accs = [synth.accept_counts(Bn, S, w["accept_seed"], r) for r in range(warm + rounds)]
    accs_d = [a.to(dev) for a in accs]
    y = torch.empty(Bn, S, H, P, device=dev)
    counts = [0] * Bn  # host model of the committed counts, for the byte accounting

    def advance(r):
        for b in range(Bn):
            counts[b] += int(accs[r][b])
            if counts[b] >= L:
                counts[b] -= L

    for r in range(warm):
        bd.ssm_spec_append(st, S, drafts[r % pool], y)
        bd.ssm_spec_rollback(st, accs_d[r])
        advance(r)
    ver_bytes = 0.0
    for r in range(warm, warm + rounds):
        ver_bytes += H * sum(m2_verify_bytes_per_head(P, N, c, S) for c in counts)
        advance(r)
    # events are created up front: creating them inside the timed loop makes it host-bound
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(rounds)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(rounds):
        r = warm + i
        ev[i][0].record()
        bd.ssm_spec_append(st, S, drafts[r % pool], y)
        ev[i][1].record()
        bd.ssm_spec_rollback(st, accs_d[r])
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ver = sum(e[0].elapsed_time(e[1]) for e in ev)
    rb = sum(e[1].elapsed_time(e[2]) for e in ev)
    accepted = sum(int(accs[r].sum()) for r in range(warm, warm + rounds))
    gbs = ver_bytes / (ver * 1e-3) / 1e9
    del st
    # the comparison point: conventional speculation writes the state after every draft and
    # restores the accepted one
    Ad, Dd = A.to(dev), D.to(dev)
    h = torch.empty(Bn * H * P * N, device=dev)
    h0 = synth.initial_state_device(shape, w["seed"], w["h0_std"])
    bd.ssm_tiles_pack(cfg, h0, h)
    del h0
    snap = torch.empty(S, Bn * H * P * N, device=dev)
    for r in range(warm):
        bd.ssm_conventional_spec_snapshot(cfg, h, snap, S, drafts[r % pool], Ad, Dd, y)
        bd.ssm_conventional_spec_select(cfg, h, snap, S, accs_d[r])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(rounds):
        r = warm + i
        ev[i][0].record()
        bd.ssm_conventional_spec_snapshot(cfg, h, snap, S, drafts[r % pool], Ad, Dd, y)
        ev[i][1].record()
        bd.ssm_conventional_spec_select(cfg, h, snap, S, accs_d[r])
        ev[i][2].record()
    torch.cuda.synchronize()
    swall = time.perf_counter() - t0
    sn = sum(e[0].elapsed_time(e[1]) for e in ev)
    sel = sum(e[1].elapsed_time(e[2]) for e in ev)
    sgbs = Bn * H * m2_snapshot_bytes_per_head(P, N, S) * rounds / (sn * 1e-3) / 1e9
    del snap, h
    return {"workload": "mamba2_spec_b256_4drafts", "accepted_tokens_per_s": accepted / wall,
            "unit": "accepted tokens/s/layer", "rounds": rounds, "mean_accept": accepted / (Bn * rounds),
            "verify_avg_us": ver / rounds * 1e3, "verify_achieved_gbs": gbs,
            "verify_frac": gbs / HBM_PEAK_GBS,
            "rollback_and_fold_avg_us": rb / rounds * 1e3, "ms_per_round": wall / rounds * 1e3,
            "conventional_snapshot": {
                "accepted_tokens_per_s": accepted / swall, "ms_per_round": swall / rounds * 1e3,
                "snapshot_avg_us": sn / rounds * 1e3, "snapshot_achieved_gbs": sgbs,
                "snapshot_frac": sgbs / HBM_PEAK_GBS, "select_avg_us": sel / rounds * 1e3},
            "speedup_vs_snapshot": swall / wall}


def bench_m2_decode(dev, shape, seed, h0_std, steps, warm, pool=16):
    """Lock-step replay decode of one Mamba-2 layer: tokens/s, mean step and the window-closing
    (fused fold) step."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    Bn, H, P, N, L = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state_device(shape, seed, h0_std)
    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, shape.groups, P, N, L, 1, bd.SSM_IN_BF16)
    st = bd.State(cfg, h0, A.to(dev), D.to(dev))
    del h0
    inputs = [synth.token_inputs_device(shape, seed, "bench-sweep", i) for i in range(pool)]
    y = torch.empty(Bn, H, P, device=dev)
    for i in range(warm):
        bd.ssm_replay_decode(st, inputs[i % pool], y)
    wall, ms = timed_calls(steps, lambda i: bd.ssm_replay_decode(st, inputs[(warm + i) % pool], y),
                           kind=lambda i: (warm + i) % L == L - 1)
    fold = [m for i, m in enumerate(ms) if (warm + i) % L == L - 1]
    rep = [m for i, m in enumerate(ms) if (warm + i) % L != L - 1]
    rep_b = sum(Bn * H * m2_replay_bytes_per_head(P, N, (warm + i) % L + 1, 2)
                for i in range(steps) if (warm + i) % L != L - 1)
    return {"window": L, "groups": shape.groups, "tokens_per_s": Bn * steps / wall,
            "mean_step_us": sum(ms) / steps * 1e3,
            "replay_avg_us": sum(rep) / max(len(rep), 1) * 1e3,
            "replay_frac": (rep_b / (sum(rep) * 1e-3) / 1e9 / HBM_PEAK_GBS) if rep else None,
            "fold_step_avg_us": sum(fold) / max(len(fold), 1) * 1e3}


def bench_lsweep(dev, steps=96, warm=32):
    """Window sweep on the serving shapes (L = 4, 8, 16, 32; the window-closing step fuses the
    fold): the checkpoint read and rewrite per window trade against the buffered entries."""
    import dataclasses
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["m2_b256"]
    out = []
    for L in (4, 8, 16, 32):
        shape = dataclasses.replace(w["shape"], window=L)
        out.append(bench_m2_decode(dev, shape, w["seed"], w["h0_std"], steps, warm))
    return out


def bench_bsweep(dev, batches=(1, 4, 16, 64, 256), min_bytes=512 << 20, max_layers=256, reps=4):
    """Per-token latency against batch size: the time of one decode step of one layer, replay
    against the conventional step, on the Mamba-2 and GDN serving head shapes (L = 16). Each point
    cycles through enough layer instances that their states (at least min_bytes, twice the 256 MB
    last-level cache) are read from HBM, as the layers of a model are between their visits. One
    HIP graph holds a window's steps, every layer in turn, for each path."""
    import dataclasses
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    out = []
    for kind, wname in ((bd.SSM_MAMBA2, "m2_b256"), (bd.SSM_GDN, "gdn_b256")):
        w = synth.WORKLOADS[wname]
        for Bn in batches:
            shape = dataclasses.replace(w["shape"], batch=Bn)
            H, G, P, N, L = shape.heads, shape.groups, shape.dim_p, shape.dim_n, shape.window
            state = Bn * H * P * N * 4
            layers = min(max_layers, max(2, -(-min_bytes // state)))
            if kind == bd.SSM_MAMBA2:
                A, D = synth.head_constants(shape, w["seed"])
                A, D = A.to(dev), D.to(dev)
            else:
                A = D = None
            cfg = bd.make_config(kind, Bn, H, G, P, N, L, 1, bd.SSM_IN_BF16)
            inputs = [synth.token_inputs_device(shape, w["seed"], "bsweep", t) for t in range(L)]
            y = torch.empty(Bn, H, P, device=dev)
            res = {"layer": "mamba2" if kind == bd.SSM_MAMBA2 else "gdn", "batch": Bn,
                   "layers_rotated": layers}
            for path in ("replay", "conventional"):
                if path == "replay":
                    objs = [bd.State(cfg, None, A, D) for _ in range(layers)]
                    step = lambda o, t: bd.ssm_replay_decode(o, inputs[t], y)  # noqa: E731
                else:
                    objs = [torch.zeros(Bn * H * P * N, device=dev) for _ in range(layers)]
                    step = lambda o, t: bd.ssm_conventional_step(cfg, o, inputs[t], A, D, y)  # noqa: E731
                for t in range(L):  # one eager window: every state back at a window boundary
                    for o in objs:
                        step(o, t)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for t in range(L):
                        for o in objs:
                            step(o, t)
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                res[path + "_us_per_step"] = e0.elapsed_time(e1) * 1e3 / (reps * L * layers)
                del g, objs
                torch.cuda.empty_cache()
            res["replay_tokens_per_s"] = Bn / (res["replay_us_per_step"] * 1e-6)
            res["speedup_vs_conventional"] = res["conventional_us_per_step"] / res["replay_us_per_step"]
            out.append(res)
    return out


def graph_steps(step, K, mem):
    """Time exactly K steps as one HIP graph: step(i) for i < K is captured from the current
    state, replayed once untimed (warm-up), the state bytes `mem` (a tensor holding all device
    state the steps touch) are restored to the captured start, and the graph is replayed once
    more inside the timed region. The timed region starts after a device synchronization and a
    GPU pre-roll (gpu_preroll, queued after the synchronization): HIP events on the stream bracket
    exactly the graph's K steps, and the GPU is already at its working clock when they start, as
    in a serving loop, so a short K is not charged the ramp out of idle; the host wall time from
    the graph launch to the closing synchronization is reported beside it. The same mechanism for
    every K, so a K that is not a multiple of the window neither drops the graph nor changes how
    the steps are launched. Returns None if the capture fails (the eager figures stand)."""
    import torch
    saved = mem.clone()
    g = torch.cuda.CUDAGraph()
    try:
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(K):
                step(i)
    except Exception as e:  # capture unsupported here: keep the eager figures
        print("graph capture failed: %s" % e, file=sys.stderr)
        return None
    g.replay()  # warm-up: the first replay uploads the graph
    torch.cuda.synchronize()
    mem.copy_(saved)
    del saved
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_preroll()
    e0.record()
    t0 = time.perf_counter()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu = e0.elapsed_time(e1) * 1e-3
    del g
    return {"gpu_s": gpu, "ms_per_step": gpu / K * 1e3, "host_wall_s": wall}


def seq_state_bytes(cfg, lay):
    """Bytes a fork copies per sequence: pointers and buffered entries, plus the checkpoint tiles
    and read copy unless checkpoints are shared."""
    H, G, P, N, cap = cfg.heads, cfg.groups, cfg.dim_p, cfg.dim_n, lay.ring_cap
    e = 2 if cfg.in_dtype == 1 else 4
    n = H * 16
    if not cfg.share_ckpt:
        n += H * P * N * 4
        if cfg.readcopy == 1:
            n += H * P * N + H * P * 4
        elif cfg.readcopy == 2:
            n += H * P * N // 2 + H * P * (N // 16) + H * 4
    if cfg.kind == 0:  # rings x, B, dt
        n += H * cap * P * e + G * cap * N * e + H * cap * 4
    else:  # rings k, v, beta, g
        n += H * cap * N * e + H * cap * P * e + H * cap * 4
        n += H * cap * (N if cfg.kind == 2 else 1) * 4
    return n


def bench_branch(dev, reps=20, pairs=64, share=0):
    """Branching on the serving state: a fork of `pairs` sequences (share = 0: every region
    copied in one launch; share = 1: pointers and buffered entries copied, the checkpoint shared,
    plus the slot reader recount) and a restore of every sequence (pointer move)."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["m2_b256"]
    shape = w["shape"]
    Bn, H, P, N = shape.batch, shape.heads, shape.dim_p, shape.dim_n
    A, D = synth.head_constants(shape, w["seed"])
    h0 = synth.initial_state_device(shape, w["seed"], w["h0_std"])
    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, shape.groups, P, N, shape.window, 1, bd.SSM_IN_BF16,
                         share_ckpt=share)
    st = bd.State(cfg, h0, A.to(dev), D.to(dev))
    del h0
    y = torch.empty(Bn, H, P, device=dev)
    for i in range(21):  # a fold, then five buffered entries
        bd.ssm_replay_decode(st, synth.token_inputs_device(shape, w["seed"], "bench-branch", i), y)
    src = list(range(0, 2 * pairs, 2))
    dst = [s + 1 for s in src]
    bd.ssm_fork(st, src, dst)
    _, ms = timed_calls(reps, lambda i: bd.ssm_fork(st, src, dst))
    fork_us = sum(ms) / reps * 1e3
    per_seq = seq_state_bytes(cfg, st.layout)
    gbs = pairs * per_seq * 2 / (fork_us * 1e-6) / 1e9
    zero = torch.zeros(Bn, dtype=torch.int32, device=dev)
    bd.ssm_restore(st, zero)
    _, ms = timed_calls(reps, lambda i: bd.ssm_restore(st, zero))
    return {"workload": "mamba2_branch_b256" + ("_shared" if share else "_copy"),
            "fork_pairs": pairs, "bytes_per_sequence": per_seq,
            "fork_avg_us": fork_us, "fork_achieved_gbs": gbs, "fork_frac": gbs / HBM_PEAK_GBS,
            "restore_avg_us": sum(ms) / reps * 1e3}


def bench_best_of_n(dev, n=4, kind=0):
    """Best-of-n decode on the serving state (kind 0: Mamba-2, 1: GDN): 256 / n prompts, each
    forked into n continuations right after a fold, then the L - 1 replay steps of the next
    window. With shared checkpoints the n continuations read one checkpoint; with copies each
    reads its own."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["gdn_b256" if kind else "m2_b256"]
    shape = w["shape"]
    Bn, H, P, N, L = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window
    A, D = synth.head_constants(shape, w["seed"])
    out = {"workload": "%s_best_of_%d_b256" % ("gdn" if kind else "mamba2", n)}
    inputs = [synth.token_inputs_device(shape, w["seed"], "bench-bon", i) for i in range(2 * L)]
    for share in (0, 1):
        h0 = synth.initial_state_device(shape, w["seed"], w["h0_std"])
        cfg = bd.make_config(shape.kind, Bn, H, shape.groups, P, N, L, 1, bd.SSM_IN_BF16,
                             share_ckpt=share)
        st = bd.State(cfg, h0, None if A is None else A.to(dev), None if D is None else D.to(dev))
        del h0
        y = torch.empty(Bn, H, P, device=dev)
        for i in range(L):  # one window: ends on the fold
            bd.ssm_replay_decode(st, inputs[i], y)
        src = [b for b in range(0, Bn, n) for _ in range(n - 1)]
        dst = [b + j for b in range(0, Bn, n) for j in range(1, n)]
        _, fms = timed_calls(1, lambda i: bd.ssm_fork(st, src, dst))
        wall, ms = timed_calls(L - 1, lambda i: bd.ssm_replay_decode(st, inputs[L + i], y))
        out["shared" if share else "copied"] = {
            "fork_us": fms[0] * 1e3, "replay_avg_us": sum(ms) / len(ms) * 1e3,
            "tokens_per_s": Bn * (L - 1) / wall,
            "checkpoint_bytes_read_per_step": (Bn // n if share else Bn) * H * P * N * 4}
        del st
        torch.cuda.empty_cache()
    return out


def bench_readcopy(dev, rc, steps=128, warm=16, layers=4, pool=16):
    """Decode with the fp8 or fp4 read copy on `layers` rotated layer instances (the fp4 copy of
    one layer fits the 256 MB last-level cache, so each step reads a different layer)."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["m2_b256_readcopy"]
    shape = w["shape"]
    Bn, H, P, N, L = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window
    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, shape.groups, P, N, L, 1, bd.SSM_IN_BF16, rc)
    sts = []
    for layer in range(layers):
        A, D = synth.head_constants(shape, w["seed"], layer)
        h0 = synth.initial_state_device(shape, w["seed"], w["h0_std"], layer)
        sts.append(bd.State(cfg, h0, A.to(dev), D.to(dev)))
        del h0
    inputs = [synth.token_inputs_device(shape, w["seed"], "bench-rc", i) for i in range(pool)]
    y = torch.empty(Bn, H, P, device=dev)
    # every layer steps once per `layers` calls, so each layer's window advances in lock step
    n_warm, n = warm * layers, steps * layers
    for i in range(n_warm):
        bd.ssm_replay_decode(sts[i % layers], inputs[i % pool], y)
    wall, ms = timed_calls(n, lambda i: bd.ssm_replay_decode(sts[i % layers],
                                                             inputs[(n_warm + i) % pool], y),
                           kind=lambda i: ((n_warm + i) // layers) % L == L - 1)
    heads = Bn * H
    rep_b = rep_ms = 0.0
    flush_ms = []
    for i, m in enumerate(ms):
        k = ((n_warm + i) // layers) % L + 1
        if k == L:
            flush_ms.append(m)
            continue
        rep_b += heads * m2_rc_replay_bytes_per_head(P, N, k, rc)
        rep_ms += m
    gbs = rep_b / (rep_ms * 1e-3) / 1e9
    return {"workload": "mamba2_readcopy_%s_b256" % ("fp8row" if rc == 1 else "fp4b16"),
            "tokens_per_s": Bn * n / wall, "unit": "tokens/s/layer", "layers_rotated": layers,
            "ms_per_step": wall / n * 1e3, "replay_avg_us": rep_ms / (n - len(flush_ms)) * 1e3,
            "replay_achieved_gbs": gbs, "replay_frac": gbs / HBM_PEAK_GBS,
            "fold_step_avg_us": sum(flush_ms) / max(len(flush_ms), 1) * 1e3,
            **fold_step_rate(heads * m2_fused_step_bytes_per_head(P, N, L, rc), flush_ms)}


def gdn_rc_replay_bytes_per_head(dv, dk, k, rc, esz=2, gsz=4):
    """GDN / KDA replay launch reading the low-precision copy instead of the fp32 state."""
    return gdn_replay_bytes_per_head(dv, dk, k, esz, gsz) - dv * dk * 4 + rc_copy_bytes_per_head(dv, dk, rc)


def bench_gdn(dev, steps=128, warm=16, layers=2, pool=16, rc=0, kda=False):
    """Gated DeltaNet (or, kda=True, Kimi Delta Attention) layer at B=256, H=32, dv=dk=128,
    L=16 on `layers` rotated layer instances: replay path (reading the fp32 state, or its fp8 /
    fp4 copy) vs the conventional read-modify-write step (fp32 state only)."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["kda_b256" if kda else "gdn_b256"]
    shape = w["shape"]
    Bn, H, dv, dk, L = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window
    gsz = 4 * dk if kda else 4
    cfg = bd.make_config(bd.SSM_KDA if kda else bd.SSM_GDN, Bn, H, H, dv, dk, L, 1,
                         bd.SSM_IN_BF16, rc)
    sts, convs = [], []
    for layer in range(layers):
        s0 = synth.initial_state_device(shape, w["seed"], w["h0_std"], layer)
        sts.append(bd.State(cfg, s0, None, None))
        if rc == 0:
            t = torch.empty(Bn * H * dv * dk, device=dev)
            bd.ssm_tiles_pack(cfg, s0, t)
            convs.append(t)
        del s0
    inputs = [synth.token_inputs_device(shape, w["seed"], "bench-gdn", i) for i in range(pool)]
    o = torch.empty(Bn, H, dv, device=dev)
    n_warm, n = warm * layers, steps * layers
    for i in range(n_warm):
        bd.ssm_replay_decode(sts[i % layers], inputs[i % pool], o)
    wall, ms = timed_calls(n, lambda i: bd.ssm_replay_decode(sts[i % layers],
                                                             inputs[(n_warm + i) % pool], o),
                           kind=lambda i: ((n_warm + i) // layers) % L == L - 1)
    heads = Bn * H
    rep_b = rep_ms = 0.0
    fold = []
    for i, m in enumerate(ms):
        k = ((n_warm + i) // layers) % L + 1
        if k == L:
            fold.append(m)
            continue
        rep_b += heads * (gdn_replay_bytes_per_head(dv, dk, k, gsz=gsz) if rc == 0 else
                          gdn_rc_replay_bytes_per_head(dv, dk, k, rc, gsz=gsz))
        rep_ms += m
    gbs = rep_b / (rep_ms * 1e-3) / 1e9
    if rc != 0:
        return {"workload": "%s_readcopy_%s_b256" % ("kda" if kda else "gdn",
                                                      "fp8row" if rc == 1 else "fp4b16"),
                "tokens_per_s": Bn * n / wall, "unit": "tokens/s/layer", "layers_rotated": layers,
                "ms_per_step": wall / n * 1e3, "replay_avg_us": rep_ms / (n - len(fold)) * 1e3,
                "replay_achieved_gbs": gbs, "replay_frac": gbs / HBM_PEAK_GBS,
                "fold_step_avg_us": sum(fold) / max(len(fold), 1) * 1e3,
                **fold_step_rate(heads * gdn_fused_step_bytes_per_head(dv, dk, L, rc, gsz=gsz), fold)}
    for i in range(n_warm):
        bd.ssm_conventional_step(cfg, convs[i % layers], inputs[i % pool], None, None, o)
    cwall, cms = timed_calls(n, lambda i: bd.ssm_conventional_step(
        cfg, convs[i % layers], inputs[(n_warm + i) % pool], None, None, o), kind=lambda i: 0)
    cgbs = heads * gdn_conv_bytes_per_head(dv, dk, gsz=gsz) / (sum(cms) / n * 1e-3) / 1e9
    return {"workload": "kda_replay_decode_b256" if kda else "gdn_replay_decode_b256",
            "tokens_per_s": Bn * n / wall,
            "unit": "tokens/s/layer", "layers_rotated": layers, "ms_per_step": wall / n * 1e3,
            "replay_avg_us": rep_ms / (n - len(fold)) * 1e3, "replay_achieved_gbs": gbs,
            "replay_frac": gbs / HBM_PEAK_GBS,
            "fold_step_avg_us": sum(fold) / max(len(fold), 1) * 1e3,
            **fold_step_rate(heads * gdn_fused_step_bytes_per_head(dv, dk, L, gsz=gsz), fold),
            "conventional": {"tokens_per_s": Bn * n / cwall, "avg_us": sum(cms) / n * 1e3,
                             "achieved_gbs": cgbs, "frac": cgbs / HBM_PEAK_GBS},
            "speedup_vs_conventional": (Bn * n / wall) / (Bn * n / cwall)}


def bench_gdn_spec(dev, rounds=64, warm=16, pool=16, layers=2, kda=False):
    """Gated DeltaNet (kda=True: Kimi Delta Attention) speculative decoding at B=256, H=32,
    dv=dk=128: 4 drafts per round verified in one replay call, U{0..4} accepted, pointer
    rollback (a fold fires whenever a sequence reaches L); `layers` rotated layer instances."""
    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth
    w = synth.WORKLOADS["gdn_b256_spec"]
    shape = w["shape"]
    Bn, H, dv, dk, L, S = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window, w["ndraft"]
    if kda:  # the same shapes and draws with one decay per key channel
        shape = dataclasses.replace(shape, kind=synth.KDA)
    gsz = 4 * dk if kda else 4
    cfg = bd.make_config(bd.SSM_KDA if kda else bd.SSM_GDN, Bn, H, H, dv, dk, L, S, bd.SSM_IN_BF16)
    sts = []
    for layer in range(layers):
        s0 = synth.initial_state_device(shape, w["seed"], w["h0_std"], layer)
        sts.append(bd.State(cfg, s0, None, None))
        del s0
    drafts = [synth.token_inputs_device(shape, w["seed"], "bench-draft", i, ntok=S)
              for i in range(pool)]
    accs = [synth.accept_counts(Bn, S, w["accept_seed"], r) for r in range(warm + rounds)]
    accs_d = [a.to(dev) for a in accs]
    o = torch.empty(Bn, S, H, dv, device=dev)
    counts = [[0] * Bn for _ in range(layers)]

    def advance(r, layer):
        for b in range(Bn):
            counts[layer][b] += int(accs[r][b])
            if counts[layer][b] >= L:
                counts[layer][b] -= L

    n_warm, n = warm * layers, rounds * layers
    for i in range(n_warm):
        r, layer = i // layers, i % layers
        bd.ssm_spec_append(sts[layer], S, drafts[i % pool], o)
        bd.ssm_spec_rollback(sts[layer], accs_d[r])
        advance(r, layer)
    ver_bytes = 0.0
    for i in range(n_warm, n_warm + n):
        r, layer = i // layers, i % layers
        ver_bytes += H * sum(gdn_verify_bytes_per_head(dv, dk, c, S, gsz=gsz) for c in counts[layer])
        advance(r, layer)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        r, layer = (n_warm + i) // layers, (n_warm + i) % layers
        ev[i][0].record()
        bd.ssm_spec_append(sts[layer], S, drafts[(n_warm + i) % pool], o)
        ev[i][1].record()
        bd.ssm_spec_rollback(sts[layer], accs_d[r])
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ver = sum(e[0].elapsed_time(e[1]) for e in ev)
    rb = sum(e[1].elapsed_time(e[2]) for e in ev)
    accepted = sum(int(accs[(n_warm + i) // layers].sum()) for i in range(n))
    gbs = ver_bytes / (ver * 1e-3) / 1e9
    del sts
    torch.cuda.empty_cache()
    # the comparison point: conventional speculation writes the state after every draft and
    # restores the accepted one (the same rounds, drafts, acceptances and rotated layers)
    hs = []
    for layer in range(layers):
        s0 = synth.initial_state_device(shape, w["seed"], w["h0_std"], layer)
        t = torch.empty(Bn * H * dv * dk, device=dev)
        bd.ssm_tiles_pack(cfg, s0, t)
        hs.append(t)
        del s0
    snap = torch.empty(S, Bn * H * dv * dk, device=dev)
    for i in range(n_warm):
        r, layer = i // layers, i % layers
        bd.ssm_conventional_spec_snapshot(cfg, hs[layer], snap, S, drafts[i % pool], None, None, o)
        bd.ssm_conventional_spec_select(cfg, hs[layer], snap, S, accs_d[r])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        r, layer = (n_warm + i) // layers, (n_warm + i) % layers
        ev[i][0].record()
        bd.ssm_conventional_spec_snapshot(cfg, hs[layer], snap, S, drafts[(n_warm + i) % pool],
                                          None, None, o)
        ev[i][1].record()
        bd.ssm_conventional_spec_select(cfg, hs[layer], snap, S, accs_d[r])
        ev[i][2].record()
    torch.cuda.synchronize()
    swall = time.perf_counter() - t0
    sn = sum(e[0].elapsed_time(e[1]) for e in ev)
    sel = sum(e[1].elapsed_time(e[2]) for e in ev)
    sgbs = Bn * H * gdn_snapshot_bytes_per_head(dv, dk, S, gsz=gsz) * n / (sn * 1e-3) / 1e9
    del snap, hs
    return {"workload": ("kda" if kda else "gdn") + "_spec_b256_4drafts",
            "accepted_tokens_per_s": accepted / wall,
            "unit": "accepted tokens/s/layer", "rounds": n, "layers_rotated": layers,
            "mean_accept": accepted / (Bn * n), "verify_avg_us": ver / n * 1e3,
            "verify_achieved_gbs": gbs, "verify_frac": gbs / HBM_PEAK_GBS,
            "rollback_and_fold_avg_us": rb / n * 1e3, "ms_per_round": wall / n * 1e3,
            "conventional_snapshot": {
                "accepted_tokens_per_s": accepted / swall, "ms_per_round": swall / n * 1e3,
                "snapshot_avg_us": sn / n * 1e3, "snapshot_achieved_gbs": sgbs,
                "snapshot_frac": sgbs / HBM_PEAK_GBS, "select_avg_us": sel / n * 1e3},
            "speedup_vs_snapshot": swall / wall}


def cpu_baseline(seconds_target: float = 10.0):
    """The fp64 oracle (sequential recurrence, OpenMP over heads) on a bounded sample of the
    serving workload: S sequences x all 128 heads x 16 tokens, S sized for ~seconds_target of
    wall time (calibrated on a 4-sequence run). Input generation is outside the timing."""
    import dataclasses

    import numpy as np
    import oracle
    from ssm_decode_state_amd import synth

    w = synth.WORKLOADS["m2_b256"]
    full = w["shape"]
    H, P, N, T = full.heads, full.dim_p, full.dim_n, 16
    A, D = synth.head_constants(full, w["seed"])

    def sample(nseq):
        shape = dataclasses.replace(full, batch=nseq)
        toks = [synth.token_inputs(shape, w["seed"], "cpu", t) for t in range(T)]
        x = torch_cat([d["x"] for d in toks]).permute(0, 2, 1, 3).reshape(nseq * H, T, P)
        Bm = torch_cat([d["B"] for d in toks]).permute(0, 2, 1, 3).reshape(nseq * H, T, N)
        Cm = torch_cat([d["C"] for d in toks]).permute(0, 2, 1, 3).reshape(nseq * H, T, N)
        dt = torch_cat([d["dt"] for d in toks]).permute(0, 2, 1).reshape(nseq * H, T)
        h0 = synth.initial_state(shape, w["seed"], w["h0_std"])
        return (np.tile(A.double().numpy(), nseq), np.tile(D.double().numpy(), nseq),
                synth.to_f64(h0.reshape(nseq * H, P, N)), synth.to_f64(x), synth.to_f64(Bm),
                synth.to_f64(Cm), synth.to_f64(dt))

    oracle.build()
    cal = 4
    args = sample(cal)
    t0 = time.perf_counter()
    oracle.m2_sequential(*args)
    t_cal = time.perf_counter() - t0
    want = cal * seconds_target / max(t_cal, 1e-3)  # sequences x 16 tokens for the target time
    nseq = int(max(1, min(full.batch, round(want))))
    reps = int(max(1, round(want / nseq)))  # beyond the full batch: repeat the same sample
    args = sample(nseq)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.m2_sequential(*args)
    el = time.perf_counter() - t0
    cores = oracle.num_threads()
    # the same oracle on one core, on a sample sized for about a third of the time
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.m2_sequential(*sample(1))
    t1 = time.perf_counter() - t0
    n1 = int(max(1, min(full.batch, round(seconds_target / 3 / max(t1, 1e-3)))))
    args1 = sample(n1)
    t0 = time.perf_counter()
    oracle.m2_sequential(*args1)
    el1 = time.perf_counter() - t0
    oracle.set_threads(None)
    gdn = cpu_baseline_gdn(seconds_target / 2)
    model = cpu_model()
    return {"value": reps * nseq * T / el, "unit": "tokens/s/layer", "cores": cores,
            "kind": "oracle",
            "sample": "%d of 256 sequences x 128 heads x %d tokens of the serving workload, run %d "
                      "time(s); fp64 sequential recurrence (C, OpenMP over heads), %.1f s"
                      % (nseq, T, reps, el),
            "single_core": {"value": n1 * T / el1, "sample": "%d sequences, %.1f s" % (n1, el1)},
            "gdn": gdn, "cpu_model": model}


def cpu_model() -> dict:
    """The host CPU as lscpu and /proc/cpuinfo name it (model name, family / model / stepping,
    sockets, cores), for the CPU baseline's record."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "CPU family", "Model", "Stepping", "Socket(s)",
                             "Core(s) per socket", "Thread(s) per core", "CPU(s)", "Vendor ID",
                             "CPU max MHz", "Hypervisor vendor"):
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        names = sorted({l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                        if l.startswith("model name")})
        info["cpuinfo_model_name"] = "; ".join(names)
    except OSError:
        pass
    info["affinity_cpus"] = len(os.sched_getaffinity(0))
    return info


def cpu_baseline_gdn(seconds_target: float = 5.0):
    """The fp64 oracle's gated delta rule on a bounded sample of the GDN serving workload (B=256,
    H=32, dv=dk=128): S sequences x all 32 heads x 16 tokens, sized like cpu_baseline."""
    import dataclasses

    import numpy as np
    import oracle
    from ssm_decode_state_amd import synth

    w = synth.WORKLOADS["gdn_b256"]
    full = w["shape"]
    H, dv, dk, T = full.heads, full.dim_p, full.dim_n, 16

    def sample(nseq):
        shape = dataclasses.replace(full, batch=nseq)
        toks = [synth.token_inputs(shape, w["seed"], "cpu", t) for t in range(T)]
        cat = {key: torch_cat([d[key] for d in toks]) for key in ("q", "k", "v", "beta", "g")}
        q, k, v = [cat[key].permute(0, 2, 1, 3).reshape(nseq * H, T, -1) for key in ("q", "k", "v")]
        beta, g = [cat[key].permute(0, 2, 1).reshape(nseq * H, T) for key in ("beta", "g")]
        S0 = synth.initial_state(shape, w["seed"], w["h0_std"])
        return (synth.to_f64(S0.reshape(nseq * H, dv, dk)), synth.to_f64(q), synth.to_f64(k),
                synth.to_f64(v), synth.to_f64(beta), synth.to_f64(g))

    cal = 4
    args = sample(cal)
    t0 = time.perf_counter()
    oracle.gdn_sequential(*args)
    t_cal = time.perf_counter() - t0
    want = cal * seconds_target / max(t_cal, 1e-3)  # sequences x 16 tokens for the target time
    nseq = int(max(1, min(full.batch, round(want))))
    reps = int(max(1, round(want / nseq)))  # beyond the full batch: repeat the same sample
    args = sample(nseq)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gdn_sequential(*args)
    el = time.perf_counter() - t0
    return {"value": reps * nseq * T / el, "unit": "tokens/s/layer", "cores": oracle.num_threads(),
            "sample": "%d of 256 sequences x 32 heads x %d tokens of the GDN serving workload, "
                      "run %d time(s); fp64 sequential gated delta rule, %.1f s"
                      % (nseq, T, reps, el)}


def torch_cat(ts):
    import torch
    return torch.cat(ts, 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-conv", action="store_true", help="skip the conventional comparison")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the headline eagerly only (for counter-collection runs, which do "
                         "not follow graph replays)")
    ap.add_argument("--copy-ref", type=int, default=0,
                    help="also run a plain copy of this many MiB (reference for HBM counters)")
    ap.add_argument("--workloads", default="all",
                    help="comma list of extra workloads: spec, fp8, fp4, gdn, gdn_spec, "
                         "gdn_fp8, gdn_fp4, kda, g8 (8 B/C groups), lsweep (window 4..32), "
                         "bsweep (batch 1..256), branch (fork and restore), kda_fp8, kda_fp4, "
                         "kda_spec; 'all' or 'none'")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the ReplaySSM decode path needs no cross-GPU exchange "
              "(sequences and heads shard independently), and this build runs on a single "
              "MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from ssm_decode_state_amd import binding as bd
    from ssm_decode_state_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS["m2_b256"]
    shape = w["shape"]
    Bn, H, G, P, N, L = (shape.batch, shape.heads, shape.groups, shape.dim_p, shape.dim_n,
                         shape.window)
    K, W = args.steps, args.warmup
    seed = w["seed"]

    A, D = synth.head_constants(shape, seed)
    Ad, Dd = A.to(dev), D.to(dev)
    h0 = synth.initial_state_device(shape, seed, w["h0_std"])
    inputs = [synth.token_inputs_device(shape, seed, "bench", t) for t in range(W + K)]
    torch.cuda.synchronize()

    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, G, P, N, L, 1, bd.SSM_IN_BF16)
    st = bd.State(cfg, h0, Ad, Dd)
    y = torch.empty(Bn, H, P, device=dev)

    # ---- first launches: one window on a separate state of the same shape loads every kernel
    #      the timed steps use (replay at each count, the fused fold, the conventional step), so
    #      a warm-up shorter than a window leaves no first launch inside the timed region (and
    #      every launch of these kernels in this process has the serving shape)
    st1 = bd.State(cfg, None, Ad, Dd)
    for t in range(L):
        bd.ssm_replay_decode(st1, inputs[0], y)
    t1 = torch.zeros(Bn * H * P * N, device=dev)
    bd.ssm_conventional_step(cfg, t1, inputs[0], Ad, Dd, y)
    torch.cuda.synchronize()
    del st1, t1

    # ---- replay path, eager: one launch per step from Python behind a GPU pre-roll. Per-kernel
    #      figures come from runs of back-to-back launches of one kernel (a window's L-1 replays,
    #      then the fused fold) with events only at the run boundaries -----------------------
    for t in range(W):
        bd.ssm_replay_decode(st, inputs[t], y)
    # the eager figure: GPU time from the first step's start to the last step's end (the pre-roll
    # keeps host launch latency out of it), for REPS passes of the K steps in a row (the state
    # moves on; each pass reuses the K inputs): the headline is the median pass, the per-kernel
    # figures sum all passes
    heads = Bn * H
    rep_bytes = rep_ms = 0.0
    flush_steps = []
    passes = []
    n_rep = 0
    for r in range(REPS):
        ks = [((W + r * K + t) % L) + 1 for t in range(K)]  # committed count after the append
        t_pass, step_ms = timed_calls(K, lambda t: bd.ssm_replay_decode(st, inputs[W + t], y),
                                      kind=lambda t, ks=ks: ks[t] == L)
        passes.append(t_pass)
        for k, ms in zip(ks, step_ms):
            if k == L:
                flush_steps.append(ms)
                continue
            rep_bytes += heads * m2_replay_bytes_per_head(P, N, k)
            rep_ms += ms
            n_rep += 1
    t_eager = sorted(passes)[REPS // 2]
    rep_avg_ms = rep_ms / max(n_rep, 1)
    rep_gbs = rep_bytes / (rep_ms * 1e-3) / 1e9 if rep_ms > 0 else float("nan")
    # the L-th step of each window is one fused pass: fold the window and emit the output from
    # the new checkpoint (checkpoint read + write, L-1 buffered entries, this token, y)
    fold_ms = sum(flush_steps) / len(flush_steps) if flush_steps else None
    fold_bytes = heads * m2_fused_step_bytes_per_head(P, N, L)
    fold_gbs = fold_bytes / (fold_ms * 1e-3) / 1e9 if fold_ms else None
    # the replay launches timed above run at counts 1..L-1 (the L-th step is the fused fold)
    mean_bytes_per_head = rep_bytes / heads / max(n_rep, 1)
    # per-count launch times (a diagnostic: the replay grows with the entries it reads): the same
    # K steps once more, an event pair around each launch
    _, each_ms = timed_calls(K, lambda t: bd.ssm_replay_decode(st, inputs[W + t], y))
    per_k = {}
    for t, ms in enumerate(each_ms):
        per_k.setdefault(((W + REPS * K + t) % L) + 1, []).append(ms)

    # ---- the headline: the back-to-back pass above -- HIP events bracket exactly the K steps
    #      (GPU time from the first step's start to the last step's end), behind a pre-roll that
    #      keeps host launch latency out. The same K steps as one captured HIP graph are reported
    #      beside it (from the state the passes left; restored after the graph's warm-up replay).
    value, ms_step = Bn * K / t_eager, t_eager / K * 1e3
    timing = ("the K steps launched back to back from Python behind a GPU pre-roll; HIP events "
              "bracket exactly the K steps, synchronized before and after; the median of %d such "
              "passes in a row" % REPS)
    graph = (None if args.no_graph else
             graph_steps(lambda i: bd.ssm_replay_decode(st, inputs[W + i], y), K, st.mem))
    if graph is not None:
        graph["value"] = Bn * K / graph["gpu_s"]
    out = {
        "metric": "SSM decode tokens/sec per layer at B=256 + % of HBM peak (replay vs "
                  "conventional)",
        "value": value, "unit": "tokens/s/layer", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "mamba2_replay_decode_b256", "batch": Bn, "heads": H,
                   "groups": G, "head_dim": P, "state_dim": N, "window": L,
                   "inputs": "bf16 x/B/C, fp32 dt", "checkpoint": "fp32"},
        "timing": timing,
        "passes_tokens_per_s": [Bn * K / t for t in passes],
        "roofline": {"bound": "hbm", "achieved": rep_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": rep_gbs / HBM_PEAK_GBS, "traffic": pmc_traffic(),
                     "algorithmic_bytes_per_launch": rep_bytes / max(n_rep, 1),
                     "kernel": "m2_replay_kernel<64,128,bf16,1q>",
                     "avg_launch_us": rep_avg_ms * 1e3,
                     "bytes_per_head_mean_k": mean_bytes_per_head,
                     "launches": n_rep},
        "fold_step": {"avg_us": None if fold_ms is None else fold_ms * 1e3,
                      "achieved_gbs": fold_gbs, "per_window": 1,
                      "kernel": "m2_fold_kernel<64,128,bf16,fused>"},
        "step_us_by_count": {str(k): sum(v) / len(v) * 1e3 for k, v in sorted(per_k.items())},
    }
    if graph is not None:
        graph["note"] = ("the K steps as one HIP graph, replayed once untimed, the state restored, "
                         "replayed again behind a GPU pre-roll with HIP events around it; the "
                         "graph launch of a short K outlasts the pre-roll, so its first steps "
                         "wait for the host")
        out["graph"] = graph
    if fold_ms is not None:
        # one window's worth of steps at the measured per-launch times: (L - 1) replays and the
        # fused fold, whatever fraction of folds the K timed steps happened to hold
        amort_us = ((L - 1) * rep_avg_ms + fold_ms) / L * 1e3
        out["window_amortized"] = {"step_us": amort_us, "tokens_per_s": Bn / (amort_us * 1e-6),
                                   "folds_in_timed_passes": len(flush_steps),
                                   "note": "((L-1) * replay + fused fold) / L from the per-launch "
                                           "event times"}

    # ---- conventional comparison on the same shapes and inputs, timed the same way -------------
    if not args.skip_conv:
        tiles = torch.empty(Bn * H * P * N, device=dev)
        bd.ssm_tiles_pack(cfg, h0, tiles)
        for t in range(W):
            bd.ssm_conventional_step(cfg, tiles, inputs[t], Ad, Dd, y)
        torch.cuda.synchronize()
        conv_passes, cms = [], []
        for r in range(REPS):
            t_c, c_ms = timed_calls(K, lambda t: bd.ssm_conventional_step(cfg, tiles, inputs[W + t],
                                                                          Ad, Dd, y),
                                    kind=lambda t: 0)
            conv_passes.append(t_c)
            cms += c_ms
        t_conv = sorted(conv_passes)[REPS // 2]
        conv_ms = sum(cms) / len(cms)
        conv_gbs = heads * m2_conv_bytes_per_head(P, N) / (conv_ms * 1e-3) / 1e9
        out["conventional"] = {"value": Bn * K / t_conv, "unit": "tokens/s/layer",
                               "ms_per_step": t_conv / K * 1e3, "avg_launch_us": conv_ms * 1e3,
                               "achieved_gbs": conv_gbs, "frac": conv_gbs / HBM_PEAK_GBS,
                               "timing": "the K steps back to back, median of %d passes, as the "
                                         "headline" % REPS}
        gconv = (None if args.no_graph else
                 graph_steps(lambda i: bd.ssm_conventional_step(cfg, tiles, inputs[W + i], Ad, Dd, y),
                             K, tiles))
        if gconv is not None:
            out["conventional"]["graph_value"] = Bn * K / gconv["gpu_s"]
        out["speedup_vs_conventional"] = out["value"] / out["conventional"]["value"]
        if graph is not None and gconv is not None:
            out["speedup_vs_conventional_graph"] = graph["value"] / out["conventional"]["graph_value"]
        out["per_token_latency_us"] = {"replay_window_amortized": out.get("window_amortized", {}).get("step_us"),
                                       "conventional": conv_ms * 1e3}

    # ---- the read ceiling: plain streaming reads, 64 MiB .. 1 GiB per launch -------------------
    out["read_ceiling"] = bench_read_ceiling(dev)
    out["roofline"]["frac_of_read_ceiling"] = rep_gbs / ceiling_at(out["read_ceiling"], rep_bytes / max(n_rep, 1))

    if args.copy_ref:
        n = args.copy_ref * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            torch.neg(src, out=dst)
        e1.record()
        torch.cuda.synchronize()
        out["copy_ref"] = {"bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 5,
                           "avg_us": e0.elapsed_time(e1) / 5 * 1e3}

    extra = ({"spec", "fp8", "fp4", "gdn", "gdn_spec", "gdn_fp8", "gdn_fp4", "kda", "g8", "lsweep",
              "bsweep", "branch", "kda_fp8", "kda_fp4", "kda_spec"}
             if args.workloads == "all" else
             set() if args.workloads == "none" else set(args.workloads.split(",")))
    if extra:
        del inputs, st, h0
        if not args.skip_conv:
            del tiles
        torch.cuda.empty_cache()
        out["workloads"] = {}
        if "spec" in extra:
            out["workloads"]["spec"] = bench_spec(dev)
            torch.cuda.empty_cache()
        if "g8" in extra:
            wg = synth.WORKLOADS["m2_b256"]
            r = bench_m2_decode(dev, dataclasses.replace(wg["shape"], groups=8), wg["seed"],
                                wg["h0_std"], 128, 32)
            out["workloads"]["groups8"] = dict(workload="mamba2_replay_decode_b256_g8", **r)
            torch.cuda.empty_cache()
        if "branch" in extra:
            out["workloads"]["branch"] = bench_branch(dev)
            out["workloads"]["branch_shared"] = bench_branch(dev, share=1)
            torch.cuda.empty_cache()
            out["workloads"]["best_of_4"] = bench_best_of_n(dev, 4)
            torch.cuda.empty_cache()
            out["workloads"]["gdn_best_of_4"] = bench_best_of_n(dev, 4, kind=1)
            torch.cuda.empty_cache()
        if "lsweep" in extra:
            out["workloads"]["window_sweep"] = bench_lsweep(dev)
            torch.cuda.empty_cache()
        if "bsweep" in extra:
            out["workloads"]["batch_sweep"] = bench_bsweep(dev)
            torch.cuda.empty_cache()
        if "fp8" in extra:
            out["workloads"]["readcopy_fp8"] = bench_readcopy(dev, 1)
            torch.cuda.empty_cache()
        if "fp4" in extra:
            out["workloads"]["readcopy_fp4"] = bench_readcopy(dev, 2)
            torch.cuda.empty_cache()
        if "gdn" in extra:
            out["workloads"]["gdn"] = bench_gdn(dev)
            torch.cuda.empty_cache()
        if "kda" in extra:
            out["workloads"]["kda"] = bench_gdn(dev, kda=True)
            torch.cuda.empty_cache()
        if "gdn_fp8" in extra:
            out["workloads"]["gdn_readcopy_fp8"] = bench_gdn(dev, layers=4, rc=1)
            torch.cuda.empty_cache()
        if "gdn_fp4" in extra:
            out["workloads"]["gdn_readcopy_fp4"] = bench_gdn(dev, layers=4, rc=2)
            torch.cuda.empty_cache()
        if "kda_fp8" in extra:
            out["workloads"]["kda_readcopy_fp8"] = bench_gdn(dev, layers=4, rc=1, kda=True)
            torch.cuda.empty_cache()
        if "kda_fp4" in extra:
            out["workloads"]["kda_readcopy_fp4"] = bench_gdn(dev, layers=4, rc=2, kda=True)
            torch.cuda.empty_cache()
        if "gdn_spec" in extra:
            out["workloads"]["gdn_spec"] = bench_gdn_spec(dev)
            torch.cuda.empty_cache()
        if "kda_spec" in extra:
            out["workloads"]["kda_spec"] = bench_gdn_spec(dev, kda=True)
            torch.cuda.empty_cache()

    annotate_ceiling({k: v for k, v in out.items() if k not in ("roofline", "read_ceiling")},
                     out["read_ceiling"])
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
