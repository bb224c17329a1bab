#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--skip-conv] [--copy-ref MB]

Workload (the headline): a Mamba-2 SSM layer decoding at serving batch -- B = 256 sequences,
H = 128 heads, head dim P = 64, state dim N = 128 (fp32 checkpoint, 4 MiB per sequence), window
L = 16, bf16 x/B/C and fp32 dt. One step = one decode token for every sequence through the whole
replay path: append to the ring, replay output from the checkpoint, and (every L-th step) the
flush that folds the window into the checkpoint. K steps are timed after W warm-up steps; K is a
multiple of L by default so the flush cost is amortised exactly.

Reported: tokens/s per layer (B * K / wall time), the in-house conventional read-modify-write step
on the same shapes and inputs, the replay kernel's achieved HBM bandwidth from per-launch HIP
events against the algorithmic bytes, and the fp64 CPU oracle timed on a bounded sample of the
same workload on this host.

Inputs are seeded synthetic draws made on the device (ssm_decode_state_amd.synth) and resident in
HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def m2_replay_bytes_per_head(P, N, k, esz=2):
    """Algorithmic bytes of one replay launch for one head at committed count k (after append):
    checkpoint read + the k-1 older ring entries read (x, B, dt) + the token's inputs read and
    appended (x, B, C, dt) + y written + the pointer pair read and the count written."""
    entry_rd = P * esz + N * esz + 4
    token = P * esz + 2 * N * esz + 4
    return P * N * 4 + (k - 1) * entry_rd + 2 * token + P * 4 + 12


def m2_flush_bytes_per_head(P, N, L, esz=2):
    """Checkpoint read + write and the L folded entries read (x, B, dt) + pointers."""
    return 2 * P * N * 4 + L * (P * esz + N * esz + 4) + 16


def m2_conv_bytes_per_head(P, N, esz=2):
    """State read + write, the token's inputs read, y written."""
    return 2 * P * N * 4 + P * esz + 2 * N * esz + 4 + P * 4


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
    nseq = int(max(1, min(full.batch, round(cal * seconds_target / max(t_cal, 1e-3)))))
    args = sample(nseq)
    t0 = time.perf_counter()
    oracle.m2_sequential(*args)
    el = time.perf_counter() - t0
    return {"value": nseq * T / el, "unit": "tokens/s/layer", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d of 256 sequences x 128 heads x %d tokens of the serving workload, fp64 "
                      "sequential recurrence (C, OpenMP over heads), %.1f s" % (nseq, T, el)}


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
    ap.add_argument("--copy-ref", type=int, default=0,
                    help="also run a plain copy of this many MiB (reference for HBM counters)")
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

    # ---- replay path -------------------------------------------------------------------------
    for t in range(W):
        bd.ssm_replay_decode(st, inputs[t], y)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0 = time.perf_counter()
    for t in range(K):
        ev[t][0].record()
        bd.ssm_replay_decode(st, inputs[W + t], y)
        ev[t][1].record()
    torch.cuda.synchronize()
    t_replay = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ks = [((W + t) % L) + 1 for t in range(K)]  # committed count after the append

    heads = Bn * H
    rep_bytes = rep_ms = 0.0
    flush_steps = []
    for k, ms in zip(ks, step_ms):
        if k == L:
            flush_steps.append(ms)
            continue
        rep_bytes += heads * m2_replay_bytes_per_head(P, N, k)
        rep_ms += ms
    n_rep = K - len(flush_steps)
    rep_avg_ms = rep_ms / max(n_rep, 1)
    rep_gbs = rep_bytes / (rep_ms * 1e-3) / 1e9 if rep_ms > 0 else float("nan")
    replay_at_L_ms = heads * m2_replay_bytes_per_head(P, N, L) / (rep_gbs * 1e9) * 1e3
    flush_ms = (sum(flush_steps) / len(flush_steps) - replay_at_L_ms) if flush_steps else None
    flush_gbs = (heads * m2_flush_bytes_per_head(P, N, L) / (flush_ms * 1e-3) / 1e9
                 if flush_ms else None)
    tok_s = Bn * K / t_replay
    mean_bytes_per_head = sum(m2_replay_bytes_per_head(P, N, k) for k in range(1, L + 1)) / L

    out = {
        "metric": "SSM decode tokens/sec per layer at B=256 + % of HBM peak (replay vs "
                  "conventional)",
        "value": tok_s, "unit": "tokens/s/layer", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": t_replay / K * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "mamba2_replay_decode_b256", "batch": Bn, "heads": H,
                   "groups": G, "head_dim": P, "state_dim": N, "window": L,
                   "inputs": "bf16 x/B/C, fp32 dt", "checkpoint": "fp32"},
        "roofline": {"bound": "hbm", "achieved": rep_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": rep_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "m2_replay_kernel<64,128,bf16,1q>",
                     "avg_launch_us": rep_avg_ms * 1e3,
                     "bytes_per_head_mean_k": mean_bytes_per_head,
                     "launches": n_rep},
        "flush": {"avg_us": None if flush_ms is None else flush_ms * 1e3,
                  "achieved_gbs": flush_gbs, "per_window": 1},
    }

    # ---- conventional comparison on the same shapes and inputs ---------------------------------
    if not args.skip_conv:
        tiles = torch.empty(Bn * H * P * N, device=dev)
        bd.ssm_tiles_pack(cfg, h0, tiles)
        for t in range(W):
            bd.ssm_conventional_step(cfg, tiles, inputs[t], Ad, Dd, y)
        torch.cuda.synchronize()
        evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        t0 = time.perf_counter()
        for t in range(K):
            evc[t][0].record()
            bd.ssm_conventional_step(cfg, tiles, inputs[W + t], Ad, Dd, y)
            evc[t][1].record()
        torch.cuda.synchronize()
        t_conv = time.perf_counter() - t0
        conv_ms = sum(a.elapsed_time(b) for a, b in evc) / K
        conv_gbs = heads * m2_conv_bytes_per_head(P, N) / (conv_ms * 1e-3) / 1e9
        out["conventional"] = {"value": Bn * K / t_conv, "unit": "tokens/s/layer",
                               "ms_per_step": t_conv / K * 1e3, "avg_launch_us": conv_ms * 1e3,
                               "achieved_gbs": conv_gbs, "frac": conv_gbs / HBM_PEAK_GBS}
        out["speedup_vs_conventional"] = out["value"] / out["conventional"]["value"]
        del tiles

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

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
