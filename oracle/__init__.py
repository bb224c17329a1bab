"""fp64 CPU oracle for the ReplaySSM decode step -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package. It
shares no code with the HIP library (ssm_decode_state_amd/csrc) and never imports it; the only
module both sides use is ssm_decode_state_amd.synth, which draws the seeded inputs.

Contents:
  ssm_oracle.c  plain fp64 loops: Mamba-2, Gated DeltaNet and Kimi Delta Attention sequential
                recurrences (the definitions), their replay and flush forms, and speculative
                rounds.
  quant.py      fp8 e4m3 / fp4 e2m1 read-copy quantizers emulated in fp32 numpy, with error bounds.
  ring.py       the ring-buffer pointer state machine (start / count / pending per sequence).

The C part is compiled with gcc on first use (or by __graft_entry__.build()) into oracle/_build/.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, no FMA contraction, OpenMP across heads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        _declare(lib)
        _lib = lib
    return _lib


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def _d(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_dp)


def _i(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_ip)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


_threads: Optional[int] = None


def num_threads() -> int:
    """OpenMP threads the batch wrappers use (set_threads, else OMP_NUM_THREADS, else all cores
    in our affinity)."""
    if _threads is not None:
        return _threads
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        return int(env)
    return len(os.sched_getaffinity(0))


def set_threads(n: Optional[int]) -> None:
    """Threads for the batch wrappers (None = back to the default). Timing only."""
    global _threads
    _threads = n
    _load().orc_set_threads(n if n is not None else num_threads())


# ----------------------------------------------------------------------------------------------
# Mamba-2
# ----------------------------------------------------------------------------------------------
def m2_sequential(A, D, h0, x, B, C, dt, snap_after: Sequence[int] = ()):
    """Sequential Mamba-2 recurrence over independent heads.

    A, D: [nh]; h0: [nh][P][N] or None (zero); x: [nh][T][P]; B, C: [nh][T][N]; dt: [nh][T].
    Returns (y [nh][T][P], h_T [nh][P][N], snaps [nh][len(snap_after)][P][N])."""
    lib = _load()
    x, B, C, dt = _f64(x), _f64(B), _f64(C), _f64(dt)
    A, D = _f64(A).reshape(-1), _f64(D).reshape(-1)
    nh, T, P = x.shape
    N = B.shape[2]
    h0 = None if h0 is None else _f64(h0)
    y = np.zeros((nh, T, P))
    hT = np.zeros((nh, P, N))
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32))
    snaps = np.zeros((nh, len(snap), P, N))
    lib.orc_m2_sequential_batch(nh, P, N, T, _d(A), _d(D), _d(h0), _d(x), _d(B), _d(C), _d(dt),
                                _d(y), _d(hT), len(snap), _i(snap), _d(snaps))
    return y, hT, snaps


def m2_replay_output(A: float, D: float, hc, x, B, Ck, dt):
    """Replay form of one output for one head: hc [P][N], entries x [k][P], B [k][N], dt [k];
    Ck [N] is the current token's C (entry k)."""
    lib = _load()
    hc, x, B, Ck, dt = _f64(hc), _f64(x), _f64(B), _f64(Ck), _f64(dt)
    k, P = x.shape
    N = B.shape[1]
    y = np.zeros(P)
    lib.orc_m2_replay_output(P, N, k, ctypes.c_double(A), ctypes.c_double(D), _d(hc), _d(x),
                             _d(B), _d(Ck), _d(dt), _d(y))
    return y


def m2_flush(A: float, hc, x, B, dt):
    """Flush form for one head: fold entries x [L][P], B [L][N], dt [L] into hc [P][N]."""
    lib = _load()
    hc, x, B, dt = _f64(hc), _f64(x), _f64(B), _f64(dt)
    L, P = x.shape
    N = B.shape[1]
    out = np.zeros((P, N))
    lib.orc_m2_flush(P, N, L, ctypes.c_double(A), _d(hc), _d(x), _d(B), _d(dt), _d(out))
    return out


def m2_spec_rounds(A, D, h0, x, B, C, dt, accept, snap_after=None):
    """Speculative rounds over independent heads.

    x [nh][R][S][P], B/C [nh][R][S][N], dt [nh][R][S]; accept [nh][R] (drafts committed per
    round). snap_after [nh][nsnap]: committed-token counts after which the state is recorded.
    Returns (y [nh][R][S][P], h_final [nh][P][N], snaps [nh][nsnap][P][N])."""
    lib = _load()
    x, B, C, dt = _f64(x), _f64(B), _f64(C), _f64(dt)
    A, D = _f64(A).reshape(-1), _f64(D).reshape(-1)
    nh, R, S, P = x.shape
    N = B.shape[3]
    acc = np.ascontiguousarray(np.asarray(accept, dtype=np.int32).reshape(nh, R))
    if snap_after is None:
        snap_after = np.zeros((nh, 0), dtype=np.int32)
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32).reshape(nh, -1))
    ns = snap.shape[1]
    h0 = None if h0 is None else _f64(h0)
    y = np.zeros((nh, R, S, P))
    hT = np.zeros((nh, P, N))
    snaps = np.zeros((nh, ns, P, N))
    lib.orc_m2_spec_rounds_batch(nh, P, N, R, S, _d(A), _d(D), _d(h0), _d(x), _d(B), _d(C),
                                 _d(dt), _i(acc), _d(y), _d(hT), ns, _i(snap), _d(snaps))
    return y, hT, snaps


# ----------------------------------------------------------------------------------------------
# Gated DeltaNet
# ----------------------------------------------------------------------------------------------
def gdn_sequential(S0, q, k, v, beta, g, scale: float = 1.0, snap_after: Sequence[int] = ()):
    """Sequential gated delta rule over independent heads.

    S0 [nh][dv][dk] or None; q, k [nh][T][dk]; v [nh][T][dv]; beta, g [nh][T].
    Returns (o [nh][T][dv], S_T [nh][dv][dk], snaps [nh][nsnap][dv][dk])."""
    lib = _load()
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    nh, T, dk = q.shape
    dv = v.shape[2]
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((nh, T, dv))
    ST = np.zeros((nh, dv, dk))
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32))
    snaps = np.zeros((nh, len(snap), dv, dk))
    lib.orc_gdn_sequential_batch(nh, dv, dk, T, ctypes.c_double(scale), _d(S0), _d(q), _d(k),
                                 _d(v), _d(beta), _d(g), _d(o), _d(ST), len(snap), _i(snap),
                                 _d(snaps))
    return o, ST, snaps


def gdn_spec_rounds(S0, q, k, v, beta, g, accept, scale: float = 1.0, snap_after=None):
    """GDN speculative rounds over independent heads.

    q, k [nh][R][S][dk], v [nh][R][S][dv], beta/g [nh][R][S]; accept [nh][R]. snap_after
    [nh][nsnap]: committed-token counts after which the state is recorded.
    Returns (o [nh][R][S][dv], S_final [nh][dv][dk], snaps [nh][nsnap][dv][dk])."""
    lib = _load()
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    nh, R, S, dk = q.shape
    dv = v.shape[3]
    acc = np.ascontiguousarray(np.asarray(accept, dtype=np.int32).reshape(nh, R))
    if snap_after is None:
        snap_after = np.zeros((nh, 0), dtype=np.int32)
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32).reshape(nh, -1))
    ns = snap.shape[1]
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((nh, R, S, dv))
    ST = np.zeros((nh, dv, dk))
    snaps = np.zeros((nh, ns, dv, dk))
    lib.orc_gdn_spec_rounds_batch(nh, dv, dk, R, S, ctypes.c_double(scale), _d(S0), _d(q), _d(k),
                                  _d(v), _d(beta), _d(g), _i(acc), _d(o), _d(ST), ns, _i(snap),
                                  _d(snaps))
    return o, ST, snaps


# ----------------------------------------------------------------------------------------------
# Kimi Delta Attention (g is [..][dk]: one log-decay per key channel)
# ----------------------------------------------------------------------------------------------
def kda_sequential(S0, q, k, v, beta, g, scale: float = 1.0, snap_after: Sequence[int] = ()):
    """Sequential KDA recurrence over independent heads.

    S0 [nh][dv][dk] or None; q, k, g [nh][T][dk]; v [nh][T][dv]; beta [nh][T].
    Returns (o [nh][T][dv], S_T [nh][dv][dk], snaps [nh][nsnap][dv][dk])."""
    lib = _load()
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    nh, T, dk = q.shape
    dv = v.shape[2]
    assert g.shape == (nh, T, dk)
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((nh, T, dv))
    ST = np.zeros((nh, dv, dk))
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32))
    ns = snap.size
    snaps = np.zeros((nh, ns, dv, dk))
    lib.orc_kda_sequential_batch(nh, dv, dk, T, ctypes.c_double(scale), _d(S0), _d(q), _d(k),
                                 _d(v), _d(beta), _d(g), _d(o), _d(ST), ns, _i(snap), _d(snaps))
    return o, ST, snaps


def kda_replay_output(Sc, qk, k, v, beta, g, scale: float = 1.0):
    """KDA replay form for one head: checkpoint Sc [dv][dk], query qk [dk], entries k [kk][dk],
    v [kk][dv], beta [kk], g [kk][dk]. Returns o [dv]."""
    lib = _load()
    Sc, qk, k, v, beta, g = _f64(Sc), _f64(qk), _f64(k), _f64(v), _f64(beta), _f64(g)
    kk, dk = k.shape
    dv = v.shape[1]
    out = np.zeros(dv)
    lib.orc_kda_replay_output(dv, dk, kk, ctypes.c_double(scale), _d(Sc), _d(qk), _d(k), _d(v),
                              _d(beta), _d(g), _d(out))
    return out


def kda_spec_rounds(S0, q, k, v, beta, g, accept, scale: float = 1.0, snap_after=None):
    """KDA speculative rounds over independent heads: q, k, g [nh][R][S][dk], v [nh][R][S][dv],
    beta [nh][R][S], accept [nh][R]. Returns (o [nh][R][S][dv], S_final, snaps)."""
    lib = _load()
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    nh, R, S, dk = q.shape
    dv = v.shape[3]
    acc = np.ascontiguousarray(np.asarray(accept, dtype=np.int32).reshape(nh, R))
    if snap_after is None:
        snap_after = np.zeros((nh, 0), dtype=np.int32)
    snap = np.ascontiguousarray(np.asarray(snap_after, dtype=np.int32).reshape(nh, -1))
    ns = snap.shape[1]
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((nh, R, S, dv))
    ST = np.zeros((nh, dv, dk))
    snaps = np.zeros((nh, ns, dv, dk))
    lib.orc_kda_spec_rounds_batch(nh, dv, dk, R, S, ctypes.c_double(scale), _d(S0), _d(q), _d(k),
                                  _d(v), _d(beta), _d(g), _i(acc), _d(o), _d(ST), ns, _i(snap),
                                  _d(snaps))
    return o, ST, snaps


def gdn_replay_output(Sc, qk, k, v, beta, g, scale: float = 1.0):
    """GDN replay (backward sweep) for one head: Sc [dv][dk], qk [dk], entries k [kk][dk],
    v [kk][dv], beta/g [kk] (entry kk is the current token)."""
    lib = _load()
    Sc, qk, k, v, beta, g = _f64(Sc), _f64(qk), _f64(k), _f64(v), _f64(beta), _f64(g)
    kk, dk = k.shape
    dv = v.shape[1]
    o = np.zeros(dv)
    lib.orc_gdn_replay_output(dv, dk, kk, ctypes.c_double(scale), _d(Sc), _d(qk), _d(k), _d(v),
                              _d(beta), _d(g), _d(o))
    return o


def replay_query(qk, k, v, beta, g, kda: bool = False):
    """The query vector r [dk] of the GDN (KDA: per-channel decay) replay form for one head: qk
    [dk], entries k [kk][dk], v [kk][dv], beta [kk], g [kk] (KDA [kk][dk]). The output is
    scale (Sc r + acc), so replacing the checkpoint Sc by Sc + E changes output p by exactly
    scale * (E r)[p]."""
    lib = _load()
    qk, k, v, beta, g = _f64(qk), _f64(k), _f64(v), _f64(beta), _f64(g)
    kk, dk = k.shape
    dv = v.shape[1]
    r = np.zeros(dk)
    lib.orc_replay_query(dv, dk, kk, 1 if kda else 0, _d(qk), _d(k), _d(v), _d(beta), _d(g),
                         _d(r))
    return r


def gdn_flush(Sc, k, v, beta, g):
    """GDN flush (UT/WY form) for one head: fold entries k [L][dk], v [L][dv], beta/g [L]."""
    lib = _load()
    Sc, k, v, beta, g = _f64(Sc), _f64(k), _f64(v), _f64(beta), _f64(g)
    L, dk = k.shape
    dv = v.shape[1]
    out = np.zeros((dv, dk))
    lib.orc_gdn_flush(dv, dk, L, _d(Sc), _d(k), _d(v), _d(beta), _d(g), _d(out))
    return out


def _declare(lib):
    i, d = ctypes.c_int, ctypes.c_double
    lib.orc_set_threads.argtypes = [i]
    lib.orc_m2_sequential.argtypes = [i, i, i, d, d] + [_dp] * 7 + [i, _ip, _dp]
    lib.orc_m2_sequential_batch.argtypes = [i, i, i, i] + [_dp] * 9 + [i, _ip, _dp]
    lib.orc_m2_replay_output.argtypes = [i, i, i, d, d] + [_dp] * 6
    lib.orc_m2_flush.argtypes = [i, i, i, d] + [_dp] * 5
    lib.orc_m2_spec_rounds_batch.argtypes = ([i] * 5 + [_dp] * 7 + [_ip, _dp, _dp, i, _ip, _dp])
    lib.orc_gdn_sequential_batch.argtypes = [i, i, i, i, d] + [_dp] * 8 + [i, _ip, _dp]
    lib.orc_gdn_replay_output.argtypes = [i, i, i, d] + [_dp] * 7
    lib.orc_gdn_flush.argtypes = [i, i, i] + [_dp] * 6
    lib.orc_gdn_spec_rounds_batch.argtypes = ([i, i, i, i, i, d] + [_dp] * 6 +
                                              [_ip, _dp, _dp, i, _ip, _dp])
    lib.orc_kda_sequential_batch.argtypes = [i, i, i, i, d] + [_dp] * 8 + [i, _ip, _dp]
    lib.orc_kda_replay_output.argtypes = [i, i, i, d] + [_dp] * 7
    lib.orc_replay_query.argtypes = [i, i, i, i] + [_dp] * 6
    lib.orc_kda_spec_rounds_batch.argtypes = ([i, i, i, i, i, d] + [_dp] * 6 +
                                              [_ip, _dp, _dp, i, _ip, _dp])
    for f in ("orc_m2_sequential", "orc_m2_sequential_batch", "orc_m2_replay_output",
              "orc_m2_flush", "orc_m2_spec_rounds_batch", "orc_gdn_sequential_batch",
              "orc_gdn_replay_output", "orc_gdn_flush", "orc_gdn_spec_rounds_batch",
              "orc_kda_sequential_batch", "orc_kda_replay_output", "orc_kda_spec_rounds_batch",
              "orc_replay_query"):
        getattr(lib, f).restype = None
