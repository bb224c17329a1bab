"""Pins of the fp64 Mamba-2 oracle against things other than itself (CPU only).

Each pin would catch a plausible slip in the oracle: a dropped input term (first-token and
no-decay closed forms), a wrong decay exponent or off-by-one in the decay window (semiseparable
brute force, IIR filter), an output taken from the pre-update state (first-token form), and a
non-linear slip (superposition). The replay and flush forms are then tied to the sequential
recurrence to fp64 rounding.
"""
import numpy as np
import pytest
import scipy.signal

import oracle


def _rand_m2(rng, nh, T, P, N, h0=True):
    A = -np.exp(rng.uniform(0, 2, nh))
    D = rng.standard_normal(nh)
    x = rng.standard_normal((nh, T, P))
    B = rng.standard_normal((nh, T, N)) / np.sqrt(N)
    C = rng.standard_normal((nh, T, N)) / np.sqrt(N)
    dt = np.log1p(np.exp(rng.normal(-2, np.sqrt(0.5), (nh, T))))
    h = rng.standard_normal((nh, P, N)) * np.sqrt(0.1) if h0 else None
    return A, D, h, x, B, C, dt


def test_first_token_from_zero_state():
    # h_1 = dt x B^T from a zero state, so y_1 = dt (B . C) x + D x (output uses the updated state)
    rng = np.random.default_rng(1)
    A, D, _, x, B, C, dt = _rand_m2(rng, 3, 1, 5, 7, h0=False)
    y, _, _ = oracle.m2_sequential(A, D, None, x, B, C, dt)
    for i in range(3):
        expect = dt[i, 0] * (B[i, 0] @ C[i, 0]) * x[i, 0] + D[i] * x[i, 0]
        np.testing.assert_allclose(y[i, 0], expect, rtol=1e-14, atol=1e-15)


def test_no_decay_closed_form():
    # A = 0 (decay 1) and zero state: y_t = sum_{i<=t} dt_i (B_i . C_t) x_i + D x_t
    rng = np.random.default_rng(2)
    _, D, _, x, B, C, dt = _rand_m2(rng, 2, 9, 4, 6, h0=False)
    A = np.zeros(2)
    y, _, _ = oracle.m2_sequential(A, D, None, x, B, C, dt)
    for i in range(2):
        for t in range(9):
            expect = sum(dt[i, s] * (B[i, s] @ C[i, t]) * x[i, s] for s in range(t + 1))
            expect = expect + D[i] * x[i, t]
            np.testing.assert_allclose(y[i, t], expect, rtol=1e-12, atol=1e-13)


def _semiseparable(A, D, h0, x, B, C, dt):
    """Brute-force quadratic form of the unrolled recurrence for one head (T small)."""
    T, P = x.shape
    y = np.zeros((T, P))
    for t in range(T):
        y[t] = np.exp(A * dt[: t + 1].sum()) * (h0 @ C[t]) + D * x[t]
        for s in range(t + 1):
            y[t] += (C[t] @ B[s]) * np.exp(A * dt[s + 1: t + 1].sum()) * dt[s] * x[s]
    return y


@pytest.mark.parametrize("T,P,N", [(1, 3, 2), (17, 4, 8), (64, 16, 16)])
def test_semiseparable_brute_force(T, P, N):
    rng = np.random.default_rng(T)
    A, D, h0, x, B, C, dt = _rand_m2(rng, 2, T, P, N)
    y, _, _ = oracle.m2_sequential(A, D, h0, x, B, C, dt)
    for i in range(2):
        ref = _semiseparable(A[i], D[i], h0[i], x[i], B[i], C[i], dt[i])
        np.testing.assert_allclose(y[i], ref, rtol=1e-11, atol=1e-12)


def test_scalar_case_is_an_iir_filter():
    # P = N = 1 with constant dt, B, C: h_t = a h_{t-1} + dt B x_t is a first-order IIR filter,
    # y = (dt B C) / (1 - a z^-1) x + D x  (scipy.signal.lfilter).
    rng = np.random.default_rng(3)
    T = 200
    A, Dv, dtv, Bv, Cv = -0.7, 0.3, 0.25, 1.3, -0.8
    x = rng.standard_normal((1, T, 1))
    B = np.full((1, T, 1), Bv)
    C = np.full((1, T, 1), Cv)
    dt = np.full((1, T), dtv)
    y, _, _ = oracle.m2_sequential([A], [Dv], None, x, B, C, dt)
    a = np.exp(dtv * A)
    ref = scipy.signal.lfilter([dtv * Bv * Cv], [1.0, -a], x[0, :, 0]) + Dv * x[0, :, 0]
    np.testing.assert_allclose(y[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def test_superposition():
    # y(h0, x) = y(h0, 0) + y(0, x): the output is linear in (initial state, inputs)
    rng = np.random.default_rng(4)
    A, D, h0, x, B, C, dt = _rand_m2(rng, 2, 20, 8, 8)
    y, _, _ = oracle.m2_sequential(A, D, h0, x, B, C, dt)
    y0, _, _ = oracle.m2_sequential(A, D, h0, np.zeros_like(x), B, C, dt)
    yx, _, _ = oracle.m2_sequential(A, D, None, x, B, C, dt)
    np.testing.assert_allclose(y, y0 + yx, rtol=1e-12, atol=1e-13)


def test_snapshots_and_final_state():
    rng = np.random.default_rng(5)
    A, D, h0, x, B, C, dt = _rand_m2(rng, 2, 12, 4, 8)
    _, hT, snaps = oracle.m2_sequential(A, D, h0, x, B, C, dt, snap_after=[4, 12])
    _, h4, _ = oracle.m2_sequential(A, D, h0, x[:, :4], B[:, :4], C[:, :4], dt[:, :4])
    np.testing.assert_array_equal(snaps[:, 0], h4)
    np.testing.assert_array_equal(snaps[:, 1], hT)


@pytest.mark.parametrize("L", [1, 4, 16])
def test_replay_and_flush_identities(L):
    # Replay output == sequential output, and flushed checkpoint == sequential state, in fp64.
    rng = np.random.default_rng(10 + L)
    T, P, N = 3 * L + 2, 6, 10
    A, D, h0, x, B, C, dt = _rand_m2(rng, 1, T, P, N)
    y, _, snaps = oracle.m2_sequential(A, D, h0, x, B, C, dt,
                                       snap_after=list(range(L, T + 1, L)))
    hc = h0[0]
    c = 0  # checkpoint position
    for t in range(T):
        k = t + 1 - c
        yr = oracle.m2_replay_output(A[0], D[0], hc, x[0, c:t + 1], B[0, c:t + 1], C[0, t],
                                     dt[0, c:t + 1])
        np.testing.assert_allclose(yr, y[0, t], rtol=1e-12, atol=1e-12)
        if k == L:
            hc = oracle.m2_flush(A[0], hc, x[0, c:t + 1], B[0, c:t + 1], dt[0, c:t + 1])
            np.testing.assert_allclose(hc, snaps[0, (t + 1) // L - 1], rtol=1e-12, atol=1e-12)
            c = t + 1


def test_spec_rounds_match_sequential_on_accepted_stream():
    # Committed state after speculative rounds equals sequential stepping over the accepted
    # drafts; every draft output equals a sequential run from the committed state.
    rng = np.random.default_rng(6)
    R, S, P, N = 7, 4, 5, 6
    A, D, h0, x, B, C, dt = _rand_m2(rng, 1, R * S, P, N)
    acc = rng.integers(0, S + 1, size=(1, R))
    xs, Bs, Cs, dts = (x.reshape(1, R, S, P), B.reshape(1, R, S, N), C.reshape(1, R, S, N),
                       dt.reshape(1, R, S))
    y, hT, _ = oracle.m2_spec_rounds(A, D, h0, xs, Bs, Cs, dts, acc)
    keep = np.concatenate([np.arange(r * S, r * S + acc[0, r]) for r in range(R)]).astype(int)
    _, hseq, _ = oracle.m2_sequential(A, D, h0, x[:, keep], B[:, keep], C[:, keep], dt[:, keep])
    np.testing.assert_allclose(hT, hseq, rtol=1e-13, atol=1e-14)
    # last round's drafts from the state committed before it
    prev = keep[keep < (R - 1) * S]
    _, hprev, _ = oracle.m2_sequential(A, D, h0, x[:, prev], B[:, prev], C[:, prev], dt[:, prev])
    sl = slice((R - 1) * S, R * S)
    yd, _, _ = oracle.m2_sequential(A, D, hprev, x[:, sl], B[:, sl], C[:, sl], dt[:, sl])
    np.testing.assert_allclose(y[0, R - 1], yd[0], rtol=1e-13, atol=1e-14)
