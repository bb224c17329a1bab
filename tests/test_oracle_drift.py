"""The contrast behind the read copy (news article, para 4), on the CPU with the oracle.

A conventional state kept in fp8 feeds its own rounding back into every step, so its output
error compounds. The read copy is a rounded copy of an exact (here fp64) checkpoint that only the
outputs read: each window's outputs replay from the copy of that window's checkpoint, so the
error stays at one rounding of the state however long the run. This is a demonstration, not a
parity check: the GPU tests bound the copy's error per output.
"""
import numpy as np
import pytest

import oracle
from oracle import quant

P, N, L, T = 8, 16, 16, 512


def _run(seed, A=-0.02, h0_std=0.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, T, P))
    B = rng.standard_normal((1, T, N)) / np.sqrt(N)
    C = rng.standard_normal((1, T, N)) / np.sqrt(N)
    dt = np.log1p(np.exp(rng.standard_normal((1, T)) * np.sqrt(0.5) - 2.0))
    h0 = rng.standard_normal((1, P, N)) * h0_std
    Av, Dv = np.array([A]), np.array([0.5])
    y, _, snaps = oracle.m2_sequential(Av, Dv, h0, x, B, C, dt, snap_after=list(range(L, T, L)))
    y = y[0]

    def rounded(h):
        codes, s = quant.fp8_row_quantize(h.astype(np.float32))
        return quant.fp8_row_decode(codes, s).astype(np.float64)

    # a conventional recurrence whose state is stored in fp8 after every step
    h, y_state = h0[0].copy(), np.zeros((T, P))
    for t in range(T):
        h = rounded(np.exp(dt[0, t] * A) * h + dt[0, t] * np.outer(x[0, t], B[0, t]))
        y_state[t] = h @ C[0, t] + Dv[0] * x[0, t]
    # the read copy: exact checkpoint per window, outputs replayed from its rounded copy
    y_copy = np.zeros((T, P))
    for w in range(T // L):
        cp = rounded(h0[0] if w == 0 else snaps[0, w - 1])
        for j in range(L):
            t, s = w * L + j, slice(w * L, w * L + j + 1)
            y_copy[t] = oracle.m2_replay_output(A, Dv[0], cp, x[0, s], B[0, s], C[0, t], dt[0, s])

    def per_window(yy):  # mean |error| over each window, relative to that window's output rms
        e = np.abs(yy - y).reshape(T // L, L * P).mean(axis=1)
        return e / np.sqrt((y ** 2).reshape(T // L, L * P).mean(axis=1))

    return per_window(y_state), per_window(y_copy)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_fp8_state_compounds_but_the_read_copy_does_not(seed):
    e_state, e_copy = _run(seed)
    first, last = slice(0, 4), slice(-4, None)
    assert e_state[last].mean() >= 2.0 * e_state[first].mean(), e_state
    assert e_copy[last].mean() <= 1.3 * e_copy[first].mean(), e_copy
    assert e_copy[last].mean() <= e_state[last].mean() / 5, (e_copy, e_state)
