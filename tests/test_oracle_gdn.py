"""Pins of the fp64 Gated DeltaNet oracle (CPU only).

Closed forms and invariants of the gated delta rule that a slip would break: pure decay when
beta = 0 (a wrong gate), the delta rule writing the value exactly along a unit key (a wrong sign
or a missing alpha inside the correction), a Householder reflection preserving the Frobenius norm
(beta = 2), and orthonormal keys reducing the state to a plain sum of outer products. The replay
(backward sweep) and UT/WY flush forms are then tied to the sequential recurrence in fp64.
"""
import numpy as np
import pytest
import scipy.stats

import oracle


def _unit(rng, shape):
    v = rng.standard_normal(shape)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _rand_gdn(rng, nh, T, dv, dk):
    S0 = rng.standard_normal((nh, dv, dk)) * np.sqrt(0.1)
    q = _unit(rng, (nh, T, dk))
    k = _unit(rng, (nh, T, dk))
    v = rng.standard_normal((nh, T, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((nh, T))))
    g = -np.log1p(np.exp(rng.standard_normal((nh, T))))
    return S0, q, k, v, beta, g


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(1)
    S0, q, k, v, beta, g = _rand_gdn(rng, 2, 10, 5, 6)
    o, ST, _ = oracle.gdn_sequential(S0, q, k, v, np.zeros_like(beta), g)
    gam = np.exp(np.cumsum(g, axis=1))
    np.testing.assert_allclose(ST, gam[:, -1, None, None] * S0, rtol=1e-13)
    for t in range(10):
        np.testing.assert_allclose(o[:, t], gam[:, t, None] * np.einsum("hpn,hn->hp", S0, q[:, t]),
                                   rtol=1e-12, atol=1e-14)


def test_delta_rule_writes_the_value():
    # alpha = 1, beta = 1, unit k: S_t k_t = v_t exactly (the correction removes the old value)
    rng = np.random.default_rng(2)
    S0, q, k, v, beta, g = _rand_gdn(rng, 1, 8, 6, 7)
    T = 8
    _, _, snaps = oracle.gdn_sequential(S0, q, k, v, np.ones_like(beta), np.zeros_like(g),
                                        snap_after=list(range(1, T + 1)))
    for t in range(T):
        np.testing.assert_allclose(snaps[0, t] @ k[0, t], v[0, t], rtol=1e-12, atol=1e-13)


def test_householder_preserves_norm():
    # alpha = 1, beta = 2, unit k, v = 0: S_t = S_{t-1} (I - 2 k k^T) is a reflection
    rng = np.random.default_rng(3)
    S0, q, k, v, beta, g = _rand_gdn(rng, 2, 12, 5, 9)
    _, _, snaps = oracle.gdn_sequential(S0, q, k, np.zeros_like(v), np.full_like(beta, 2.0),
                                        np.zeros_like(g), snap_after=list(range(1, 13)))
    n0 = np.linalg.norm(S0, axis=(1, 2))
    for t in range(12):
        np.testing.assert_allclose(np.linalg.norm(snaps[:, t], axis=(1, 2)), n0, rtol=1e-12)


def test_orthonormal_keys_sum_of_outer_products():
    # alpha = 1, beta = 1, S0 = 0 and orthonormal keys: S_T = sum_t v_t k_t^T and
    # o_t = sum_{i<=t} v_i (k_i . q_t). Keys from a library QR.
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 5, 6
    Q = scipy.stats.ortho_group.rvs(dk, random_state=5)
    k = Q[:T][None]
    q = _unit(rng, (1, T, dk))
    v = rng.standard_normal((1, T, dv))
    o, ST, _ = oracle.gdn_sequential(None, q, k, v, np.ones((1, T)), np.zeros((1, T)))
    np.testing.assert_allclose(ST[0], v[0].T @ k[0], rtol=1e-12, atol=1e-13)
    for t in range(T):
        expect = sum(v[0, i] * (k[0, i] @ q[0, t]) for i in range(t + 1))
        np.testing.assert_allclose(o[0, t], expect, rtol=1e-12, atol=1e-13)


def test_scale_multiplies_output():
    rng = np.random.default_rng(6)
    S0, q, k, v, beta, g = _rand_gdn(rng, 1, 5, 4, 4)
    o1, _, _ = oracle.gdn_sequential(S0, q, k, v, beta, g, scale=1.0)
    o2, _, _ = oracle.gdn_sequential(S0, q, k, v, beta, g, scale=0.25)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-15)


@pytest.mark.parametrize("L", [1, 4, 16])
def test_replay_and_flush_identities(L):
    rng = np.random.default_rng(20 + L)
    T, dv, dk = 3 * L + 3, 6, 8
    S0, q, k, v, beta, g = _rand_gdn(rng, 1, T, dv, dk)
    o, _, snaps = oracle.gdn_sequential(S0, q, k, v, beta, g, snap_after=list(range(L, T + 1, L)))
    Sc = S0[0]
    c = 0
    for t in range(T):
        orp = oracle.gdn_replay_output(Sc, q[0, t], k[0, c:t + 1], v[0, c:t + 1],
                                       beta[0, c:t + 1], g[0, c:t + 1])
        np.testing.assert_allclose(orp, o[0, t], rtol=1e-12, atol=1e-12)
        if t + 1 - c == L:
            Sc = oracle.gdn_flush(Sc, k[0, c:t + 1], v[0, c:t + 1], beta[0, c:t + 1],
                                  g[0, c:t + 1])
            np.testing.assert_allclose(Sc, snaps[0, (t + 1) // L - 1], rtol=1e-11, atol=1e-12)
            c = t + 1


def test_spec_rounds_match_sequential_on_accepted_stream():
    # Committed state after speculative rounds equals sequential stepping over the accepted
    # drafts; every draft output equals a sequential run from the state committed before it.
    rng = np.random.default_rng(16)
    R, S, dv, dk = 6, 4, 5, 7
    S0, q, k, v, beta, g = _rand_gdn(rng, 1, R * S, dv, dk)
    acc = rng.integers(0, S + 1, size=(1, R))
    acc[0, 1] = 0  # a round that rejects every draft
    o, ST, _ = oracle.gdn_spec_rounds(S0, q.reshape(1, R, S, dk), k.reshape(1, R, S, dk),
                                      v.reshape(1, R, S, dv), beta.reshape(1, R, S),
                                      g.reshape(1, R, S), acc, scale=0.7)
    keep = np.concatenate([np.arange(r * S, r * S + acc[0, r]) for r in range(R)]).astype(int)
    _, Sseq, _ = oracle.gdn_sequential(S0, q[:, keep], k[:, keep], v[:, keep], beta[:, keep],
                                       g[:, keep], scale=0.7)
    np.testing.assert_allclose(ST, Sseq, rtol=1e-13, atol=1e-14)
    for r in (1, R - 1):
        prev = keep[keep < r * S]
        _, Sprev, _ = oracle.gdn_sequential(S0, q[:, prev], k[:, prev], v[:, prev],
                                            beta[:, prev], g[:, prev])
        sl = slice(r * S, (r + 1) * S)
        od, _, _ = oracle.gdn_sequential(Sprev, q[:, sl], k[:, sl], v[:, sl], beta[:, sl],
                                         g[:, sl], scale=0.7)
        np.testing.assert_allclose(o[0, r], od[0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_replay_query_is_the_checkpoint_read_vector(kda):
    """replay_query returns the r of o = scale (Sc r + acc): the output's change under a change E
    of the checkpoint is scale * E r (checked through replay_output, itself pinned to stepping);
    with no entries r = q; with beta = 0 it is q times the product of the decays."""
    rng = np.random.default_rng(7)
    dv, dk, kk = 12, 10, 6
    Sc = rng.standard_normal((dv, dk))
    q = rng.standard_normal(dk)
    k = rng.standard_normal((kk, dk))
    v = rng.standard_normal((kk, dv))
    beta = rng.random(kk)
    g = -rng.random((kk, dk)) if kda else -rng.random(kk)
    fo = oracle.kda_replay_output if kda else oracle.gdn_replay_output
    r = oracle.replay_query(q, k, v, beta, g, kda)
    E = rng.standard_normal((dv, dk)) * 1e-2
    d = fo(Sc + E, q, k, v, beta, g, 0.7) - fo(Sc, q, k, v, beta, g, 0.7)
    np.testing.assert_allclose(d, 0.7 * E @ r, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(oracle.replay_query(q, k[:0], v[:0], beta[:0], g[:0], kda), q)
    r0 = oracle.replay_query(q, k, v, np.zeros(kk), g, kda)
    decay = np.exp(g.sum(axis=0)) if kda else np.exp(g.sum())
    np.testing.assert_allclose(r0, q * decay, rtol=1e-14)
