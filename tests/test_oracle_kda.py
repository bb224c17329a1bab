"""Pins of the fp64 Kimi Delta Attention oracle (CPU only).

KDA is the gated delta rule with one decay per key channel. Pins that a slip would break:
equal channel decays reduce it to the Gated DeltaNet oracle (a separate function); beta = 0 is
a pure column-wise decay with a closed form (a decay applied to the wrong axis breaks it); a unit
key along one channel with alpha = beta = 1 writes the value into exactly that column; the
channels decay independently (a broadcast slip mixes them). The replay form (backward sweep with
an elementwise decay) and the speculative rounds are then tied to the sequential recurrence.
"""
import numpy as np
import pytest

import oracle


def _unit(rng, shape):
    v = rng.standard_normal(shape)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _rand_kda(rng, nh, T, dv, dk):
    S0 = rng.standard_normal((nh, dv, dk)) * np.sqrt(0.1)
    q = _unit(rng, (nh, T, dk))
    k = _unit(rng, (nh, T, dk))
    v = rng.standard_normal((nh, T, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((nh, T))))
    g = -np.log1p(np.exp(rng.standard_normal((nh, T, dk))))
    return S0, q, k, v, beta, g


def test_equal_channel_decays_reduce_to_gdn():
    rng = np.random.default_rng(21)
    S0, q, k, v, beta, g = _rand_kda(rng, 2, 9, 5, 6)
    gs = g[..., 0]  # one decay per token, copied to every channel
    gv = np.repeat(gs[..., None], 6, axis=-1)
    ok, Sk, _ = oracle.kda_sequential(S0, q, k, v, beta, gv, scale=0.8)
    og, Sg, _ = oracle.gdn_sequential(S0, q, k, v, beta, gs, scale=0.8)
    np.testing.assert_allclose(ok, og, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sk, Sg, rtol=1e-13, atol=1e-14)


def test_beta_zero_is_columnwise_decay():
    rng = np.random.default_rng(22)
    S0, q, k, v, beta, g = _rand_kda(rng, 1, 7, 4, 5)
    beta[:] = 0.0
    o, ST, _ = oracle.kda_sequential(S0, q, k, v, beta, g)
    decay = np.exp(g[0].sum(axis=0))  # per key channel n
    np.testing.assert_allclose(ST[0], S0[0] * decay[None, :], rtol=1e-13)
    # each output is the decayed state times that token's query
    St = S0[0] * np.exp(g[0, :3].sum(axis=0))[None, :]
    np.testing.assert_allclose(o[0, 2], St @ q[0, 2], rtol=1e-12, atol=1e-14)


def test_unit_key_writes_one_column():
    dv, dk, j = 4, 6, 2
    S0 = np.arange(dv * dk, dtype=float).reshape(1, dv, dk) / 7.0
    k = np.zeros((1, 1, dk)); k[0, 0, j] = 1.0
    q = np.zeros((1, 1, dk)); q[0, 0, j] = 1.0
    v = np.array([[[1.5, -2.0, 0.25, 3.0]]])
    beta = np.ones((1, 1)); g = np.zeros((1, 1, dk))
    o, ST, _ = oracle.kda_sequential(S0, q, k, v, beta, g)
    exp = S0[0].copy(); exp[:, j] = v[0, 0]
    np.testing.assert_allclose(ST[0], exp, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-15)


def test_channels_decay_independently():
    # with beta = 0 and a decay on one channel only, every other column is untouched
    rng = np.random.default_rng(23)
    S0, q, k, v, beta, g = _rand_kda(rng, 1, 5, 3, 4)
    beta[:] = 0.0
    g[:] = 0.0
    g[0, :, 1] = -0.5
    _, ST, _ = oracle.kda_sequential(S0, q, k, v, beta, g)
    np.testing.assert_array_equal(ST[0][:, [0, 2, 3]], S0[0][:, [0, 2, 3]])
    np.testing.assert_allclose(ST[0][:, 1], S0[0][:, 1] * np.exp(-2.5), rtol=1e-14)


@pytest.mark.parametrize("L", [1, 4, 16])
def test_replay_identity(L):
    rng = np.random.default_rng(24 + L)
    S0, q, k, v, beta, g = _rand_kda(rng, 1, L, 5, 7)
    o, _, _ = oracle.kda_sequential(S0, q, k, v, beta, g, scale=0.6)
    for t in range(L):
        orep = oracle.kda_replay_output(S0[0], q[0, t], k[0, :t + 1], v[0, :t + 1], beta[0, :t + 1],
                                        g[0, :t + 1], scale=0.6)
        np.testing.assert_allclose(orep, o[0, t], rtol=1e-11, atol=1e-13)


def test_spec_rounds_match_sequential_on_accepted_stream():
    rng = np.random.default_rng(25)
    R, S, dv, dk = 5, 4, 4, 6
    S0, q, k, v, beta, g = _rand_kda(rng, 1, R * S, dv, dk)
    acc = rng.integers(0, S + 1, size=(1, R))
    o, ST, _ = oracle.kda_spec_rounds(S0, q.reshape(1, R, S, dk), k.reshape(1, R, S, dk),
                                      v.reshape(1, R, S, dv), beta.reshape(1, R, S),
                                      g.reshape(1, R, S, dk), acc)
    keep = np.concatenate([np.arange(r * S, r * S + acc[0, r]) for r in range(R)]).astype(int)
    _, Sseq, _ = oracle.kda_sequential(S0, q[:, keep], k[:, keep], v[:, keep], beta[:, keep],
                                       g[:, keep])
    np.testing.assert_allclose(ST, Sseq, rtol=1e-13, atol=1e-14)
    prev = keep[keep < (R - 1) * S]
    _, Sprev, _ = oracle.kda_sequential(S0, q[:, prev], k[:, prev], v[:, prev], beta[:, prev],
                                        g[:, prev])
    sl = slice((R - 1) * S, R * S)
    od, _, _ = oracle.kda_sequential(Sprev, q[:, sl], k[:, sl], v[:, sl], beta[:, sl], g[:, sl])
    np.testing.assert_allclose(o[0, R - 1], od[0], rtol=1e-13, atol=1e-14)
