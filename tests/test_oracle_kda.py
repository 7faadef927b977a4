"""Pins of the Kimi Delta Attention oracle (a per key channel forget gate in the Gated DeltaNet
delta rule; the pages name the layer type without a formula) to facts other than itself: the
Gated DeltaNet step it reduces to with a uniform gate, exact rational unrolling of its product
form, special cases that reduce to a GEMV or to masking key channels; and of the replay model
(checkpoint + ring) to the conventional recurrence."""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from oracle import (KDAReplay, kda_kappa_step, kda_spec_round, kda_step, gdn_step,
                    normwise_err, token)


def _dyadic(rng, shape, den):
    return (rng.integers(-4, 5, size=shape) / den).astype(np.float32)


def test_kda_uniform_gate_is_gdn_bit_exact(oracle_lib):
    """Every channel gated alike by alpha: the Gated DeltaNet step. On dyadic inputs both are exact
    in fp64, so they agree bit for bit; on random inputs to rounding."""
    rng = np.random.default_rng(0)
    B, H, d = 2, 3, 4
    S = _dyadic(rng, (B, H, d, d), 8).astype(np.float64)
    S2 = S.copy()
    for t in range(6):
        q = _dyadic(rng, (B, H, d), 4)
        k = (rng.choice([-0.5, 0.5], size=(B, H, d))).astype(np.float32)    # unit norm at d = 4
        v = _dyadic(rng, (B, H, d), 2)
        beta = np.full((B, H), 0.5, np.float32)
        al = np.full((B, H), 0.5, np.float32)
        o1 = kda_step(q, k, v, beta, np.repeat(al[..., None], d, axis=-1), S)
        o2 = gdn_step(q, k, v, beta, al, S2)
        assert np.array_equal(o1, o2) and np.array_equal(S, S2), t
    sh = wl.GDNShape(batch=2, nheads=3, d_k=8, d_v=6, window=4)
    ins = wl.gdn_token_inputs(sh, 3, 0, ntok=10)
    S = wl.gdn_state0(sh, 3).astype(np.float64)
    S2 = S.copy()
    for t in range(10):
        tk = token(ins, t)
        a = np.repeat(tk["alpha"][..., None], sh.d_k, axis=-1)
        o1 = kda_step(tk["q"], tk["k"], tk["v"], tk["beta"], a, S)
        o2 = gdn_step(tk["q"], tk["k"], tk["v"], tk["beta"], tk["alpha"], S2)
        assert normwise_err(o1, o2) < 1e-14 and normwise_err(S, S2) < 1e-14, t


def _exact_kda(S0, ins, T):
    """S_t = S_0 M_1 ... M_t + sum_{j<=t} beta_j v_j k_j^T M_{j+1} ... M_t with
    M_i = diag(a_i) (I - beta_i k_i k_i^T), o_t = S_t q_t, in exact rationals (one (b, h))."""
    F = Fraction
    dv, dk = S0.shape

    def mat(rows):
        return [[F(float(x)) for x in r] for r in rows]

    def mul(X, Y):
        return [[sum(X[i][l] * Y[l][j] for l in range(len(Y))) for j in range(len(Y[0]))]
                for i in range(len(X))]

    def Mi(t):
        a = [F(float(x)) for x in ins["alpha"][t]]
        k = [F(float(x)) for x in ins["k"][t]]
        be = F(float(ins["beta"][t]))
        return [[a[i] * ((1 if i == j else 0) - be * k[i] * k[j]) for j in range(dk)] for i in range(dk)]

    outs = []
    S0f = mat(S0)
    for t in range(T):
        S = S0f
        for i in range(t + 1):
            S = mul(S, Mi(i))
        for j in range(t + 1):
            be = F(float(ins["beta"][j]))
            v = [F(float(x)) for x in ins["v"][j]]
            k = [F(float(x)) for x in ins["k"][j]]
            R = [[be * v[i] * k[c] for c in range(dk)] for i in range(dv)]
            for i in range(j + 1, t + 1):
                R = mul(R, Mi(i))
            S = [[S[i][c] + R[i][c] for c in range(dk)] for i in range(dv)]
        q = [F(float(x)) for x in ins["q"][t]]
        outs.append([float(sum(S[i][c] * q[c] for c in range(dk))) for i in range(dv)])
    return np.array(outs)


def test_kda_exact_rational_unroll(oracle_lib):
    sh = wl.GDNShape(batch=1, nheads=1, d_k=3, d_v=3, window=4)
    T = 6
    ins = wl.kda_token_inputs(sh, 5, 0, ntok=T)
    s0 = wl.kda_state0(sh, 5)
    S = s0.astype(np.float64)
    got = np.stack([kda_step(*(token(ins, t)[k] for k in ("q", "k", "v", "beta", "alpha")), S)
                    for t in range(T)])[:, 0, 0]
    one = {k: v[:, 0, 0] for k, v in ins.items()}
    ref = _exact_kda(s0[0, 0], one, T)
    assert normwise_err(got, ref) < 1e-14
    # the same closed form with the gate applied to the value channels (rows) must disagree
    bad = dict(one)
    S = s0.astype(np.float64)
    wrong = []
    for t in range(T):
        tk = token(ins, t)
        S *= tk["alpha"][0, 0][:, None]                    # rows scaled instead of columns
        wrong.append(gdn_step(tk["q"], tk["k"], tk["v"], tk["beta"], np.ones((1, 1), np.float32),
                              S)[0, 0])
    assert normwise_err(np.stack(wrong), ref) > 1e-3


def test_kda_no_write_no_decay_is_gemv(oracle_lib):
    sh = wl.GDNShape(batch=2, nheads=2, d_k=8, d_v=5, window=4)
    ins = token(wl.kda_token_inputs(sh, 6, 0), 0)
    S = wl.kda_state0(sh, 6).astype(np.float64)
    S_before = S.copy()
    o = kda_step(ins["q"], ins["k"], ins["v"], np.zeros((2, 2), np.float32),
                 np.ones((2, 2, 8), np.float32), S)
    assert np.array_equal(S, S_before)
    assert normwise_err(o, np.einsum("bhij,bhj->bhi", S_before, ins["q"].astype(np.float64))) < 1e-15


def test_kda_gate_masks_key_channels(oracle_lib):
    """beta = 0 and a gate of 1 on some key channels and 0 on the others: the state keeps exactly
    its columns of the open channels, the output sums over them only."""
    sh = wl.GDNShape(batch=1, nheads=2, d_k=6, d_v=4, window=4)
    ins = token(wl.kda_token_inputs(sh, 7, 0), 0)
    S = wl.kda_state0(sh, 7).astype(np.float64)
    S_before = S.copy()
    mask = np.array([1, 0, 1, 1, 0, 0], np.float32)
    o = kda_step(ins["q"], ins["k"], ins["v"], np.zeros((1, 2), np.float32),
                 np.broadcast_to(mask, (1, 2, 6)).copy(), S)
    assert np.array_equal(S, S_before * mask)
    want = np.einsum("bhij,bhj->bhi", S_before * mask, ins["q"].astype(np.float64))
    assert normwise_err(o, want) < 1e-15


def test_kda_closed_gate_overwrite(oracle_lib):
    """Gate 0 on every channel forgets the state: S = beta v k^T and o = beta (k . q) v."""
    sh = wl.GDNShape(batch=1, nheads=1, d_k=4, d_v=3, window=4)
    ins = token(wl.kda_token_inputs(sh, 8, 0), 0)
    S = wl.kda_state0(sh, 8).astype(np.float64)
    o = kda_step(ins["q"], ins["k"], ins["v"], ins["beta"], np.zeros((1, 1, 4), np.float32), S)
    be = float(ins["beta"][0, 0])
    k = ins["k"][0, 0].astype(np.float64)
    v = ins["v"][0, 0].astype(np.float64)
    assert np.array_equal(S[0, 0], be * np.outer(v, k) - 0.0)
    assert normwise_err(o[0, 0], be * float(k @ ins["q"][0, 0].astype(np.float64)) * v) < 1e-15


def test_kda_kappa_pins(oracle_lib):
    rng = np.random.default_rng(3)
    B, H, d = 1, 2, 5
    S = np.abs(rng.standard_normal((B, H, d, d)))
    q = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
    k = rng.standard_normal((B, H, d)).astype(np.float32)
    v = rng.standard_normal((B, H, d)).astype(np.float32)
    a = rng.uniform(0.2, 1.0, size=(B, H, d)).astype(np.float32)
    zero = np.zeros((B, H), np.float32)
    st, M = S.copy(), S.copy()
    assert np.array_equal(kda_step(q, k, v, zero, a, st), kda_kappa_step(q, k, v, zero, a, M))
    assert np.array_equal(st, M)
    sh = wl.GDNShape(batch=2, nheads=3, d_k=8, d_v=8, window=4)
    s0 = wl.kda_state0(sh, 1).astype(np.float64)
    ins = wl.kda_token_inputs(sh, 1, 0, ntok=12)
    M = np.abs(s0)
    for t in range(12):
        args = [ins[kk][t] for kk in ("q", "k", "v", "beta", "alpha")]
        o = kda_step(*args, s0)
        kap = kda_kappa_step(*args, M)
        assert np.all(np.abs(o) <= kap * (1 + 1e-12)), t


# ------------------------------------------------------------------ replay model vs conventional

@pytest.mark.parametrize("W", [1, 4, 16])
def test_kda_replay_equals_conventional(oracle_lib, W):
    sh = wl.GDNShape(batch=2, nheads=2, d_k=8, d_v=6, window=W)
    s0 = wl.kda_state0(sh, 2)
    T = 40
    ins = wl.kda_token_inputs(sh, 2, 0, ntok=T)
    rp = KDAReplay(s0, W)
    S = s0.astype(np.float64)
    for t in range(T):
        tk = token(ins, t)
        o = rp.decode(tk)
        ref = kda_step(tk["q"], tk["k"], tk["v"], tk["beta"], tk["alpha"], S)
        assert normwise_err(o, ref) < 1e-12, t
        assert normwise_err(rp.materialize(), S) < 1e-12, t


@pytest.mark.parametrize("W,K", [(8, 3), (16, 6), (4, 4)])
def test_kda_spec_rounds_equal_recompute(oracle_lib, W, K):
    sh = wl.GDNShape(batch=3, nheads=2, d_k=8, d_v=4, window=W, max_draft=K)
    s0 = wl.kda_state0(sh, 4)
    rp = KDAReplay(s0, W, K)
    S = s0.astype(np.float64)
    acc = wl.spec_accepted(sh.batch, 12, K, seed=4)
    for r in range(12):
        dr = wl.kda_token_inputs(sh, 4, 10 + r, ntok=K)
        o = rp.verify(dr)
        if r % 5 == 4:
            rp.rollback(rp.bk.len.copy())
            ref = kda_spec_round(dr, S, np.zeros(sh.batch, np.int32))
        else:
            rp.commit(acc[r])
            ref = kda_spec_round(dr, S, acc[r])
        assert normwise_err(o, ref) < 1e-12, r
        assert normwise_err(rp.materialize(), S) < 1e-12, r
        if r % 3 == 1:
            tk = token(wl.kda_token_inputs(sh, 4, 100 + r), 0)
            o1 = rp.decode(tk)
            assert normwise_err(o1, kda_step(tk["q"], tk["k"], tk["v"], tk["beta"], tk["alpha"], S)) < 1e-12
