"""Pins of the CPU oracle to facts other than itself (closed forms, special cases, exact rational
unrolling). A plausible slip in the oracle -- a dropped D term, the output read from the state
before the update, a wrong sign on A, B and C swapped, a wrong head-to-group map, the GDN
correction applied from the left -- fails at least one of these.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from oracle import gdn_step, m2_step, normwise_err, token


def _m2_case(P=3, N=4, H=2, G=1, B=1, T=8, seed=7):
    sh = wl.M2Shape(batch=B, nheads=H, ngroups=G, head_dim=P, d_state=N, window=4)
    prm = wl.m2_params(sh, seed)
    s0 = wl.m2_state0(sh, seed)
    ins = wl.m2_token_inputs(sh, seed, 0, ntok=T)
    return sh, prm, s0, ins


def _run_m2(prm, s0, ins):
    st = s0.astype(np.float64).copy()
    ys = [m2_step(prm["A"], prm["D"], *(token(ins, t)[k] for k in ("x", "B", "C", "dt")), st)
          for t in range(ins["x"].shape[0])]
    return np.stack(ys), st


# ---------------------------------------------------------------- Mamba-2: exact unrolled sum

def _exact_m2(prm, s0, ins, hpg):
    """Closed form of the recurrence, in exact rationals:
    h_t = (prod_{i<=t} a_i) h_0 + sum_{j<=t} (prod_{j<i<=t} a_i) dt_j x_j B_j^T,
    y_t = h_t C_t + D x_t, a_i = exp(dt_i A) (the double value, as the oracle uses)."""
    T, B, H, P = ins["x"].shape
    N = ins["B"].shape[-1]
    F = Fraction
    out = np.zeros((T, B, H, P))
    for b in range(B):
        for h in range(H):
            g = h // hpg
            A = float(prm["A"][h])
            a = [F(math.exp(float(ins["dt"][t, b, h]) * A)) for t in range(T)]
            for t in range(T):
                dec0 = F(1)
                for i in range(t + 1):
                    dec0 *= a[i]
                for p in range(P):
                    acc = F(0)
                    for n in range(N):
                        hv = dec0 * F(float(s0[b, h, p, n]))
                        for j in range(t + 1):
                            dj = F(1)
                            for i in range(j + 1, t + 1):
                                dj *= a[i]
                            hv += dj * F(float(ins["dt"][j, b, h])) * F(float(ins["x"][j, b, h, p])) \
                                * F(float(ins["B"][j, b, g, n]))
                        acc += hv * F(float(ins["C"][t, b, g, n]))
                    acc += F(float(prm["D"][h])) * F(float(ins["x"][t, b, h, p]))
                    out[t, b, h, p] = float(acc)
    return out


@pytest.mark.parametrize("H,G", [(2, 1), (2, 2)])
def test_m2_exact_unroll(oracle_lib, H, G):
    sh, prm, s0, ins = _m2_case(H=H, G=G, T=7)
    ys, _ = _run_m2(prm, s0, ins)
    ref = _exact_m2(prm, s0, ins, H // G)
    assert normwise_err(ys, ref) < 1e-13


def test_m2_exact_unroll_detects_group_map(oracle_lib):
    # the closed form with a wrong head->group map must disagree: guards the pin itself
    sh, prm, s0, ins = _m2_case(H=2, G=2, T=3)
    ys, _ = _run_m2(prm, s0, ins)
    ins_sw = dict(ins)
    ins_sw["B"] = ins["B"][:, :, ::-1].copy()
    ins_sw["C"] = ins["C"][:, :, ::-1].copy()
    assert normwise_err(ys, _exact_m2(prm, s0, ins_sw, 1)) > 1e-3


# ---------------------------------------------------------------- Mamba-2: special cases

def test_m2_dt_zero_is_checkpoint_gemv(oracle_lib):
    sh, prm, s0, ins = _m2_case(P=16, N=16, H=4, G=4, B=2, T=5)
    ins["dt"][:] = 0.0
    ys, st = _run_m2(prm, s0, ins)
    s64 = s0.astype(np.float64)
    for t in range(5):
        ref = np.einsum("bhpn,bhn->bhp", s64, ins["C"][t].astype(np.float64)) \
            + prm["D"].astype(np.float64)[None, :, None] * ins["x"][t]
        assert normwise_err(ys[t], ref) < 1e-14
    assert np.array_equal(st, s64)


def test_m2_zero_input_is_pure_decay(oracle_lib):
    sh, prm, s0, ins = _m2_case(P=16, N=16, H=4, G=4, B=2, T=6)
    ins["x"][:] = 0.0
    ys, _ = _run_m2(prm, s0, ins)
    lam = np.ones((2, 4))
    for t in range(6):
        lam = lam * np.exp(ins["dt"][t].astype(np.float64) * prm["A"].astype(np.float64)[None])
        ref = lam[..., None] * np.einsum("bhpn,bhn->bhp", s0.astype(np.float64),
                                         ins["C"][t].astype(np.float64))
        assert normwise_err(ys[t], ref) < 1e-13


def test_m2_no_decay_is_one_matmul(oracle_lib):
    sh, prm, s0, ins = _m2_case(P=16, N=16, H=4, G=2, B=2, T=9)
    prm = dict(prm)
    prm["A"] = np.zeros_like(prm["A"])
    _, st = _run_m2(prm, s0, ins)
    for b in range(2):
        for h in range(4):
            g = h // 2
            X = ins["x"][:, b, h].astype(np.float64) * ins["dt"][:, b, h, None]
            ref = s0[b, h].astype(np.float64) + X.T @ ins["B"][:, b, g].astype(np.float64)
            assert np.max(np.abs(st[b, h] - ref)) < 1e-13


def test_m2_linearity(oracle_lib):
    sh, prm, s0, ins = _m2_case(P=16, N=16, H=4, G=4, B=2, T=6)
    y_full, _ = _run_m2(prm, s0, ins)
    ins0 = dict(ins)
    ins0["x"] = np.zeros_like(ins["x"])
    y_h0, _ = _run_m2(prm, s0, ins0)
    y_x, _ = _run_m2(prm, np.zeros_like(s0), ins)
    assert normwise_err(y_full, y_h0 + y_x) < 1e-13


def test_m2_single_step_post_update(oracle_lib):
    # one step by hand: a = exp(dt A), h1 = a h0 + dt x B^T, y = h1 C + D x
    sh, prm, s0, ins = _m2_case(P=5, N=6, H=3, G=3, B=1, T=1)
    ys, st = _run_m2(prm, s0, ins)
    for h in range(3):
        a = math.exp(float(ins["dt"][0, 0, h]) * float(prm["A"][h]))
        x = ins["x"][0, 0, h].astype(np.float64)
        h1 = a * s0[0, h].astype(np.float64) + float(ins["dt"][0, 0, h]) * np.outer(
            x, ins["B"][0, 0, h].astype(np.float64))
        y = h1 @ ins["C"][0, 0, h].astype(np.float64) + float(prm["D"][h]) * x
        assert np.max(np.abs(st[0, h] - h1)) < 1e-15
        assert np.max(np.abs(ys[0, 0, h] - y)) < 1e-14


# ---------------------------------------------------------------- Gated DeltaNet

def _gdn_case(d=8, H=2, B=2, T=6, seed=3):
    sh = wl.GDNShape(batch=B, nheads=H, d_k=d, d_v=d, window=4)
    return sh, wl.gdn_state0(sh, seed), wl.gdn_token_inputs(sh, seed, 0, ntok=T)


def _run_gdn(s0, ins):
    st = s0.astype(np.float64).copy()
    os_ = [gdn_step(*(token(ins, t)[k] for k in ("q", "k", "v", "beta", "alpha")), st)
           for t in range(ins["q"].shape[0])]
    return np.stack(os_), st


def test_gdn_no_write_is_gemv(oracle_lib):
    sh, s0, ins = _gdn_case()
    ins["alpha"][:] = 1.0
    ins["beta"][:] = 0.0
    os_, st = _run_gdn(s0, ins)
    for t in range(ins["q"].shape[0]):
        ref = np.einsum("bhij,bhj->bhi", s0.astype(np.float64), ins["q"][t].astype(np.float64))
        assert normwise_err(os_[t], ref) < 1e-14
    assert np.array_equal(st, s0.astype(np.float64))


def test_gdn_unit_key_overwrites_one_column(oracle_lib):
    sh, s0, ins = _gdn_case(T=1)
    ins["alpha"][:] = 1.0
    ins["beta"][:] = 1.0
    ins["k"][:] = 0.0
    cols = [3, 5]
    for h, c in enumerate(cols):
        ins["k"][0, :, h, c] = 1.0
    os_, st = _run_gdn(s0, ins)
    for b in range(2):
        for h, c in enumerate(cols):
            ref = s0[b, h].astype(np.float64).copy()
            ref[:, c] = ins["v"][0, b, h]
            assert np.array_equal(st[b, h], ref)
            assert np.max(np.abs(os_[0, b, h] - ref @ ins["q"][0, b, h].astype(np.float64))) < 1e-14


def test_gdn_reflection_keeps_norm(oracle_lib):
    sh, s0, ins = _gdn_case(T=5)
    ins["alpha"][:] = 1.0
    ins["beta"][:] = 2.0
    ins["v"][:] = 0.0
    _, st = _run_gdn(s0, ins)
    k64 = ins["k"].astype(np.float64)
    # k is unit length only to fp32 rounding; the exact invariant is for a unit k, so allow that
    dev = np.max(np.abs(np.sum(k64 * k64, axis=-1) - 1.0))
    n0 = np.linalg.norm(s0.astype(np.float64), axis=(-2, -1))
    n1 = np.linalg.norm(st, axis=(-2, -1))
    assert np.max(np.abs(n1 / n0 - 1.0)) < 20 * dev + 1e-13


def test_gdn_exact_product_form(oracle_lib):
    """S_T = S_0 M_1..M_T + sum_t beta_t v_t k_t^T M_{t+1}..M_T with
    M_t = alpha_t (I - beta_t k_t k_t^T), evaluated as explicit matrix products in exact rationals."""
    sh, s0, ins = _gdn_case(d=3, H=1, B=1, T=5)
    os_, st = _run_gdn(s0, ins)
    F = Fraction
    d, T = 3, 5

    def mat(a):
        return [[F(float(v)) for v in row] for row in a]

    def mm(X, Y):
        return [[sum(X[i][k] * Y[k][j] for k in range(len(Y))) for j in range(len(Y[0]))]
                for i in range(len(X))]

    def Mt(t):
        k = [F(float(v)) for v in ins["k"][t, 0, 0]]
        be, al = F(float(ins["beta"][t, 0, 0])), F(float(ins["alpha"][t, 0, 0]))
        return [[al * ((1 if i == j else 0) - be * k[i] * k[j]) for j in range(d)] for i in range(d)]

    Ms = [Mt(t) for t in range(T)]
    for tt in range(T):
        S = mat(s0[0, 0])
        for t in range(tt + 1):
            S = mm(S, Ms[t])
        for t in range(tt + 1):
            k = [F(float(v)) for v in ins["k"][t, 0, 0]]
            v = [F(float(v)) for v in ins["v"][t, 0, 0]]
            be = F(float(ins["beta"][t, 0, 0]))
            R = [[be * v[i] * k[j] for j in range(d)] for i in range(d)]
            for u in range(t + 1, tt + 1):
                R = mm(R, Ms[u])
            S = [[S[i][j] + R[i][j] for j in range(d)] for i in range(d)]
        q = [F(float(v)) for v in ins["q"][tt, 0, 0]]
        o = np.array([float(sum(S[i][j] * q[j] for j in range(d))) for i in range(d)])
        assert normwise_err(os_[tt, 0, 0], o) < 1e-13
    assert np.max(np.abs(st[0, 0] - np.array([[float(v) for v in r] for r in S]))) < 1e-13


def test_batch_permutation_equivariance(oracle_lib):
    sh, prm, s0, ins = _m2_case(P=8, N=8, H=2, G=2, B=3, T=3)
    perm = [2, 0, 1]
    ys, _ = _run_m2(prm, s0, ins)
    insp = {k: v[:, perm].copy() for k, v in ins.items()}
    ysp, _ = _run_m2(prm, s0[perm].copy(), insp)
    assert np.array_equal(ys[:, perm], ysp)
