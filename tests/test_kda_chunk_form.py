"""The chunk form that the Kimi Delta Attention prefill and fold compute on the matrix cores, written
out in fp64 numpy and checked against the oracle's recurrence (oracle.kda_step, the reading
S <- S diag(a) (I - beta k k^T) + beta v k^T, o = S q): every token's output and the state after
every chunk. This pins the algebra of the chunk form (the gate ratios split over the two operands
of A and M, the WY factor T taken over A, the output and end-of-chunk formulas), not the kernels,
which the GPU tests compare with the oracle directly."""
import numpy as np
import pytest

import workloads as wl
from oracle import kda_step

CHUNK = 16


def _chunk(q, k, v, beta, a, S):
    """n <= 16 tokens of one (b, h) pair in the chunk form; S [dv, dk] float64, updated in place.
    Returns the outputs [n, dv]."""
    n = q.shape[0]
    gam = np.cumprod(a, axis=0)                  # Gam_t = a_0 o ... o a_t, per key channel
    kh, kt, qh = k * gam, k / gam, q * gam
    A = kh @ kt.T                                # A[t][j] = kh_t . kt_j (used for j < t)
    T = np.zeros((n, n))
    for t in range(n):                           # T[t][t] = beta_t,
        for c in range(t + 1):                   # T[t][c] = -beta_t sum_{c<=i<t} A[t][i] T[i][c]
            acc = sum(A[t, i] * T[i, c] for i in range(c, t))
            T[t, c] = beta[t] * ((1.0 if t == c else 0.0) - acc)
    Z = v - kh @ S.T                             # Z[q] = v_q - S kh_q
    U = T @ Z
    M = np.tril(qh @ kt.T)                       # M[t][j] = qh_t . kt_j for j <= t, else 0
    O = qh @ S.T + M @ U
    S[:] = (S + U.T @ kt) * gam[-1]              # (S + U^T Kt) diag(Gam_{n-1})
    return O


@pytest.mark.parametrize("d,T,gate", [(16, 40, None), (32, 16, None), (16, 37, 0.07), (8, 21, 0.9)])
def test_chunk_form_matches_recurrence(d, T, gate):
    """Random prompts (the KDA input recipe, or every gate set to `gate`), chunks of 16 and a
    ragged last chunk: outputs and chunk-end states equal the recurrence to fp64 rounding."""
    sh = wl.GDNShape(batch=1, nheads=2, d_k=d, d_v=d, window=16)
    ins = wl.kda_token_inputs(sh, 3, 0, ntok=T)
    if gate is not None:
        ins["alpha"][:] = np.float32(gate)
    s0 = wl.kda_state0(sh, 3).astype(np.float64)
    ref = s0.copy()
    o_ref = np.stack([kda_step(*(ins[x][t] for x in ("q", "k", "v", "beta", "alpha")), ref)
                      for t in range(T)])
    f = {x: ins[x].astype(np.float64) for x in ins}
    for h in range(sh.nheads):
        S = s0[0, h].copy()
        states = s0[0, h].copy()
        r = s0[0:1, h:h + 1].copy()
        for t0 in range(0, T, CHUNK):
            t1 = min(T, t0 + CHUNK)
            O = _chunk(f["q"][t0:t1, 0, h], f["k"][t0:t1, 0, h], f["v"][t0:t1, 0, h],
                       f["beta"][t0:t1, 0, h], f["alpha"][t0:t1, 0, h], S)
            scale = np.max(np.abs(o_ref[t0:t1, 0, h]))
            assert np.max(np.abs(O - o_ref[t0:t1, 0, h])) <= 1e-11 * scale, (h, t0)
            for t in range(t0, t1):         # the recurrence's state at the chunk's end
                kda_step(*(ins[x][t][0:1, h:h + 1] for x in ("q", "k", "v", "beta", "alpha")), r)
            states = r[0, 0]
            assert np.max(np.abs(S - states)) <= 1e-11 * np.max(np.abs(states)), (h, t0)


def test_single_token_chunk_is_the_step():
    """One token: the chunk form reduces to S diag(a) + beta (v - S (a o k)) k^T and o = S q."""
    rng = np.random.default_rng(0)
    d = 8
    q, k, v = rng.standard_normal((3, 1, d))
    a = rng.uniform(0.2, 1.0, (1, d))
    beta = np.array([0.7])
    S = rng.standard_normal((d, d))
    S0 = S.copy()
    O = _chunk(q, k, v, beta, a, S)
    Sa = S0 * a[0]
    want = Sa + beta[0] * np.outer(v[0] - Sa @ k[0], k[0])
    np.testing.assert_allclose(S, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O[0], want @ q[0], rtol=1e-13, atol=1e-13)
