"""Edge cases of the Mamba-2 replay path against the CPU oracle: every compiled head shape at the
smallest ring (W = 1: every token fills the ring and folds), an odd ring and the largest ring
(W = 32); speculative verify at K = W (the whole ring is drafts) and at W = 1."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import Bookkeeping, m2_spec_round, m2_step, normwise_err
from tests.gpu_helpers import dev, host, m2_dev_tokens, say

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2


def _ctx(sh, prm, bf16=False):
    c = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                   ngroups=sh.ngroups, max_draft=sh.max_draft, bf16_read=bf16)
    c.set_params(dev(prm["A"]), dev(prm["D"]))
    return c


def _check_bk(ctx, model):
    h, l, n, e = ctx.bookkeeping()
    mh, ml, mn = model.snapshot()
    assert (h, l, n, e) == (list(mh), list(ml), list(mn), 0), (h, l, n, e, mh, ml, mn)


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (64, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("W,bf16", [(1, False), (5, False), (32, False), (5, True)])
def test_decode_shapes_and_windows(P, N, W, bf16):
    """2 W + 3 decode steps: every output, the bookkeeping after every step and the materialised
    state at the end."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=2, head_dim=P, d_state=N, window=W)
    n = 2 * W + 3
    say(f"decode P={P} N={N} W={W} bf16={bf16}: {n} steps")
    prm = wl.m2_params(sh, 11)
    s0 = wl.m2_state0(sh, 11)
    ins = wl.m2_token_inputs(sh, 11, 0, ntok=n)
    d = m2_dev_tokens(sh, ins, n)
    ctx = _ctx(sh, prm, bf16)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W)
    ref = s0.astype(np.float64).copy()
    y = torch.empty(sh.batch, sh.nheads, P, device="cuda")
    tol = TOL_BF16 if bf16 else TOL
    for t in range(n):
        ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
        model.decode()
        yr = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        yh = host(y)
        err = normwise_err(yh.reshape(sh.batch, -1), yr.reshape(sh.batch, -1)) if bf16 else \
            normwise_err(yh, yr)
        assert err < tol, (t, err)
        _check_bk(ctx, model)
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL


@pytest.mark.parametrize("W,K", [(1, 1), (4, 4), (32, 6)])
def test_verify_ring_extremes(W, K):
    """Rounds of K drafts (all accepted, none accepted, seeded prefixes, a rollback), with decode
    steps between some rounds; K = W makes every round fold whatever the ring holds first."""
    sh = wl.M2Shape(batch=4, nheads=4, ngroups=2, head_dim=16, d_state=16, window=W, max_draft=K)
    say(f"verify W={W} K={K}")
    prm = wl.m2_params(sh, 12)
    s0 = wl.m2_state0(sh, 12)
    ctx = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W, K)
    ref = s0.astype(np.float64).copy()
    acc = wl.spec_accepted(sh.batch, 24, K, seed=12)
    yk = torch.empty(K, sh.batch, sh.nheads, 16, device="cuda")
    y = torch.empty(sh.batch, sh.nheads, 16, device="cuda")
    for r in range(24):
        ins = wl.m2_token_inputs(sh, 12, 300 + r, ntok=K)
        ctx.verify(yk, **m2_dev_tokens(sh, ins, K))
        model.verify(K)
        if r % 6 == 0:
            a = np.full(sh.batch, K, np.int32)           # every draft accepted
        elif r % 6 == 1:
            a = np.zeros(sh.batch, np.int32)              # none
        else:
            a = np.minimum(acc[r], K).astype(np.int32)
        if r % 6 == 5:
            a[:] = 0
            ctx.rollback(dev(np.array(model.len, dtype=np.int32)))
            model.rollback(model.len.copy())
        else:
            ctx.commit(dev(a))
            model.commit(a)
        yr = m2_spec_round(prm["A"], prm["D"], ins, ref, a)
        assert normwise_err(host(yk), yr) < TOL, r
        _check_bk(ctx, model)
        if r % 4 == 3:
            t = wl.m2_token_inputs(sh, 12, 700 + r)
            ctx.decode_step(y, **{k: v[0] for k, v in m2_dev_tokens(sh, t, 1).items()})
            model.decode()
            yr = m2_step(prm["A"], prm["D"], t["x"][0], t["B"][0], t["C"][0], t["dt"][0], ref)
            assert normwise_err(host(y), yr) < TOL, r
            _check_bk(ctx, model)
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL
