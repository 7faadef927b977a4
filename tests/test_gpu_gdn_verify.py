"""GPU parity of Gated DeltaNet speculative decoding (rssm_verify / rssm_verify_commit /
rssm_rollback, C ABI -> HIP) against the CPU oracle's recomputation of each round from the
committed state, and of the conventional snapshot comparator. Normwise 1e-5 per head vector;
bookkeeping bit-exact."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import Bookkeeping, gdn_spec_round, gdn_step, normwise_err
from tests.gpu_helpers import dev, gdn_dev_tokens, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _check_bk(ctx, model):
    h, l, n, e = ctx.bookkeeping()
    mh, ml, mn = model.snapshot()
    assert (h, l, n, e) == (list(mh), list(ml), list(mn), 0), (h, l, n, e, mh, ml, mn)


@pytest.mark.parametrize("d,W,K", [(16, 8, 3), (16, 4, 4), (64, 16, 6), (128, 16, 6),
                                   (128, 32, 6), (64, 1, 1), (128, 20, 5)])
def test_gdn_speculative_rounds(d, W, K):
    """Rounds of K drafts committed with seeded, full and empty acceptances or discarded, decode
    steps between some rounds: every draft output, the bookkeeping and the materialised state."""
    sh = wl.GDNShape(batch=4, nheads=2, d_k=d, d_v=d, window=W, max_draft=K)
    say(f"gdn verify d={d} W={W} K={K}")
    s0 = wl.gdn_state0(sh, 21)
    ctx = rb.Context("gdn", sh.batch, sh.nheads, d, d, W, max_draft=K)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W, K)
    ref = s0.astype(np.float64).copy()
    acc = wl.spec_accepted(sh.batch, 24, K, seed=21)
    ok = torch.empty(K, sh.batch, sh.nheads, d, device="cuda")
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    worst = 0.0
    for r in range(24):
        ins = wl.gdn_token_inputs(sh, 21, 300 + r, ntok=K)
        ctx.verify(ok, **gdn_dev_tokens(sh, ins, K))
        model.verify(K)
        _check_bk(ctx, model)
        if r % 6 == 0:
            a = np.full(sh.batch, K, np.int32)
        elif r % 6 == 1:
            a = np.zeros(sh.batch, np.int32)
        else:
            a = np.minimum(acc[r], K).astype(np.int32)
        if r % 6 == 5:                      # discard every draft
            a[:] = 0
            ctx.rollback(dev(np.array(model.len, dtype=np.int32)))
            model.rollback(model.len.copy())
        else:
            ctx.commit(dev(a))
            model.commit(a)
        o_ref = gdn_spec_round(ins, ref, a)
        err = normwise_err(host(ok), o_ref)
        worst = max(worst, err)
        assert err < TOL, (r, err)
        _check_bk(ctx, model)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, r
        if r % 4 == 3:
            t = wl.gdn_token_inputs(sh, 21, 700 + r)
            ctx.decode_step(o, **{k: v[0] for k, v in gdn_dev_tokens(sh, t, 1).items()})
            model.decode()
            orf = gdn_step(t["q"][0], t["k"][0], t["v"][0], t["beta"][0], t["alpha"][0], ref)
            assert normwise_err(host(o), orf) < TOL, r
            _check_bk(ctx, model)
    say(f"  worst draft output {worst:.3e}")


def test_gdn_speculative_serving_shape_sampled():
    """batch 512, 32 heads, 128 x 128, W = 16, K = 6: bookkeeping of every sequence after every
    call, outputs of sampled sequences against the oracle."""
    sh = wl.GDNShape(batch=512, nheads=32, d_k=128, d_v=128, window=16, max_draft=6)
    K, rounds = 6, 16
    s0 = wl.gdn_state0(sh, 0)
    acc = wl.spec_accepted(sh.batch, rounds, K, seed=0)
    ctx = rb.Context("gdn", sh.batch, sh.nheads, 128, 128, sh.window, max_draft=K)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window, K)
    sub = np.array([0, 7, 300, 511])
    ref = s0[sub].astype(np.float64)
    ok = torch.empty(K, sh.batch, sh.nheads, 128, device="cuda")
    pool = [wl.gdn_token_inputs(sh, 0, s, ntok=K) for s in range(3)]
    dpool = [gdn_dev_tokens(sh, p, K) for p in pool]
    worst = 0.0
    for r in range(rounds):
        ins = pool[r % 3]
        ctx.verify(ok, **dpool[r % 3])
        model.verify(K)
        _check_bk(ctx, model)
        ctx.commit(dev(acc[r]))
        model.commit(acc[r])
        _check_bk(ctx, model)
        o_ref = gdn_spec_round({k: v[:, sub] for k, v in ins.items()}, ref, acc[r][sub])
        worst = max(worst, normwise_err(host(ok)[:, sub], o_ref))
    say(f"  gdn spec worst normwise {worst:.3e}")
    assert worst < TOL


def test_gdn_snapshot_comparator_rounds():
    """The conventional comparator: per-draft snapshots in a slot pool, commit by pointer; outputs
    and committed states against the oracle's recomputation."""
    sh = wl.GDNShape(batch=5, nheads=2, d_k=16, d_v=16, window=8, max_draft=3)
    K = 3
    s0 = wl.gdn_state0(sh, 13)
    cfg = rb.make_config(rb.RSSM_GDN, sh.batch, sh.nheads, sh.nheads, 16, 16, sh.window, K)
    pool = torch.zeros((2 * K + 1,) + s0.shape, device="cuda")
    pool[2 * K] = dev(s0)
    slot_of = torch.full((sh.batch,), 2 * K, dtype=torch.int32, device="cuda")
    acc = wl.spec_accepted(sh.batch, 12, K, seed=13)
    ref = s0.astype(np.float64).copy()
    ok = torch.empty(K, sh.batch, sh.nheads, 16, device="cuda")
    for r in range(12):
        ins = wl.gdn_token_inputs(sh, 13, r, ntok=K)
        rb.step_baseline_spec(cfg, pool, slot_of, ok, **gdn_dev_tokens(sh, ins, K))
        rb.rssm_baseline_commit(cfg, slot_of, dev(acc[r]), K)
        o_ref = gdn_spec_round(ins, ref, acc[r])
        assert normwise_err(host(ok), o_ref) < TOL, r
        sl = host(slot_of)
        st = host(pool)
        committed = np.stack([st[sl[b], b] for b in range(sh.batch)])
        assert normwise_err(committed, ref) < TOL, r
