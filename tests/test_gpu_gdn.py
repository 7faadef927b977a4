"""GPU parity of the Gated DeltaNet ReplaySSM path (C ABI -> HIP kernels) against the CPU oracle.
Normwise relative error 1e-5 (fp32); bookkeeping bit-exact."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import Bookkeeping, gdn_step, normwise_err
from tests.gpu_helpers import dev, gdn_dev_tokens, host, say, tok0

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _ctx(sh: wl.GDNShape):
    return rb.Context("gdn", sh.batch, sh.nheads, sh.d_v, sh.d_k, sh.window)


def _step_ref(ins, t, ref, sel=slice(None)):
    return gdn_step(ins["q"][t][sel], ins["k"][t][sel], ins["v"][t][sel], ins["beta"][t][sel],
                    ins["alpha"][t][sel], ref)


@pytest.mark.parametrize("d,W", [(16, 4), (64, 16), (128, 16), (128, 1), (16, 20), (64, 24), (128, 32)])
def test_decode_every_call(d, W):
    sh = wl.GDNShape(batch=3, nheads=3, d_k=d, d_v=d, window=W)
    T = 3 * W + 5 if W > 1 else 9
    say(f"gdn decode d={d} W={W} T={T}")
    s0 = wl.gdn_state0(sh, 0)
    ins = wl.gdn_token_inputs(sh, 0, 0, ntok=T)
    dd = gdn_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    worst = 0.0
    for t in range(T):
        ctx.decode_step(o, **{k: v[t] for k, v in dd.items()})
        o_ref = _step_ref(ins, t, ref)
        model.decode()
        err = normwise_err(host(o), o_ref)
        worst = max(worst, err)
        assert err < TOL, (t, err)
        h, l, n, e = ctx.bookkeeping()
        assert (h, l, n, e) == (list(model.head), list(model.len), list(model.ndraft), 0)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, t
    say(f"  worst normwise {worst:.3e}")


@pytest.mark.parametrize("d,W", [(64, 8), (128, 24)])
def test_consolidate_and_masked_init(d, W):
    """Masked re-init, consolidation with a threshold, materialisation after every operation. At
    W = 24 the consolidation folds up to 23 entries (two 16-entry blocks)."""
    sh = wl.GDNShape(batch=4, nheads=2, d_k=d, d_v=d, window=W)
    say(f"gdn consolidate d={d} W={W}")
    s0 = wl.gdn_state0(sh, 1)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    sched = (["d"] * (W - 3) + [("mask", [0, 1, 0, 1])] + ["d"] * 2 + [("cons", 3)] + ["d"] * (W + 1)
             + [("cons", 1)])
    for i, op in enumerate(sched):
        if op == "d":
            ins = wl.gdn_token_inputs(sh, 1, 50 + i)
            ctx.decode_step(o, **tok0(gdn_dev_tokens(sh, ins, 1)))
            o_ref = _step_ref(ins, 0, ref)
            model.decode()
            assert normwise_err(host(o), o_ref) < TOL, i
        elif op[0] == "mask":
            fresh = wl.gdn_state0(sh, 77)
            m = np.array(op[1], dtype=np.int32)
            ctx.init_checkpoint(dev(fresh), dev(m))
            ref[m != 0] = fresh[m != 0]
            model.init(m)
        else:
            ctx.consolidate(op[1])
            model.consolidate(op[1])
        h, l, n, e = ctx.bookkeeping()
        assert (h, l, n, e) == (list(model.head), list(model.len), list(model.ndraft), 0), i
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, i


def test_no_write_special_case_is_gemv():
    """alpha = 1, beta = 0: the state never changes and o = S0 q."""
    sh = wl.GDNShape(batch=2, nheads=4, d_k=128, d_v=128, window=16)
    s0 = wl.gdn_state0(sh, 2)
    ins = wl.gdn_token_inputs(sh, 2, 0, ntok=20)
    ins["alpha"][:] = 1.0
    ins["beta"][:] = 0.0
    dd = gdn_dev_tokens(sh, ins, 20)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(2, 4, 128, device="cuda")
    for t in range(20):
        ctx.decode_step(o, **{k: v[t] for k, v in dd.items()})
        ref = np.einsum("bhij,bhj->bhi", s0.astype(np.float64), ins["q"][t].astype(np.float64))
        assert normwise_err(host(o), ref) < TOL


@pytest.mark.parametrize("d", [16, 128])
def test_rmw_comparator(d):
    sh = wl.GDNShape(batch=3, nheads=2, d_k=d, d_v=d, window=4)
    s0 = wl.gdn_state0(sh, 3)
    ins = wl.gdn_token_inputs(sh, 3, 0, ntok=12)
    dd = gdn_dev_tokens(sh, ins, 12)
    cfg = rb.make_config(rb.RSSM_GDN, sh.batch, sh.nheads, sh.nheads, d, d, 4)
    st = dev(s0)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(1, sh.batch, sh.nheads, d, device="cuda")
    for t in range(8):
        rb.step_baseline(cfg, st, o, **{k: v[t:t + 1] for k, v in dd.items()})
        o_ref = _step_ref(ins, t, ref)
        assert normwise_err(host(o)[0], o_ref) < TOL
    assert normwise_err(host(st), ref) < TOL
    K = 4
    snaps = torch.empty((K,) + s0.shape, device="cuda")
    ok = torch.empty(K, sh.batch, sh.nheads, d, device="cuda")
    before = host(st).copy()
    rb.step_baseline(cfg, st, ok, snapshots=snaps, **{k: v[8:12] for k, v in dd.items()})
    assert np.array_equal(host(st), before)
    for k in range(K):
        o_ref = _step_ref(ins, 8 + k, ref)
        assert normwise_err(host(ok)[k], o_ref) < TOL
        assert normwise_err(host(snaps)[k], ref) < TOL


SUBSET = np.array([0, 3, 77, 128, 200, 255])


def test_serving_shape_sampled():
    """batch 256, 32 heads, d_k = d_v = 128, W = 16, 512 steps: sampled sequences against the
    oracle, all sequences against the on-GPU read-modify-write kernel."""
    sh = wl.GDN_SERVE
    steps, pool = 512, 32
    say("gdn serving shape: generating inputs")
    s0 = wl.gdn_state0(sh, 0)
    slots = [wl.gdn_token_inputs(sh, 0, s) for s in range(pool)]
    dslots = [tok0(gdn_dev_tokens(sh, s, 1)) for s in slots]
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    cfg = rb.make_config(rb.RSSM_GDN, sh.batch, sh.nheads, sh.nheads, sh.d_v, sh.d_k, sh.window)
    st = dev(s0)
    o = torch.empty(sh.batch, sh.nheads, sh.d_v, device="cuda")
    o2 = torch.empty(1, sh.batch, sh.nheads, sh.d_v, device="cuda")
    sub = torch.from_numpy(SUBSET).cuda()
    os_ = torch.empty(steps, len(SUBSET), sh.nheads, sh.d_v, device="cuda")
    worst_pair = 0.0
    for t in range(steps):
        tok = dslots[t % pool]
        ctx.decode_step(o, **tok)
        os_[t] = o.index_select(0, sub)
        rb.step_baseline(cfg, st, o2, **{k: v.unsqueeze(0) for k, v in tok.items()})
        if t % 64 == 63:
            worst_pair = max(worst_pair, normwise_err(host(o), host(o2)[0]))
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    h, l, n, e = ctx.bookkeeping()
    assert l == [steps % sh.window] * sh.batch and e == 0
    ref = s0[SUBSET].astype(np.float64)
    worst = 0.0
    oh = host(os_)
    for t in range(steps):
        s = slots[t % pool]
        o_ref = _step_ref(s, 0, ref, SUBSET)
        worst = max(worst, normwise_err(oh[t], o_ref))
    say(f"  worst normwise {worst:.3e} (replay vs rmw {worst_pair:.3e})")
    assert worst < TOL
    assert worst_pair < 2 * TOL
    assert normwise_err(host(mat)[SUBSET], ref) < TOL
    assert normwise_err(host(st)[SUBSET], ref) < TOL
