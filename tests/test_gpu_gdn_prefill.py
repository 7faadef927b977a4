"""GPU parity of the Gated DeltaNet prefill (rssm_prefill, C ABI -> HIP matrix-core kernel) against
the CPU oracle: every prompt token's output, the checkpoint it leaves, the bookkeeping, and the
decode steps that follow. Normwise relative error 1e-5 per head vector (fp32); at the serving shape a
head vector over it must be within its rounding bound C_FP32 u32 kappa element by element (kappa
from the absolute-value recurrence, oracle.gdn_kappa_step)."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import C_FP32, U32, cond_check, gdn_kappa_step, gdn_step, normwise_err
from tests.gpu_helpers import dev, gdn_dev_tokens, gdn_kappa_torch, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _ctx(sh):
    return rb.Context("gdn", sh.batch, sh.nheads, sh.d_v, sh.d_k, sh.window)


def _oracle_run(ins, t_range, ref):
    """Conventional steps t in t_range on the fp64 state ref (in place); outputs stacked."""
    return np.stack([gdn_step(ins["q"][t], ins["k"][t], ins["v"][t], ins["beta"][t],
                              ins["alpha"][t], ref) for t in t_range])


def _tok(d, t):
    return {k: v[t] for k, v in d.items()}


@pytest.mark.parametrize("dd", [16, 64, 128])
@pytest.mark.parametrize("T", [1, 16, 37])
def test_gdn_prefill_shapes(dd, T):
    """Every compiled head shape; prompts of one token, one full 16-token chunk and a ragged
    three-chunk prompt; then 5 decode steps from the new checkpoint."""
    sh = wl.GDNShape(batch=2, nheads=4, d_k=dd, d_v=dd, window=8)
    say(f"gdn prefill d={dd} T={T}")
    s0 = wl.gdn_state0(sh, 0)
    ins = wl.gdn_token_inputs(sh, 0, 0, ntok=T + 5)
    d = gdn_dev_tokens(sh, ins, T + 5)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    o = torch.empty(T, sh.batch, sh.nheads, dd, device="cuda")
    ctx.prefill(o, **{k: v[:T] for k, v in d.items()})
    o_ref = _oracle_run(ins, range(T), ref)
    err = normwise_err(host(o), o_ref)
    assert err < TOL, err
    h, l, n, e = ctx.bookkeeping()
    assert l == [0] * sh.batch and n == [0] * sh.batch and e == 0
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL
    o1 = torch.empty(sh.batch, sh.nheads, dd, device="cuda")
    for t in range(T, T + 5):
        ctx.decode_step(o1, **_tok(d, t))
        orf = gdn_step(ins["q"][t], ins["k"][t], ins["v"][t], ins["beta"][t], ins["alpha"][t], ref)
        assert normwise_err(host(o1), orf) < TOL, t
    say(f"  prompt outputs {err:.3e}")


def test_gdn_prefill_after_buffered_entries():
    """Sequences with different ring fills (masked re-init after some decode steps) are
    consolidated, then take a 20-token prompt; the second prompt continues the same state."""
    sh = wl.GDNShape(batch=3, nheads=4, d_k=64, d_v=64, window=8)
    s0 = wl.gdn_state0(sh, 1)
    ins = wl.gdn_token_inputs(sh, 1, 0, ntok=43)
    d = gdn_dev_tokens(sh, ins, 43)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    o1 = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
    _oracle_run(ins, range(2), ref)
    for t in range(2):
        ctx.decode_step(o1, **_tok(d, t))
    fresh = wl.gdn_state0(sh, 9)
    m = np.array([0, 1, 0], dtype=np.int32)
    ctx.init_checkpoint(dev(fresh), dev(m))
    ref[m != 0] = fresh[m != 0]
    ctx.decode_step(o1, **_tok(d, 2))
    _oracle_run(ins, range(2, 3), ref)
    for lo in (3, 23):
        o = torch.empty(20, sh.batch, sh.nheads, 64, device="cuda")
        ctx.prefill(o, **{k: v[lo:lo + 20] for k, v in d.items()})
        o_ref = _oracle_run(ins, range(lo, lo + 20), ref)
        assert normwise_err(host(o), o_ref) < TOL, lo
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, lo
        h, l, n, e = ctx.bookkeeping()
        assert l == [0] * sh.batch and e == 0


def test_gdn_prefill_serving_shape_sampled():
    """Batch 256, 32 heads, 128x128, a 64-token prompt: the outputs of sampled sequences against the
    oracle, and every sequence against 64 decode steps of the same tokens on the GPU."""
    sh = wl.GDN_SERVE
    T = 64
    say("gdn prefill serving shape: generating inputs")
    s0 = wl.gdn_state0(sh, 0)
    ins = wl.gdn_token_inputs(sh, 0, 100, ntok=T)
    d = gdn_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(T, sh.batch, sh.nheads, sh.d_v, device="cuda")
    ctx.prefill(o, **d)
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    ctx2 = _ctx(sh)
    ctx2.init_checkpoint(dev(s0))
    kap_state = dev(np.abs(s0))
    o1 = torch.empty(sh.batch, sh.nheads, sh.d_v, device="cuda")
    sub = np.array([0, 31, 128, 255])
    pair = []
    oh = host(o)
    od = np.empty((T, len(sub), sh.nheads, sh.d_v), np.float32)
    for t in range(T):
        tok = _tok(d, t)
        ctx2.decode_step(o1, **tok)
        kap = host(gdn_kappa_torch(kap_state, tok["q"], tok["k"], tok["v"], tok["beta"],
                                   tok["alpha"]))
        o1h = host(o1)
        od[t] = o1h[sub]
        pair.append(cond_check(oh[t], o1h, 2 * C_FP32 * U32 * kap, 2 * TOL))
    ref = s0[sub].astype(np.float64)
    M = np.abs(ref)
    o_ref, kref = [], []
    for t in range(T):
        a = [ins[k][t][sub] for k in ("q", "k", "v", "beta", "alpha")]
        o_ref.append(gdn_step(*a, ref))
        kref.append(gdn_kappa_step(*a, M))
    o_ref, kref = np.stack(o_ref), np.stack(kref)
    cp = cond_check(oh[:, sub], o_ref, C_FP32 * U32 * kref, TOL)
    cd = cond_check(od, o_ref, C_FP32 * U32 * kref, TOL)
    worst_pair = max(pair, key=lambda c: c.ratio_all)
    say(f"  prefill vs oracle: {cp}")
    say(f"  decode vs oracle: {cd}")
    say(f"  prefill vs decode, all sequences (worst token): {worst_pair}")
    assert cp.ok and cd.ok and cp.ratio_all <= 1 and cd.ratio_all <= 1
    assert all(c.ok and c.ratio_all <= 1 for c in pair)
    assert normwise_err(host(mat)[sub], ref) < TOL
