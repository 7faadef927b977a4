"""GPU parity of the Mamba-2 prefill (rssm_prefill, C ABI -> HIP matrix-core kernel) against the CPU
oracle: every prompt token's output, the checkpoint it leaves, the bookkeeping, and the decode
steps that follow. Normwise relative error 1e-5 per head vector (fp32); at the serving shape a head
vector over it must be within its rounding bound C_FP32 u32 kappa element by element."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import C_FP32, U32, cond_check, m2_kappa_step, m2_step, m2_step_f32, normwise_err
from tests.gpu_helpers import dev, host, m2_dev_tokens, m2_kappa_torch, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _ctx(sh, prm, bf16=False):
    c = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                   ngroups=sh.ngroups, bf16_read=bf16)
    A, D = dev(prm["A"]), dev(prm["D"])
    c.set_params(A, D)
    return c


def _oracle_run(prm, ins, t_range, ref):
    """Conventional steps t in t_range on the fp64 state ref (in place); outputs stacked."""
    return np.stack([m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t],
                             ins["dt"][t], ref) for t in t_range])


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (64, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("T", [1, 16, 37])
def test_prefill_shapes(P, N, T):
    """Every compiled head shape; prompts of one token, one full 16-token chunk and a ragged
    three-chunk prompt; then 5 decode steps from the new checkpoint."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=2, head_dim=P, d_state=N, window=8)
    say(f"prefill P={P} N={N} T={T}")
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    ins = wl.m2_token_inputs(sh, 0, 0, ntok=T + 5)
    d = m2_dev_tokens(sh, ins, T + 5)
    ctx = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    y = torch.empty(T, sh.batch, sh.nheads, P, device="cuda")
    ctx.prefill(y, **{k: v[:T] for k, v in d.items()})
    y_ref = _oracle_run(prm, ins, range(T), ref)
    err = normwise_err(host(y), y_ref)
    assert err < TOL, err
    h, l, n, e = ctx.bookkeeping()
    assert l == [0] * sh.batch and n == [0] * sh.batch and e == 0
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL
    y1 = torch.empty(sh.batch, sh.nheads, P, device="cuda")
    for t in range(T, T + 5):
        ctx.decode_step(y1, **{k: v[t] for k, v in d.items()})
        yr = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        assert normwise_err(host(y1), yr) < TOL, t
    say(f"  prompt outputs {err:.3e}")


@pytest.mark.parametrize("G", [4, 1])
def test_prefill_after_buffered_entries(G):
    """Sequences with different ring fills (masked re-init after some decode steps) are
    consolidated, then take a 20-token prompt; the second prompt continues the same state."""
    sh = wl.M2Shape(batch=3, nheads=4, ngroups=G, head_dim=16, d_state=16, window=8)
    prm = wl.m2_params(sh, 1)
    s0 = wl.m2_state0(sh, 1)
    ins = wl.m2_token_inputs(sh, 1, 0, ntok=3 + 20 + 20)
    d = m2_dev_tokens(sh, ins, 43)
    ctx = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    y1 = torch.empty(sh.batch, sh.nheads, 16, device="cuda")
    _oracle_run(prm, ins, range(2), ref)
    for t in range(2):
        ctx.decode_step(y1, **{k: v[t] for k, v in d.items()})
    fresh = wl.m2_state0(sh, 9)
    m = np.array([0, 1, 0], dtype=np.int32)
    ctx.init_checkpoint(dev(fresh), dev(m))
    ref[m != 0] = fresh[m != 0]
    ctx.decode_step(y1, **{k: v[2] for k, v in d.items()})
    _oracle_run(prm, ins, range(2, 3), ref)
    for lo in (3, 23):
        y = torch.empty(20, sh.batch, sh.nheads, 16, device="cuda")
        ctx.prefill(y, **{k: v[lo:lo + 20] for k, v in d.items()})
        y_ref = _oracle_run(prm, ins, range(lo, lo + 20), ref)
        assert normwise_err(host(y), y_ref) < TOL, lo
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, lo
        h, l, n, e = ctx.bookkeeping()
        assert l == [0] * sh.batch and e == 0


def test_prefill_bf16_copy_refreshed():
    """With the bf16 read copy: the prefill refreshes it, so the decode steps after the prompt
    read the new checkpoint (within the bf16 tolerance), and the fp32 checkpoint matches."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=4, head_dim=64, d_state=128, window=16)
    prm = wl.m2_params(sh, 2)
    s0 = wl.m2_state0(sh, 2)
    ins = wl.m2_token_inputs(sh, 2, 0, ntok=40)
    d = m2_dev_tokens(sh, ins, 40)
    ctx = _ctx(sh, prm, bf16=True)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    y = torch.empty(32, sh.batch, sh.nheads, 64, device="cuda")
    ctx.prefill(y, **{k: v[:32] for k, v in d.items()})
    assert normwise_err(host(y), _oracle_run(prm, ins, range(32), ref)) < TOL
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL
    y1 = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
    for t in range(32, 40):
        ctx.decode_step(y1, **{k: v[t] for k, v in d.items()})
        yr = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        assert normwise_err(host(y1).reshape(sh.batch, -1), yr.reshape(sh.batch, -1)) < 2e-2, t


def test_prefill_serving_shape_sampled():
    """Batch 256, 128 heads, 64x128, a 64-token prompt: the outputs of sampled sequences against the
    oracle, and every sequence against 64 decode steps of the same tokens on the GPU. Heads over
    1e-5 must be within the fp32 rounding bound; the fp32 conventional recurrence (oracle) is run
    on the same sample to show its own error there."""
    sh = wl.M2_SERVE
    T = 64
    say("prefill serving shape: generating inputs")
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    ins = wl.m2_token_inputs(sh, 0, 100, ntok=T)
    d = m2_dev_tokens(sh, ins, T)
    ctx = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    y = torch.empty(T, sh.batch, sh.nheads, sh.head_dim, device="cuda")
    ctx.prefill(y, **d)
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    ctx2 = _ctx(sh, prm)
    ctx2.init_checkpoint(dev(s0))
    A, D = dev(prm["A"]), dev(prm["D"])
    kap_state = dev(np.abs(s0))
    y1 = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    # sequence 17 has a head whose output nearly cancels at token 25 (|y| 6e-4)
    sub = np.array([0, 17, 77, 200, 255])
    pair = []
    yh = host(y)
    yd = np.empty((T, len(sub), sh.nheads, sh.head_dim), np.float32)
    for t in range(T):
        tok = {k: v[t] for k, v in d.items()}
        ctx2.decode_step(y1, **tok)
        kap = host(m2_kappa_torch(kap_state, A, D, tok["x"], tok["B"], tok["C"], tok["dt"]))
        y1h = host(y1)
        yd[t] = y1h[sub]
        pair.append(cond_check(yh[t], y1h, 2 * C_FP32 * U32 * kap, 2 * TOL))
    ref = s0[sub].astype(np.float64)
    r32 = s0[sub].copy()
    M = np.abs(ref)
    y_ref, y32, kref = [], [], []
    for t in range(T):
        a = [ins[k][t][sub] for k in ("x", "B", "C", "dt")]
        y_ref.append(m2_step(prm["A"], prm["D"], *a, ref))
        y32.append(m2_step_f32(prm["A"], prm["D"], *a, r32))
        kref.append(m2_kappa_step(prm["A"], prm["D"], *a, M))
    y_ref, y32, kref = np.stack(y_ref), np.stack(y32), np.stack(kref)
    bound = C_FP32 * U32 * kref
    cp = cond_check(yh[:, sub], y_ref, bound, TOL)
    cd = cond_check(yd, y_ref, bound, TOL)
    c32 = cond_check(y32, y_ref, bound, TOL)
    say(f"  prefill vs oracle: {cp}")
    say(f"  decode vs oracle: {cd}")
    say(f"  fp32 conventional recurrence (oracle) vs oracle: {c32}")
    for c, name in ((cp, "prefill"), (cd, "decode")):
        if c.where is not None:
            t, b, h = c.where
            say(f"  {name}: token {t}, sequence {sub[b]}, head {h}: normwise "
                f"{normwise_err(yh[t, sub[b], h] if name == 'prefill' else yd[t, b, h], y_ref[t, b, h]):.3e},"
                f" fp32 conventional {normwise_err(y32[t, b, h], y_ref[t, b, h]):.3e}")
    worst_pair = max(pair, key=lambda c: c.ratio_all)
    say(f"  prefill vs decode, all sequences (worst token): {worst_pair}")
    assert cp.ok and cd.ok and cp.ratio_all <= 1 and cd.ratio_all <= 1
    assert all(c.ok and c.ratio_all <= 1 for c in pair)
    assert normwise_err(host(mat)[sub], ref) < TOL
