"""GPU parity of the Mamba-2 ReplaySSM path (C ABI -> HIP kernels) against the CPU oracle.

Tolerances: normwise relative error (max over output vectors of max|d| / max|ref|) 1e-5 for the
fp32 paths and 2e-2 for the bf16 read copy; bookkeeping (head, len, ndraft, error bits)
bit-exact. At the serving shape an output vector that misses its tolerance must instead be within
its rounding bound element by element: C_FP32 u32 kappa for fp32 (kappa the sum of the absolute
values of the output's terms, oracle.m2_kappa_step), plus Lam u16 sum_n |S0[p,n]| |C_n| for the
bf16 read copy.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import (C_FP32, U16, U32, Bookkeeping, cond_check, m2_kappa_step, m2_spec_kappa,
                    m2_spec_round, m2_step, normwise_err)
from tests.gpu_helpers import dev, host, m2_dev_tokens, m2_kappa_torch, say, tok0

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ctx(sh: wl.M2Shape, prm, bf16=False, store_c=True):
    c = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                   ngroups=sh.ngroups, max_draft=sh.max_draft, bf16_read=bf16, store_c=store_c)
    A, D = dev(prm["A"]), dev(prm["D"])
    c.set_params(A, D)
    return c, A, D


def _check_bk(ctx, model: Bookkeeping, err=None):
    h, l, n, e = ctx.bookkeeping()
    mh, ml, mn = model.snapshot()
    assert h == list(mh) and l == list(ml) and n == list(mn), (h, l, n, mh, ml, mn)
    if err is not None:
        assert e == err
    return e


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("G", [4, 1])
def test_tiny_decode_every_call(bf16, G):
    """B=2, H=4, P=N=16, W=4, 64 steps: every y, the materialised state after every call and the
    bookkeeping after every call."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=G, head_dim=16, d_state=16, window=4)
    say(f"tiny decode bf16={bf16} G={G}")
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    ins = wl.m2_token_inputs(sh, 0, 0, ntok=64)
    d = m2_dev_tokens(sh, ins, 64)
    ctx, A, D = _ctx(sh, prm, bf16)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window)
    ref = s0.astype(np.float64).copy()
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    worst = 0.0
    for t in range(64):
        tok = {k: v[t] for k, v in d.items()}
        ctx.decode_step(y, **tok)
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        model.decode()
        err = normwise_err(host(y), y_ref)
        worst = max(worst, err)
        assert err < (TOL_BF16 if bf16 else TOL), (t, err)
        _check_bk(ctx, model, 0)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, t
    say(f"  worst normwise {worst:.3e}")


def test_rmw_comparator_tiny():
    sh = wl.M2Shape(batch=3, nheads=4, ngroups=2, head_dim=16, d_state=16, window=4)
    prm = wl.m2_params(sh, 2)
    s0 = wl.m2_state0(sh, 2)
    ins = wl.m2_token_inputs(sh, 2, 0, ntok=24)
    d = m2_dev_tokens(sh, ins, 24)
    cfg = rb.make_config(rb.RSSM_MAMBA2, sh.batch, sh.nheads, sh.ngroups, 16, 16, 4)
    A, D = dev(prm["A"]), dev(prm["D"])
    st = dev(s0)
    ref = s0.astype(np.float64).copy()
    y = torch.empty(1, sh.batch, sh.nheads, 16, device="cuda")
    for t in range(24):
        rb.step_baseline(cfg, st, y, A, D, **{k: v[t:t + 1] for k, v in d.items()})
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        assert normwise_err(host(y)[0], y_ref) < TOL
    assert normwise_err(host(st), ref) < TOL
    # snapshot mode: K tokens from the state, state read-only, one snapshot per token
    K = 5
    snaps = torch.empty((K,) + s0.shape, device="cuda")
    yk = torch.empty(K, sh.batch, sh.nheads, 16, device="cuda")
    before = host(st).copy()
    rb.step_baseline(cfg, st, yk, A, D, snapshots=snaps, **{k: v[:K] for k, v in d.items()})
    assert np.array_equal(host(st), before)
    r2 = before.astype(np.float64)
    for k in range(K):
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][k], ins["B"][k], ins["C"][k], ins["dt"][k], r2)
        assert normwise_err(host(yk)[k], y_ref) < TOL
        assert normwise_err(host(snaps)[k], r2) < TOL


@pytest.mark.parametrize("P,N", [(16, 16), (32, 32), (64, 64), (64, 128), (128, 128)])
def test_rmw_comparator_workgroup_sizes(P, N):
    """The conventional kernel on the workgroup sizes of few tiles, which depend on the token
    count: one token, a 5-draft snapshot launch, then 12 tokens in one launch (the single-token
    workgroup of large grids is covered by the next test)."""
    sh = wl.M2Shape(batch=2, nheads=3, ngroups=3, head_dim=P, d_state=N, window=16)
    prm = wl.m2_params(sh, 7)
    s0 = wl.m2_state0(sh, 7)
    ins = wl.m2_token_inputs(sh, 7, 0, ntok=13)
    d = m2_dev_tokens(sh, ins, 13)
    cfg = rb.make_config(rb.RSSM_MAMBA2, sh.batch, sh.nheads, sh.ngroups, P, N, 16)
    A, D = dev(prm["A"]), dev(prm["D"])
    st = dev(s0)
    ref = s0.astype(np.float64).copy()
    y1 = torch.empty(1, sh.batch, sh.nheads, P, device="cuda")
    rb.step_baseline(cfg, st, y1, A, D, **{k: v[0:1] for k, v in d.items()})
    y_ref = m2_step(prm["A"], prm["D"], ins["x"][0], ins["B"][0], ins["C"][0], ins["dt"][0], ref)
    assert normwise_err(host(y1)[0], y_ref) < TOL
    assert normwise_err(host(st), ref) < TOL
    K = 5
    snaps = torch.empty((K,) + s0.shape, device="cuda")
    yk = torch.empty(K, sh.batch, sh.nheads, P, device="cuda")
    rb.step_baseline(cfg, st, yk, A, D, snapshots=snaps, **{k: v[1:1 + K] for k, v in d.items()})
    r2 = ref.copy()
    for k in range(K):
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][1 + k], ins["B"][1 + k], ins["C"][1 + k],
                        ins["dt"][1 + k], r2)
        assert normwise_err(host(yk)[k], y_ref) < TOL
        assert normwise_err(host(snaps)[k], r2) < TOL
    y12 = torch.empty(12, sh.batch, sh.nheads, P, device="cuda")
    rb.step_baseline(cfg, st, y12, A, D, **{k: v[1:13] for k, v in d.items()})
    for k in range(12):
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][1 + k], ins["B"][1 + k], ins["C"][1 + k],
                        ins["dt"][1 + k], ref)
        assert normwise_err(host(y12)[k], y_ref) < TOL, k
    assert normwise_err(host(st), ref) < TOL


@pytest.mark.parametrize("P,N", [(64, 128), (128, 128), (64, 64), (32, 32)])
def test_rmw_comparator_single_token_large_grid(P, N):
    """One token over 16k tiles, where the conventional kernel takes its single-token workgroup
    (clamp(P N / 8, 64, 1024) threads: 1024 at 64 x 128 and 128 x 128, 512 at 64 x 64, 128 at
    32 x 32), at each of those shapes."""
    sh = wl.M2Shape(batch=64, nheads=256, ngroups=16, head_dim=P, d_state=N, window=16)
    say(f"conventional kernel, one token, 16k tiles of {P}x{N}")
    prm = wl.m2_params(sh, 8)
    s0 = wl.m2_state0(sh, 8)
    ins = wl.m2_token_inputs(sh, 8, 0, ntok=1)
    d = m2_dev_tokens(sh, ins, 1)
    cfg = rb.make_config(rb.RSSM_MAMBA2, sh.batch, sh.nheads, sh.ngroups, P, N, 16)
    st = dev(s0)
    ref = s0.astype(np.float64)
    y = torch.empty(1, sh.batch, sh.nheads, P, device="cuda")
    rb.step_baseline(cfg, st, y, dev(prm["A"]), dev(prm["D"]), **d)
    y_ref = m2_step(prm["A"], prm["D"], ins["x"][0], ins["B"][0], ins["C"][0], ins["dt"][0], ref)
    assert normwise_err(host(y)[0], y_ref) < TOL
    assert normwise_err(host(st), ref) < TOL


def test_ragged_lengths_masked_init_consolidate():
    """Sequences at different buffer fills (masked re-init), grouped B/C, partial folds."""
    sh = wl.M2Shape(batch=5, nheads=4, ngroups=2, head_dim=32, d_state=32, window=4)
    prm = wl.m2_params(sh, 3)
    s0 = wl.m2_state0(sh, 3)
    ctx, A, D = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window)
    ref = s0.astype(np.float64).copy()
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    schedule = ["d", "d", ("mask", [1, 0, 1, 0, 0]), "d", "d", "d", ("cons", 2), "d", "d",
                ("mask", [0, 0, 0, 1, 1]), "d", "d", "d", "d", "d", ("cons", 1), "d"]
    for i, op in enumerate(schedule):
        if op == "d":
            ins = wl.m2_token_inputs(sh, 3, 10 + i)
            tok = tok0(m2_dev_tokens(sh, ins, 1))
            ctx.decode_step(y, **tok)
            y_ref = m2_step(prm["A"], prm["D"], ins["x"][0], ins["B"][0], ins["C"][0], ins["dt"][0], ref)
            model.decode()
            assert normwise_err(host(y), y_ref) < TOL, i
        elif op[0] == "mask":
            fresh = wl.m2_state0(sh, 100 + i)
            m = np.array(op[1], dtype=np.int32)
            ctx.init_checkpoint(dev(fresh), dev(m))
            ref[m != 0] = fresh[m != 0]
            model.init(m)
        else:
            ctx.consolidate(op[1])
            model.consolidate(op[1])
        _check_bk(ctx, model, 0)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, i


@pytest.mark.parametrize("bf16", [False, True])
def test_speculative_rounds(bf16):
    """verify K drafts -> causal outputs equal conventional steps from the committed state;
    commit by pointer; interleaved decodes; discarded drafts."""
    sh = wl.M2Shape(batch=6, nheads=4, ngroups=4, head_dim=16, d_state=16, window=8, max_draft=3)
    prm = wl.m2_params(sh, 4)
    s0 = wl.m2_state0(sh, 4)
    ctx, A, D = _ctx(sh, prm, bf16)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window, sh.max_draft)
    ref = s0.astype(np.float64).copy()
    acc = wl.spec_accepted(sh.batch, 40, sh.max_draft, seed=4)
    tol = TOL_BF16 if bf16 else TOL
    yk = torch.empty(3, sh.batch, sh.nheads, 16, device="cuda")
    y = torch.empty(sh.batch, sh.nheads, 16, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    for r in range(40):
        K = 1 + r % 3
        ins = wl.m2_token_inputs(sh, 4, 200 + r, ntok=K)
        ctx.verify(yk[:K], **m2_dev_tokens(sh, ins, K))
        model.verify(K)
        _check_bk(ctx, model)
        a = np.minimum(acc[r], K).astype(np.int32)
        if r % 7 == 6:
            a[:] = 0
            ctx.rollback(dev(np.array(model.len, dtype=np.int32)))
            model.rollback(model.len.copy())
        else:
            ctx.commit(dev(a))
            model.commit(a)
        y_ref = m2_spec_round(prm["A"], prm["D"], ins, ref, a)
        assert normwise_err(host(yk[:K]), y_ref) < tol, r
        _check_bk(ctx, model, 0)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, r
        if r % 3 == 2:
            t = wl.m2_token_inputs(sh, 4, 500 + r)
            ctx.decode_step(y, **tok0(m2_dev_tokens(sh, t, 1)))
            model.decode()
            y_ref = m2_step(prm["A"], prm["D"], t["x"][0], t["B"][0], t["C"][0], t["dt"][0], ref)
            assert normwise_err(host(y), y_ref) < tol, r
            _check_bk(ctx, model, 0)


def test_golden_bookkeeping_trace_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "bookkeeping_w4_k2.json")))
    sh = wl.M2Shape(batch=g["batch"], nheads=2, ngroups=2, head_dim=16, d_state=16,
                    window=g["window"], max_draft=g["max_draft"])
    prm = wl.m2_params(sh, 0)
    ctx, A, D = _ctx(sh, prm)
    y = torch.empty(sh.max_draft, sh.batch, sh.nheads, 16, device="cuda")
    for i, op in enumerate(g["ops"]):
        kind = op["op"]
        if kind == "init":
            ctx.init_checkpoint(dev(wl.m2_state0(sh, 0)))
        elif kind == "init_mask":
            ctx.init_checkpoint(dev(wl.m2_state0(sh, 1)), dev(np.array(op["arg"], dtype=np.int32)))
        elif kind == "decode":
            ctx.decode_step(y[0], **tok0(m2_dev_tokens(sh, wl.m2_token_inputs(sh, 0, i), 1)))
        elif kind == "verify":
            K = op["K"]
            ctx.verify(y[:K], **m2_dev_tokens(sh, wl.m2_token_inputs(sh, 0, i, ntok=K), K))
        elif kind == "commit":
            ctx.commit(dev(np.array(op["arg"], dtype=np.int32)))
        elif kind == "rollback":
            ctx.rollback(dev(np.array(op["arg"], dtype=np.int32)))
        elif kind == "consolidate":
            ctx.consolidate(op["arg"])
        if kind == "read_err":
            assert ctx.bookkeeping()[3] == op["err"], (i, op)
            continue
        h, l, n = _peek(ctx)
        assert (h, l, n) == (op["head"], op["len"], op["ndraft"]), (i, op, h, l, n)


def _peek(ctx):
    """head / len / ndraft without reading (and so without clearing) the error word."""
    import ctypes
    B = ctx.cfg.batch
    arr = ctypes.c_int32 * B
    h, l, n = arr(), arr(), arr()
    st = rb.load_library().rssm_read_bookkeeping(ctx.handle, h, l, n, None, rb._stream(None))
    assert st == 0
    return list(h), list(l), list(n)


def test_rollback_prefix_bit_exact():
    """Run A: consolidate(W-K+1), verify K drafts, commit a. Run B: same consolidate, verify only
    the first a drafts, commit a. Outputs of the a drafts, bookkeeping, the materialised state and
    every later output are bit-identical."""
    sh = wl.M2Shape(batch=4, nheads=4, ngroups=4, head_dim=64, d_state=128, window=16, max_draft=6)
    prm = wl.m2_params(sh, 5)
    s0 = dev(wl.m2_state0(sh, 5))
    K, a = 6, 4
    outs = []
    for run in ("A", "B"):
        ctx, A, D = _ctx(sh, prm)
        ctx.init_checkpoint(s0)
        y = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
        for t in range(13):
            ctx.decode_step(y, **tok0(m2_dev_tokens(sh, wl.m2_token_inputs(sh, 5, t), 1)))
        ctx.consolidate(sh.window - K + 1)
        ins = wl.m2_token_inputs(sh, 5, 99, ntok=K)
        n = K if run == "A" else a
        yk = torch.empty(n, sh.batch, sh.nheads, 64, device="cuda")
        ctx.verify(yk, **m2_dev_tokens(sh, {k: v[:n] for k, v in ins.items()}, n))
        ctx.commit(dev(np.full(sh.batch, a, dtype=np.int32)))
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        later = []
        for t in range(5):
            ctx.decode_step(y, **tok0(m2_dev_tokens(sh, wl.m2_token_inputs(sh, 5, 300 + t), 1)))
            later.append(host(y).copy())
        outs.append((host(yk)[:a].copy(), ctx.bookkeeping(), host(mat).copy(), later))
    (ya, bka, ma, la), (yb, bkb, mb, lb) = outs
    assert np.array_equal(ya, yb)
    assert bka == bkb
    assert np.array_equal(ma, mb)
    for u, v in zip(la, lb):
        assert np.array_equal(u, v)


def test_rollback_to_shorter_prefix_equals_shorter_run():
    sh = wl.M2Shape(batch=3, nheads=4, ngroups=4, head_dim=16, d_state=16, window=8)
    prm = wl.m2_params(sh, 6)
    s0 = dev(wl.m2_state0(sh, 6))
    toks = [tok0(m2_dev_tokens(sh, wl.m2_token_inputs(sh, 6, t), 1)) for t in range(5)]
    res = []
    for n_dec, rb_len in ((5, [2, 0, 5]), (2, None)):
        ctx, A, D = _ctx(sh, prm)
        ctx.init_checkpoint(s0)
        y = torch.empty(3, 4, 16, device="cuda")
        for t in range(n_dec):
            ctx.decode_step(y, **toks[t])
        if rb_len is not None:
            ctx.rollback(dev(np.array(rb_len, dtype=np.int32)))
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        res.append((host(mat).copy(), ctx.bookkeeping()))
    # sequence 0 rolled back to 2 equals the 2-token run; 1 (len 0) equals the initial state
    assert np.array_equal(res[0][0][0], res[1][0][0])
    assert np.array_equal(res[0][0][1], host(s0)[1])
    assert res[0][1][1] == [2, 0, 5]


def test_out_of_range_commit_and_rollback_raise_bits():
    sh = wl.M2Shape(batch=4, nheads=2, ngroups=2, head_dim=16, d_state=16, window=4, max_draft=2)
    prm = wl.m2_params(sh, 7)
    ctx, A, D = _ctx(sh, prm)
    ctx.init_checkpoint(dev(wl.m2_state0(sh, 7)))
    yk = torch.empty(2, 4, 2, 16, device="cuda")
    ctx.verify(yk, **m2_dev_tokens(sh, wl.m2_token_inputs(sh, 7, 1, ntok=2), 2))
    ctx.commit(dev(np.array([0, 3, -1, 2], dtype=np.int32)))
    h, l, n, e = ctx.bookkeeping()
    assert l == [0, 0, 0, 2] and n == [0, 0, 0, 0] and e == rb.RSSM_DEV_COMMIT_RANGE
    ctx.rollback(dev(np.array([0, 0, 1, 3], dtype=np.int32)))
    h, l, n, e = ctx.bookkeeping()
    assert l == [0, 0, 0, 2] and e == rb.RSSM_DEV_ROLLBACK_RANGE
    assert ctx.bookkeeping()[3] == 0
    # host-side call-order checks
    with pytest.raises(rb.RssmError):
        ctx.commit(dev(np.zeros(4, dtype=np.int32)))
    ctx.verify(yk, **m2_dev_tokens(sh, wl.m2_token_inputs(sh, 7, 2, ntok=2), 2))
    with pytest.raises(rb.RssmError):
        ctx.decode_step(yk[0], **tok0(m2_dev_tokens(sh, wl.m2_token_inputs(sh, 7, 3), 1)))
    ctx.rollback(dev(np.zeros(4, dtype=np.int32)))


def test_determinism_and_head_permutation():
    sh = wl.M2Shape(batch=3, nheads=8, ngroups=8, head_dim=64, d_state=128, window=16)
    prm = wl.m2_params(sh, 8)
    s0 = wl.m2_state0(sh, 8)
    ins = wl.m2_token_inputs(sh, 8, 0, ntok=20)
    perm = np.array([3, 1, 7, 0, 2, 6, 5, 4])
    runs = []
    for p in (None, None, perm):
        pp = {k: v for k, v in prm.items()} if p is None else {k: v[p].copy() for k, v in prm.items()}
        ss = s0 if p is None else s0[:, p].copy()
        ii = ins if p is None else {"x": ins["x"][:, :, p].copy(), "B": ins["B"][:, :, p].copy(),
                                    "C": ins["C"][:, :, p].copy(), "dt": ins["dt"][:, :, p].copy()}
        ctx, A, D = _ctx(sh, pp)
        ctx.init_checkpoint(dev(ss))
        d = m2_dev_tokens(sh, ii, 20)
        y = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
        ys = []
        for t in range(20):
            ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
            ys.append(host(y).copy())
        runs.append(np.stack(ys))
    assert np.array_equal(runs[0], runs[1])
    assert np.array_equal(runs[0][:, :, perm], runs[2])


# ---------------------------------------------------------------------------------------------
# serving shape: batch 256, 128 heads, head_dim 64, d_state 128, W = 16, 512 steps
# ---------------------------------------------------------------------------------------------

SUBSET = np.array([0, 1, 37, 101, 128, 190, 254, 255])


@pytest.mark.parametrize("bf16,steps,G", [(False, 512, 128), (True, 512, 128), (False, 128, 8),
                                          (False, 128, 1)])
def test_serving_shape_sampled(bf16, steps, G):
    """Serving shape (batch 256, 128 heads, 64x128, W = 16): sampled sequences against the oracle
    at every step, all sequences against the read-modify-write kernel; also with B/C shared by
    groups of heads (G = 8, G = 1). With the bf16 read copy: every replayed element within the
    bf16 rounding bound of the checkpoint term, and no drift (the worst error of the last 64 steps
    no larger than that of the first 64: every fold restarts the copy from the fp32 checkpoint)."""
    sh = wl.M2_SERVE if G == 128 else wl.M2Shape(batch=256, nheads=128, ngroups=G, head_dim=64,
                                                   d_state=128, window=16)
    say(f"serving shape bf16={bf16} steps={steps} G={G}: generating inputs")
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    pool = 32
    slots = [wl.m2_token_inputs(sh, 0, s) for s in range(pool)]
    dslots = [tok0(m2_dev_tokens(sh, s, 1)) for s in slots]
    ctx, A, D = _ctx(sh, prm, bf16)
    ctx.init_checkpoint(dev(s0))
    cfg = rb.make_config(rb.RSSM_MAMBA2, sh.batch, sh.nheads, sh.ngroups, sh.head_dim, sh.d_state,
                         sh.window)
    st_rmw = dev(s0)
    kap_state = dev(np.abs(s0)) if not bf16 else None
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    y2 = torch.empty(1, sh.batch, sh.nheads, sh.head_dim, device="cuda")
    sub = torch.from_numpy(SUBSET).cuda()
    ys = torch.empty(steps, len(SUBSET), sh.nheads, sh.head_dim, device="cuda")
    pair = []
    say("  running GPU steps")
    for t in range(steps):
        tok = dslots[t % pool]
        ctx.decode_step(y, **tok)
        ys[t] = y.index_select(0, sub)
        if not bf16:
            rb.step_baseline(cfg, st_rmw, y2, A, D, **{k: v.unsqueeze(0) for k, v in tok.items()})
            kap = m2_kappa_torch(kap_state, A, D, tok["x"], tok["B"], tok["C"], tok["dt"])
            if t % 64 == 63:     # replay vs read-modify-write at every sequence
                pair.append(cond_check(host(y), host(y2)[0], 2 * C_FP32 * U32 * host(kap), 2 * TOL))
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    h, l, n, e = ctx.bookkeeping()
    assert l == [steps % sh.window] * sh.batch and h == [0] * sh.batch and e == 0
    say("  oracle on the sampled sequences")
    ref = s0[SUBSET].astype(np.float64)
    M = np.abs(ref)        # absolute-value recurrence: kappa of every output
    ck = ref.copy()        # the checkpoint the kernel reads: the state at the last fold
    win_dt = []            # dt of the entries buffered since that fold
    tol = TOL_BF16 if bf16 else TOL
    worst_ratio = worst_ratio_all = 0.0
    worst = worst_tok = 0.0
    n_over = 0
    per_step = []
    ys_h = host(ys)
    W = sh.window
    for t in range(steps):
        s = {k: v[0][SUBSET] for k, v in slots[t % pool].items()}
        args = (s["x"], s["B"], s["C"], s["dt"])
        y_ref = m2_step(prm["A"], prm["D"], *args, ref)
        kap = m2_kappa_step(prm["A"], prm["D"], *args, M)
        bound = C_FP32 * U32 * kap
        win_dt.append(s["dt"].astype(np.float64))
        if bf16 and t % W + 1 < W:
            # bf16 rounding of the checkpoint read: |dy| <= Lam * u16 * sum_n |S0[p,n]| |C_n|
            lam = np.exp(prm["A"].astype(np.float64)[None, :] * np.sum(win_dt, axis=0))
            hh = np.arange(sh.nheads) // (sh.nheads // sh.ngroups)
            Cg = np.abs(s["C"].astype(np.float64))[:, hh]
            bound = bound + lam[..., None] * U16 * np.einsum("bhpn,bhn->bhp", np.abs(ck), Cg)
        c = cond_check(ys_h[t], y_ref, bound, tol)
        assert c.ok, (t, c)
        worst_ratio = max(worst_ratio, c.ratio_over)
        worst_ratio_all = max(worst_ratio_all, c.ratio_all)
        worst = max(worst, c.worst)
        n_over += c.n_over
        per_step.append(normwise_err(ys_h[t].reshape(len(SUBSET), -1), y_ref.reshape(len(SUBSET), -1)))
        worst_tok = max(worst_tok, per_step[-1])
        if t % W + 1 == W:
            ck = ref.copy()
            win_dt = []
    say(f"  per head: worst normwise {worst:.3e}, {n_over} head vectors over {tol:g}, worst "
        f"|d|/bound over them {worst_ratio:.3f}, over all elements {worst_ratio_all:.3f}; per "
        f"sequence-token {worst_tok:.3e}")
    for c in pair:
        say(f"  replay vs read-modify-write, all sequences: {c}")
        assert c.ok
    assert worst_ratio_all <= 1.0
    if bf16:
        first, last = max(per_step[:64]), max(per_step[-64:])
        say(f"  bf16 drift: worst per sequence-token error, first 64 steps {first:.3e}, last 64 "
            f"{last:.3e}")
        assert last <= first
    assert normwise_err(host(mat)[SUBSET], ref) < TOL
    if not bf16:
        assert normwise_err(host(st_rmw)[SUBSET], ref) < TOL


@pytest.mark.parametrize("batch", [1, 32])
def test_bf16_small_batches(batch):
    sh = wl.M2Shape(batch=batch, nheads=128, ngroups=128, head_dim=64, d_state=128, window=16)
    prm = wl.m2_params(sh, 9)
    s0 = wl.m2_state0(sh, 9)
    ins = wl.m2_token_inputs(sh, 9, 0, ntok=40)
    d = m2_dev_tokens(sh, ins, 40)
    ctx, A, D = _ctx(sh, prm, bf16=True)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64)
    y = torch.empty(batch, 128, 64, device="cuda")
    for t in range(40):
        ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
        y_ref = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        assert normwise_err(host(y), y_ref) < TOL_BF16


@pytest.mark.parametrize("G", [128, 8])
def test_speculative_serving_shape_sampled(G):
    """batch 512, K = 6 drafts per round into the W = 16 ring, censored-geometric acceptance:
    bookkeeping of all 512 sequences bit-exact after every call, outputs of sampled sequences.
    With B / C shared by groups of 16 heads (G = 8), sequences whose drafts do not fit are folded
    by a consolidation launch before the verify, whose draft appends then never overwrite a ring
    slot another head of the group still reads."""
    sh = wl.M2_SPEC if G == 128 else wl.M2Shape(batch=512, nheads=128, ngroups=G, head_dim=64,
                                                  d_state=128, window=16, max_draft=6)
    K, rounds = 6, 24
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    acc = wl.spec_accepted(sh.batch, rounds, K, seed=0)
    ctx, A, D = _ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window, K)
    sub = np.array([0, 5, 300, 511])
    ref = s0[sub].astype(np.float64)
    M = np.abs(ref)
    yk = torch.empty(K, sh.batch, sh.nheads, sh.head_dim, device="cuda")
    worst, worst_ratio, n_over = 0.0, 0.0, 0
    pool = [wl.m2_token_inputs(sh, 0, s, ntok=K) for s in range(3)]
    dpool = [m2_dev_tokens(sh, p, K) for p in pool]
    for r in range(rounds):
        ins = pool[r % 3]
        ctx.verify(yk, **dpool[r % 3])
        model.verify(K)
        _check_bk(ctx, model, 0)
        ctx.commit(dev(acc[r]))
        model.commit(acc[r])
        _check_bk(ctx, model, 0)
        sub_ins = {k: v[:, sub] for k, v in ins.items()}
        y_ref = m2_spec_round(prm["A"], prm["D"], sub_ins, ref, acc[r][sub])
        kap = m2_spec_kappa(prm["A"], prm["D"], sub_ins, M, acc[r][sub])
        c = cond_check(host(yk)[:, sub], y_ref, C_FP32 * U32 * kap, TOL)
        assert c.ok and c.ratio_all <= 1.0, (r, c)
        worst, n_over = max(worst, c.worst), n_over + c.n_over
        worst_ratio = max(worst_ratio, c.ratio_all)
    say(f"  spec G={G}: worst normwise {worst:.3e}, {n_over} head vectors over {TOL:g}, worst "
        f"|d|/bound {worst_ratio:.3f}")


def test_snapshot_comparator_rounds():
    """The conventional speculative comparator: per-draft snapshots in a slot pool, commit by
    pointing each sequence at its accepted snapshot; outputs and committed states against the
    oracle's recomputation from the accepted prefix."""
    sh = wl.M2Shape(batch=5, nheads=2, ngroups=2, head_dim=16, d_state=16, window=8, max_draft=3)
    K = 3
    prm = wl.m2_params(sh, 11)
    s0 = wl.m2_state0(sh, 11)
    cfg = rb.make_config(rb.RSSM_MAMBA2, sh.batch, sh.nheads, sh.ngroups, 16, 16, sh.window, K)
    A, D = dev(prm["A"]), dev(prm["D"])
    pool = torch.zeros((2 * K + 1,) + s0.shape, device="cuda")
    pool[2 * K] = dev(s0)
    slot_of = torch.full((sh.batch,), 2 * K, dtype=torch.int32, device="cuda")
    acc = wl.spec_accepted(sh.batch, 12, K, seed=11)
    ref = s0.astype(np.float64).copy()
    yk = torch.empty(K, sh.batch, sh.nheads, 16, device="cuda")
    for r in range(12):
        ins = wl.m2_token_inputs(sh, 11, r, ntok=K)
        rb.step_baseline_spec(cfg, pool, slot_of, yk, A, D, **m2_dev_tokens(sh, ins, K))
        rb.rssm_baseline_commit(cfg, slot_of, dev(acc[r]), K)
        y_ref = m2_spec_round(prm["A"], prm["D"], ins, ref, acc[r])
        assert normwise_err(host(yk), y_ref) < TOL, r
        sl = host(slot_of)
        st = host(pool)
        committed = np.stack([st[sl[b], b] for b in range(sh.batch)])
        assert normwise_err(committed, ref) < TOL, r


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_conventional_step_over_per_sequence_tiles(kind):
    """rssm_step_baseline_seqs: the conventional step on states kept in scattered per-sequence
    blocks (pointer array), in place and with snapshots, equals the contiguous form bit for bit
    and the oracle within tolerance."""
    B, H, d, W = 5, 3, 16, 4
    if kind == "mamba2":
        sh = wl.M2Shape(batch=B, nheads=H, ngroups=H, head_dim=d, d_state=d, window=W)
        prm = wl.m2_params(sh, 13)
        s0 = wl.m2_state0(sh, 13)
        ins = wl.m2_token_inputs(sh, 13, 0, ntok=4)
        d_in = m2_dev_tokens(sh, ins, 4)
        A, D = dev(prm["A"]), dev(prm["D"])
        cfg = rb.make_config(rb.RSSM_MAMBA2, B, H, H, d, d, W)
    else:
        sh = wl.GDNShape(batch=B, nheads=H, d_k=d, d_v=d, window=W)
        gen = wl.gdn_token_inputs if kind == "gdn" else wl.kda_token_inputs
        s0 = (wl.gdn_state0 if kind == "gdn" else wl.kda_state0)(sh, 13)
        ins = gen(sh, 13, 0, ntok=4)
        d_in = {k: dev(v) for k, v in ins.items()}
        A = D = None
        cfg = rb.make_config(rb.RSSM_GDN if kind == "gdn" else rb.RSSM_KDA, B, H, H, d, d, W)
    # per-sequence blocks scattered in a larger pool, in reverse order with gaps
    pool = torch.zeros(2 * B + 1, H, d, d, device="cuda")
    slots = [2 * (B - 1 - b) + 1 for b in range(B)]
    for b in range(B):
        pool[slots[b]] = dev(s0[b])
    ptrs = torch.tensor([pool[sl].data_ptr() for sl in slots], dtype=torch.int64, device="cuda")
    st = dev(s0)
    y1 = torch.empty(4, B, H, d, device="cuda")
    y2 = torch.empty(4, B, H, d, device="cuda")
    rb.step_baseline(cfg, st, y1, A, D, **d_in)
    rb.step_baseline_seqs(cfg, ptrs, y2, A, D, **d_in)
    assert np.array_equal(host(y1), host(y2))
    got = host(pool)
    for b in range(B):
        assert np.array_equal(got[slots[b]], host(st)[b])
    assert np.count_nonzero(got[[0, 2, 4, 6, 8, 10]]) == 0       # gaps untouched
    snaps = torch.empty(4, B, H, d, d, device="cuda")
    before = host(pool).copy()
    rb.step_baseline_seqs(cfg, ptrs, y2, A, D, snapshots=snaps, **d_in)
    assert np.array_equal(host(pool), before)                    # read-only with snapshots
    ref = s0.astype(np.float64).copy()
    for t in range(4):
        if kind == "mamba2":
            y_ref = m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
        else:
            from oracle import gdn_step, kda_step
            step = gdn_step if kind == "gdn" else kda_step
            y_ref = step(*(ins[k][t] for k in ("q", "k", "v", "beta", "alpha")), ref)
        assert normwise_err(host(y1)[t], y_ref) < TOL, t
