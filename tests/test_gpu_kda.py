"""GPU parity of the Kimi Delta Attention ReplaySSM path (C ABI -> HIP kernels) against the CPU
oracle (a per key channel forget gate in the delta rule). Normwise relative error 1e-5 per head
vector (fp32); at the serving shapes a head vector over it must be within its rounding bound
C_FP32 u32 kappa element by element (kappa from oracle.kda_kappa_step); bookkeeping bit-exact."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import (C_FP32, U32, Bookkeeping, cond_check, kda_kappa_step, kda_spec_kappa,
                    kda_spec_round, kda_step, normwise_err)
from tests.gpu_helpers import dev, host, kda_dev_tokens, kda_kappa_torch, say, tok0

pytestmark = pytest.mark.gpu

TOL = 1e-5
KEYS = ("q", "k", "v", "beta", "alpha")


def _ctx(sh: wl.GDNShape):
    return rb.Context("kda", sh.batch, sh.nheads, sh.d_v, sh.d_k, sh.window, max_draft=sh.max_draft)


def _ref_step(ins, t, ref, sel=slice(None)):
    return kda_step(*(ins[k][t][sel] for k in KEYS), ref)


def _check_bk(ctx, model, err=0):
    h, l, n, e = ctx.bookkeeping()
    mh, ml, mn = model.snapshot()
    assert (h, l, n, e) == (list(mh), list(ml), list(mn), err), (h, l, n, e, mh, ml, mn)


@pytest.mark.parametrize("d,W", [(16, 4), (64, 16), (128, 16), (128, 1), (16, 20), (64, 5),
                                 (128, 32)])
def test_kda_decode_every_call(d, W):
    """Every output, the bookkeeping and the materialised state after every decode step, over
    several windows (W = 1: every token folds; W = 32: the largest ring)."""
    sh = wl.GDNShape(batch=3, nheads=3, d_k=d, d_v=d, window=W)
    T = 3 * W + 5 if W > 1 else 9
    say(f"kda decode d={d} W={W} T={T}")
    s0 = wl.kda_state0(sh, 0)
    ins = wl.kda_token_inputs(sh, 0, 0, ntok=T)
    dd = kda_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    worst = 0.0
    for t in range(T):
        ctx.decode_step(o, **{k: v[t] for k, v in dd.items()})
        o_ref = _ref_step(ins, t, ref)
        model.decode()
        err = normwise_err(host(o), o_ref)
        worst = max(worst, err)
        assert err < TOL, (t, err)
        _check_bk(ctx, model)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, t
    say(f"  worst normwise {worst:.3e}")


@pytest.mark.parametrize("d,W", [(64, 8), (128, 24)])
def test_kda_consolidate_and_masked_init(d, W):
    """Masked re-init (ragged fills), consolidation with a threshold, a full consolidation, the
    materialised state and bookkeeping after every operation."""
    sh = wl.GDNShape(batch=4, nheads=2, d_k=d, d_v=d, window=W)
    say(f"kda consolidate d={d} W={W}")
    s0 = wl.kda_state0(sh, 1)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    sched = (["d"] * (W - 3) + [("mask", [0, 1, 0, 1])] + ["d"] * 2 + [("cons", 3)] + ["d"] * (W + 1)
             + [("cons", 1)] + ["d"] * 3)
    for i, op in enumerate(sched):
        if op == "d":
            ins = wl.kda_token_inputs(sh, 1, 50 + i)
            ctx.decode_step(o, **tok0(kda_dev_tokens(sh, ins, 1)))
            o_ref = _ref_step(ins, 0, ref)
            model.decode()
            assert normwise_err(host(o), o_ref) < TOL, i
        elif op[0] == "mask":
            fresh = wl.kda_state0(sh, 77)
            m = np.array(op[1], dtype=np.int32)
            ctx.init_checkpoint(dev(fresh), dev(m))
            ref[m != 0] = fresh[m != 0]
            model.init(m)
        else:
            ctx.consolidate(op[1])
            model.consolidate(op[1])
        _check_bk(ctx, model)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, i


@pytest.mark.parametrize("d,W,K", [(16, 8, 3), (16, 4, 4), (64, 16, 6), (128, 16, 6),
                                   (128, 24, 8), (64, 1, 1), (16, 20, 17), (64, 32, 20)])
def test_kda_speculative_rounds(d, W, K):
    """Rounds of K drafts committed with seeded, full and empty acceptances or discarded, decode
    steps between some rounds: every draft output, the bookkeeping and the materialised state."""
    sh = wl.GDNShape(batch=4, nheads=2, d_k=d, d_v=d, window=W, max_draft=K)
    say(f"kda verify d={d} W={W} K={K}")
    s0 = wl.kda_state0(sh, 21)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W, K)
    ref = s0.astype(np.float64).copy()
    acc = wl.spec_accepted(sh.batch, 24, K, seed=21)
    ok = torch.empty(K, sh.batch, sh.nheads, d, device="cuda")
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    worst = 0.0
    for r in range(24):
        ins = wl.kda_token_inputs(sh, 21, 300 + r, ntok=K)
        ctx.verify(ok, **kda_dev_tokens(sh, ins, K))
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
        o_ref = kda_spec_round(ins, ref, a)
        err = normwise_err(host(ok), o_ref)
        worst = max(worst, err)
        assert err < TOL, (r, err)
        _check_bk(ctx, model)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, r
        if r % 4 == 3:
            t1 = wl.kda_token_inputs(sh, 21, 700 + r)
            ctx.decode_step(o, **tok0(kda_dev_tokens(sh, t1, 1)))
            model.decode()
            assert normwise_err(host(o), _ref_step(t1, 0, ref)) < TOL, r
            _check_bk(ctx, model)
    say(f"  worst normwise {worst:.3e}")


def test_kda_rollback_prefix_bit_exact():
    """Verify K drafts and commit a, against verify only the first a drafts and commit a: the a
    outputs, bookkeeping, materialised state and later outputs are bit-identical."""
    sh = wl.GDNShape(batch=3, nheads=4, d_k=128, d_v=128, window=16, max_draft=6)
    s0 = dev(wl.kda_state0(sh, 5))
    K, a = 6, 4
    outs = []
    for run in ("A", "B"):
        ctx = _ctx(sh)
        ctx.init_checkpoint(s0)
        o = torch.empty(sh.batch, sh.nheads, 128, device="cuda")
        for t in range(13):
            ctx.decode_step(o, **tok0(kda_dev_tokens(sh, wl.kda_token_inputs(sh, 5, t), 1)))
        ctx.consolidate(sh.window - K + 1)
        ins = wl.kda_token_inputs(sh, 5, 99, ntok=K)
        n = K if run == "A" else a
        ok = torch.empty(n, sh.batch, sh.nheads, 128, device="cuda")
        ctx.verify(ok, **kda_dev_tokens(sh, {k: v[:n] for k, v in ins.items()}, n))
        ctx.commit(dev(np.full(sh.batch, a, dtype=np.int32)))
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        later = []
        for t in range(5):
            ctx.decode_step(o, **tok0(kda_dev_tokens(sh, wl.kda_token_inputs(sh, 5, 300 + t), 1)))
            later.append(host(o).copy())
        outs.append((host(ok)[:a].copy(), ctx.bookkeeping(), host(mat).copy(), later))
    (ya, bka, ma, la), (yb, bkb, mb, lb) = outs
    assert np.array_equal(ya, yb) and bka == bkb and np.array_equal(ma, mb)
    for u, v in zip(la, lb):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("d", [16, 128])
def test_kda_conventional_comparator(d):
    """The conventional kernel in place over single tokens and over a 7-token launch, in snapshot
    mode, and the speculative comparator with its slot pool."""
    sh = wl.GDNShape(batch=3, nheads=2, d_k=d, d_v=d, window=8, max_draft=3)
    s0 = wl.kda_state0(sh, 9)
    cfg = rb.make_config(rb.RSSM_KDA, sh.batch, sh.nheads, sh.nheads, d, d, sh.window, 3)
    ins = wl.kda_token_inputs(sh, 9, 0, ntok=10)
    dd = kda_dev_tokens(sh, ins, 10)
    st = dev(s0)
    ref = s0.astype(np.float64).copy()
    o1 = torch.empty(1, sh.batch, sh.nheads, d, device="cuda")
    for t in range(3):
        rb.step_baseline(cfg, st, o1, **{k: v[t:t + 1] for k, v in dd.items()})
        assert normwise_err(host(o1)[0], _ref_step(ins, t, ref)) < TOL, t
    o7 = torch.empty(7, sh.batch, sh.nheads, d, device="cuda")
    rb.step_baseline(cfg, st, o7, **{k: v[3:10] for k, v in dd.items()})
    for t in range(3, 10):
        assert normwise_err(host(o7)[t - 3], _ref_step(ins, t, ref)) < TOL, t
    assert normwise_err(host(st), ref) < TOL
    K = 3
    snaps = torch.empty((K,) + s0.shape, device="cuda")
    ok = torch.empty(K, sh.batch, sh.nheads, d, device="cuda")
    before = host(st).copy()
    dr = wl.kda_token_inputs(sh, 9, 1, ntok=K)
    rb.step_baseline(cfg, st, ok, snapshots=snaps, **kda_dev_tokens(sh, dr, K))
    assert np.array_equal(host(st), before)
    r2 = before.astype(np.float64)
    for k in range(K):
        assert normwise_err(host(ok)[k], _ref_step(dr, k, r2)) < TOL
        assert normwise_err(host(snaps)[k], r2) < TOL
    pool = torch.zeros((2 * K + 1,) + s0.shape, device="cuda")
    pool[2 * K] = dev(s0)
    slot_of = torch.full((sh.batch,), 2 * K, dtype=torch.int32, device="cuda")
    acc = wl.spec_accepted(sh.batch, 8, K, seed=9)
    ref = s0.astype(np.float64).copy()
    for r in range(8):
        dr = wl.kda_token_inputs(sh, 9, 20 + r, ntok=K)
        rb.step_baseline_spec(cfg, pool, slot_of, ok, **kda_dev_tokens(sh, dr, K))
        rb.rssm_baseline_commit(cfg, slot_of, dev(acc[r]), K)
        o_ref = kda_spec_round(dr, ref, acc[r])
        assert normwise_err(host(ok), o_ref) < TOL, r
        sl = host(slot_of)
        stp = host(pool)
        assert normwise_err(np.stack([stp[sl[b], b] for b in range(sh.batch)]), ref) < TOL, r


def test_kda_fork_export_import():
    """Per-sequence copies carry the gate rows: a forked sequence continues exactly like its
    source, and an exported then re-imported sequence continues as before."""
    sh = wl.GDNShape(batch=3, nheads=2, d_k=64, d_v=64, window=8)
    s0 = wl.kda_state0(sh, 11)
    ins = wl.kda_token_inputs(sh, 11, 0, ntok=20)
    dd = kda_dev_tokens(sh, ins, 20)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
    for t in range(11):                     # one fold, then 3 buffered entries
        ctx.decode_step(o, **{k: v[t] for k, v in dd.items()})
    ctx.fork(torch.tensor([1], dtype=torch.int32, device="cuda"),
             torch.tensor([2], dtype=torch.int32, device="cuda"))
    nbytes = ctx.seq_state_bytes()
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    ctx.export(torch.tensor([0], dtype=torch.int32, device="cuda"), buf)
    perm = torch.tensor([0, 1, 1], device="cuda")
    outs = []
    for t in range(11, 20):
        tok = {k: v[t].index_select(0, perm).contiguous() for k, v in dd.items()}
        ctx.decode_step(o, **tok)
        oh = host(o)
        assert np.array_equal(oh[1], oh[2]), t
        outs.append(oh[0].copy())
    ctx.import_(torch.tensor([0], dtype=torch.int32, device="cuda"), buf)
    h, l, n, e = ctx.bookkeeping()
    assert e == 0
    for i, t in enumerate(range(11, 20)):
        tok = {k: v[t].index_select(0, perm).contiguous() for k, v in dd.items()}
        ctx.decode_step(o, **tok)
        assert np.array_equal(host(o)[0], outs[i]), t


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("T", [1, 16, 37])
def test_kda_prefill(d, T):
    """Every compiled head shape; prompts of one token, one full 16-token chunk and a ragged
    three-chunk prompt into the checkpoint; the outputs, the state and the bookkeeping against the
    oracle, then 5 decode steps from the new checkpoint."""
    sh = wl.GDNShape(batch=2, nheads=3, d_k=d, d_v=d, window=8)
    say(f"kda prefill d={d} T={T}")
    s0 = wl.kda_state0(sh, 4)
    ins = wl.kda_token_inputs(sh, 4, 0, ntok=T + 5)
    dd = kda_dev_tokens(sh, ins, T + 5)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    o = torch.empty(T, sh.batch, sh.nheads, d, device="cuda")
    ctx.prefill(o, **{k: v[:T] for k, v in dd.items()})
    o_ref = np.stack([_ref_step(ins, t, ref) for t in range(T)])
    err = normwise_err(host(o), o_ref)
    assert err < TOL, err
    h, l, n, e = ctx.bookkeeping()
    assert l == [0] * sh.batch and n == [0] * sh.batch and e == 0
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat), ref) < TOL
    o1 = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    for t in range(T, T + 5):
        ctx.decode_step(o1, **tok0({k: v[t:t + 1] for k, v in dd.items()}))
        assert normwise_err(host(o1), _ref_step(ins, t, ref)) < TOL, t
    say(f"  prompt outputs {err:.3e}")


def test_kda_prefill_after_buffered_entries():
    """Buffered entries are folded first: 5 decode steps, then a 20-token prompt, then a second
    prompt continuing the same state, against the oracle run over the same tokens."""
    sh = wl.GDNShape(batch=3, nheads=2, d_k=64, d_v=64, window=8)
    s0 = wl.kda_state0(sh, 5)
    ins = wl.kda_token_inputs(sh, 5, 0, ntok=45)
    dd = kda_dev_tokens(sh, ins, 45)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    o1 = torch.empty(sh.batch, sh.nheads, 64, device="cuda")
    for t in range(5):
        ctx.decode_step(o1, **tok0({k: v[t:t + 1] for k, v in dd.items()}))
        _ref_step(ins, t, ref)
    for lo in (5, 25):
        o = torch.empty(20, sh.batch, sh.nheads, 64, device="cuda")
        ctx.prefill(o, **{k: v[lo:lo + 20] for k, v in dd.items()})
        o_ref = np.stack([_ref_step(ins, t, ref) for t in range(lo, lo + 20)])
        assert normwise_err(host(o), o_ref) < TOL, lo
        mat = torch.empty(s0.shape, device="cuda")
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, lo
        h, l, n, e = ctx.bookkeeping()
        assert l == [0] * sh.batch and e == 0


@pytest.mark.parametrize("d", [16, 64, 128])
def test_kda_fold_vector_path_windows(d):
    """Windows whose gate product in some key channel falls below 2^-64 (a run of gates 1e-6 in a
    few channels, one gate of exactly 0) are folded entry by entry on the vector units, the rest of
    the same launches on the matrix cores: every output, the materialised state (which folds the
    buffered entries) and the bookkeeping after every step, W = 16."""
    sh = wl.GDNShape(batch=2, nheads=3, d_k=d, d_v=d, window=16)
    T = 40
    say(f"kda fold vector-path windows d={d}")
    s0 = wl.kda_state0(sh, 8)
    ins = wl.kda_token_inputs(sh, 8, 0, ntok=T)
    ins["alpha"][3:12, 0, 1, :3] = 1e-6         # first window of tile (0, 1)
    ins["alpha"][20, 1, 2, d - 1] = 0.0         # second window of tile (1, 2)
    dd = kda_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window)
    ref = s0.astype(np.float64).copy()
    o = torch.empty(sh.batch, sh.nheads, d, device="cuda")
    mat = torch.empty(s0.shape, device="cuda")
    for t in range(T):
        ctx.decode_step(o, **{k: v[t] for k, v in dd.items()})
        o_ref = _ref_step(ins, t, ref)
        model.decode()
        assert normwise_err(host(o), o_ref) < TOL, t
        _check_bk(ctx, model)
        ctx.materialize(mat)
        assert normwise_err(host(mat), ref) < TOL, t


def _prefill_against_oracle(sh, s0, ins, T):
    dd = kda_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    o = torch.empty(T, sh.batch, sh.nheads, sh.d_v, device="cuda")
    ctx.prefill(o, **dd)
    o_ref = np.stack([_ref_step(ins, t, ref) for t in range(T)])
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    return host(o), o_ref, host(mat), ref


@pytest.mark.parametrize("d", [16, 64, 128])
def test_kda_prefill_token_path_chunks(d):
    """Chunks whose gate product in some channel falls below 2^-64 (a run of gates 1e-5 in a few
    channels, a single gate of exactly 0) go through the token-by-token path; the other tiles and
    chunks of the same launch take the matrix-core form. Outputs and state against the oracle."""
    sh = wl.GDNShape(batch=2, nheads=3, d_k=d, d_v=d, window=8)
    T = 53
    say(f"kda prefill token-path chunks d={d}")
    s0 = wl.kda_state0(sh, 6)
    ins = wl.kda_token_inputs(sh, 6, 0, ntok=T)
    ins["alpha"][16:32, 0, 1, :5] = 1e-5        # chunk 1 of tile (0, 1)
    ins["alpha"][40, 1, 2, d - 1] = 0.0         # chunk 2 of tile (1, 2)
    ins["alpha"][50, 0, 0, 3] = 0.0             # the ragged last chunk of tile (0, 0)
    oh, o_ref, mh, ref = _prefill_against_oracle(sh, s0, ins, T)
    assert normwise_err(oh, o_ref) < TOL
    assert normwise_err(mh, ref) < TOL


@pytest.mark.parametrize("d", [64, 128])
def test_kda_prefill_strong_gates(d):
    """Every gate 0.07: the chunk products reach 0.07^16 ~ 2^-61, just inside the matrix-core form
    (1 / Gam up to 2^61 on one operand); outputs and state against the oracle."""
    sh = wl.GDNShape(batch=2, nheads=2, d_k=d, d_v=d, window=8)
    T = 40
    say(f"kda prefill strong gates d={d}")
    s0 = wl.kda_state0(sh, 7)
    ins = wl.kda_token_inputs(sh, 7, 0, ntok=T)
    ins["alpha"][:] = np.float32(0.07)
    oh, o_ref, mh, ref = _prefill_against_oracle(sh, s0, ins, T)
    assert normwise_err(oh, o_ref) < TOL
    assert normwise_err(mh, ref) < TOL


def test_kda_prefill_serving_shape_sampled():
    """Batch 256, 32 heads, 128x128, a 64-token prompt: the outputs of sampled sequences against the
    oracle, and every sequence against 64 decode steps of the same tokens on the GPU, each within
    its rounding bound where the normwise criterion does not hold."""
    sh = wl.KDA_SERVE
    T = 64
    say("kda prefill serving shape: generating inputs")
    s0 = wl.kda_state0(sh, 0)
    ins = wl.kda_token_inputs(sh, 0, 100, ntok=T)
    dd = kda_dev_tokens(sh, ins, T)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(T, sh.batch, sh.nheads, sh.d_v, device="cuda")
    ctx.prefill(o, **dd)
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
        tok = tok0({k: v[t:t + 1] for k, v in dd.items()})
        ctx2.decode_step(o1, **tok)
        kap = host(kda_kappa_torch(kap_state, tok["q"], tok["k"], tok["v"], tok["beta"], tok["alpha"]))
        o1h = host(o1)
        od[t] = o1h[sub]
        pair.append(cond_check(oh[t], o1h, 2 * C_FP32 * U32 * kap, 2 * TOL))
    ref = s0[sub].astype(np.float64)
    M = np.abs(ref)
    o_ref, kref = [], []
    for t in range(T):
        a = [ins[k][t][sub] for k in KEYS]
        o_ref.append(kda_step(*a, ref))
        kref.append(kda_kappa_step(*a, M))
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


# ---------------------------------------------------------------------------------------------
# serving shapes: batch 256 x 32 heads, 128 x 128, W = 16; speculative batch 512, K = 6
# ---------------------------------------------------------------------------------------------

def test_kda_serving_shape_sampled():
    """Batch 256, 32 heads, 128 x 128, W = 16, 512 steps over a 32-slot token pool (the
    benchmark's schedule): sampled sequences against the oracle every step, every sequence against
    the conventional kernel every 32 steps, the materialised state and bookkeeping at the end."""
    sh = wl.KDA_SERVE
    steps, pool_n = 512, 32
    say("kda serving shape: generating inputs")
    s0 = wl.kda_state0(sh, 0)
    slots = [wl.kda_token_inputs(sh, 0, s) for s in range(pool_n)]
    dslots = [tok0(kda_dev_tokens(sh, s, 1)) for s in slots]
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    cfg = rb.make_config(rb.RSSM_KDA, sh.batch, sh.nheads, sh.nheads, sh.d_v, sh.d_k, sh.window)
    st = dev(s0)
    kap_state = dev(np.abs(s0))
    sub = np.array([0, 3, 128, 255])
    subt = torch.from_numpy(sub).cuda()
    o = torch.empty(sh.batch, sh.nheads, sh.d_v, device="cuda")
    o2 = torch.empty(1, sh.batch, sh.nheads, sh.d_v, device="cuda")
    os_ = torch.empty(steps, len(sub), sh.nheads, sh.d_v, device="cuda")
    pair = []
    for t in range(steps):
        tok = dslots[t % pool_n]
        ctx.decode_step(o, **tok)
        os_[t] = o.index_select(0, subt)
        rb.step_baseline(cfg, st, o2, **{k: v.unsqueeze(0) for k, v in tok.items()})
        kap = kda_kappa_torch(kap_state, *(tok[k] for k in KEYS))
        if t % 32 == 31:
            pair.append(cond_check(host(o), host(o2)[0], 2 * C_FP32 * U32 * host(kap), 2 * TOL))
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    h, l, n, e = ctx.bookkeeping()
    assert l == [steps % sh.window] * sh.batch and e == 0
    say("  oracle on the sampled sequences")
    ref = s0[sub].astype(np.float64)
    M = np.abs(ref)
    oh = host(os_)
    worst, ratio, n_over = 0.0, 0.0, 0
    for t in range(steps):
        a = [slots[t % pool_n][k][0][sub] for k in KEYS]
        o_ref = kda_step(*a, ref)
        kap = kda_kappa_step(*a, M)
        c = cond_check(oh[t], o_ref, C_FP32 * U32 * kap, TOL)
        assert c.ok and c.ratio_all <= 1.0, (t, c)
        worst, n_over, ratio = max(worst, c.worst), n_over + c.n_over, max(ratio, c.ratio_all)
    say(f"  worst normwise {worst:.3e}, {n_over} head vectors over {TOL:g}, worst |d|/bound "
        f"{ratio:.3f}")
    for c in pair:
        say(f"  replay vs conventional kernel, all sequences: {c}")
        assert c.ok and c.ratio_all <= 1.0
    assert normwise_err(host(mat)[sub], ref) < TOL
    assert normwise_err(host(st)[sub], ref) < TOL


def test_kda_speculative_serving_shape_sampled():
    """Batch 512, 32 heads, 128 x 128, K = 6 drafts into the W = 16 ring, censored-geometric
    acceptance, 24 rounds: bookkeeping of every sequence bit-exact after every call, outputs of
    sampled sequences against the oracle's recomputation."""
    sh = wl.GDNShape(batch=512, nheads=32, d_k=128, d_v=128, window=16, max_draft=6)
    K, rounds = 6, 24
    s0 = wl.kda_state0(sh, 0)
    acc = wl.spec_accepted(sh.batch, rounds, K, seed=0)
    ctx = _ctx(sh)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, sh.window, K)
    sub = np.array([0, 7, 300, 511])
    ref = s0[sub].astype(np.float64)
    M = np.abs(ref)
    ok = torch.empty(K, sh.batch, sh.nheads, sh.d_v, device="cuda")
    pool = [wl.kda_token_inputs(sh, 0, s, ntok=K) for s in range(3)]
    dpool = [kda_dev_tokens(sh, p, K) for p in pool]
    worst, ratio = 0.0, 0.0
    for r in range(rounds):
        ins = pool[r % 3]
        ctx.verify(ok, **dpool[r % 3])
        model.verify(K)
        _check_bk(ctx, model)
        ctx.commit(dev(acc[r]))
        model.commit(acc[r])
        _check_bk(ctx, model)
        sub_ins = {k: v[:, sub] for k, v in ins.items()}
        o_ref = kda_spec_round(sub_ins, ref, acc[r][sub])
        kap = kda_spec_kappa(sub_ins, M, acc[r][sub])
        c = cond_check(host(ok)[:, sub], o_ref, C_FP32 * U32 * kap, TOL)
        assert c.ok and c.ratio_all <= 1.0, (r, c)
        worst, ratio = max(worst, c.worst), max(ratio, c.ratio_all)
    say(f"  kda spec worst normwise {worst:.3e}, worst |d|/bound {ratio:.3f}")
