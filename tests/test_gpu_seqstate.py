"""GPU tests of the per-sequence state copies (rssm_fork / rssm_export / rssm_import) through the C
ABI: a forked or re-imported sequence continues exactly like its source (bit-exact outputs, state
and bookkeeping), and matches the oracle's recurrence; bad indices only set the device error bit."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import gdn_step, m2_step, normwise_err
from tests.gpu_helpers import dev, gdn_dev_tokens, host, m2_dev_tokens, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _m2_ctx(sh, prm, bf16=False):
    c = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                   ngroups=sh.ngroups, max_draft=sh.max_draft, bf16_read=bf16)
    c.set_params(dev(prm["A"]), dev(prm["D"]))
    return c


def _i32(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


def _tok(d, t, perm=None):
    """Token t of device inputs, with the batch rows permuted by perm (sequence b takes row
    perm[b]) so that a fork destination can be fed its source's tokens."""
    tok = {k: v[t] for k, v in d.items()}
    if perm is not None:
        p = torch.tensor(perm, device="cuda")
        tok = {k: v.index_select(0, p).contiguous() for k, v in tok.items()}
    return tok


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("P,N,G", [(16, 16, 2), (64, 128, 4)])
def test_fork_continues_like_source(bf16, P, N, G):
    sh = wl.M2Shape(batch=4, nheads=4, ngroups=G, head_dim=P, d_state=N, window=8)
    say(f"fork P={P} N={N} G={G} bf16={bf16}")
    prm = wl.m2_params(sh, 3)
    s0 = wl.m2_state0(sh, 3)
    ins = wl.m2_token_inputs(sh, 3, 0, ntok=30)
    d = m2_dev_tokens(sh, ins, 30)
    ctx = _m2_ctx(sh, prm, bf16)
    ctx.init_checkpoint(dev(s0))
    y = torch.empty(sh.batch, sh.nheads, P, device="cuda")
    for t in range(11):                     # one fold, then 3 buffered entries
        ctx.decode_step(y, **_tok(d, t))
    ctx.init_checkpoint(dev(wl.m2_state0(sh, 4)), dev(np.array([0, 1, 0, 0], np.int32)))
    ctx.decode_step(y, **_tok(d, 11))       # lengths now 4, 1, 4, 4
    ctx.fork(_i32([0, 1]), _i32([2, 3]))
    h, l, n, e = ctx.bookkeeping()
    assert (h[2], l[2], h[3], l[3]) == (h[0], l[0], h[1], l[1]) and e == 0
    m = torch.empty(s0.shape, device="cuda")
    ctx.materialize(m)
    mh = host(m)
    assert np.array_equal(mh[2], mh[0]) and np.array_equal(mh[3], mh[1])
    perm = [0, 1, 0, 1]                     # sequences 2, 3 take the tokens of 0, 1
    for t in range(12, 30):
        ctx.decode_step(y, **_tok(d, t, perm))
        yh = host(y)
        assert np.array_equal(yh[2], yh[0]) and np.array_equal(yh[3], yh[1]), t
    ctx.materialize(m)
    mh = host(m)
    assert np.array_equal(mh[2], mh[0]) and np.array_equal(mh[3], mh[1])


def test_export_import_restores_state():
    """Export two sequences, decode on, import them back (once into their own slots, once into
    other slots): the state, the bookkeeping and every later output equal those at the export,
    and the outputs match the oracle continued from the exported state."""
    sh = wl.M2Shape(batch=4, nheads=4, ngroups=4, head_dim=32, d_state=32, window=8, max_draft=3)
    prm = wl.m2_params(sh, 5)
    s0 = wl.m2_state0(sh, 5)
    ins = wl.m2_token_inputs(sh, 5, 0, ntok=40)
    d = m2_dev_tokens(sh, ins, 40)
    ctx = _m2_ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    y = torch.empty(sh.batch, sh.nheads, 32, device="cuda")
    for t in range(13):
        ctx.decode_step(y, **_tok(d, t))
        m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)
    nbytes = ctx.seq_state_bytes()
    buf = torch.empty(2 * nbytes, dtype=torch.uint8, device="cuda")
    ctx.export(_i32([1, 3]), buf)
    m = torch.empty(s0.shape, device="cuda")
    ctx.materialize(m)
    snap = host(m)
    bk_snap = ctx.bookkeeping()
    ref_snap = ref.copy()
    with pytest.raises(rb.RssmError):        # no snapshots while drafts are pending
        ctx.verify(torch.empty(2, sh.batch, sh.nheads, 32, device="cuda"),
                   **{k: v[13:15] for k, v in d.items()})
        ctx.export(_i32([0]), buf)
    ctx.rollback(_i32(bk_snap[1]))           # discard the drafts (lengths unchanged)
    for t in range(15, 20):
        ctx.decode_step(y, **_tok(d, t))
    ctx.import_(_i32([1, 3]), buf)           # back into their own slots
    ctx.materialize(m)
    mh = host(m)
    assert np.array_equal(mh[1], snap[1]) and np.array_equal(mh[3], snap[3])
    h, l, n, e = ctx.bookkeeping()
    assert (h[1], l[1], h[3], l[3]) == (bk_snap[0][1], bk_snap[1][1], bk_snap[0][3], bk_snap[1][3])
    ctx.import_(_i32([0, 2]), buf)           # and into other slots: 0 <- 1, 2 <- 3
    ctx.materialize(m)
    mh = host(m)
    assert np.array_equal(mh[0], snap[1]) and np.array_equal(mh[2], snap[3])
    # continue all four from the snapshot with the tokens of sequences 1 and 3
    perm = [1, 1, 3, 3]
    refc = ref_snap[perm].copy()
    for t in range(20, 32):
        ctx.decode_step(y, **_tok(d, t, perm))
        yr = m2_step(prm["A"], prm["D"], ins["x"][t][perm], ins["B"][t][perm], ins["C"][t][perm],
                     ins["dt"][t][perm], refc)
        yh = host(y)
        assert np.array_equal(yh[0], yh[1]) and np.array_equal(yh[2], yh[3]), t
        assert normwise_err(yh, yr) < TOL, t


def test_bad_indices_set_error_bit():
    sh = wl.M2Shape(batch=3, nheads=2, ngroups=2, head_dim=16, d_state=16, window=4)
    prm = wl.m2_params(sh, 6)
    s0 = wl.m2_state0(sh, 6)
    ins = wl.m2_token_inputs(sh, 6, 0, ntok=2)
    d = m2_dev_tokens(sh, ins, 2)
    ctx = _m2_ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    y = torch.empty(sh.batch, sh.nheads, 16, device="cuda")
    ctx.decode_step(y, **_tok(d, 0))
    m = torch.empty(s0.shape, device="cuda")
    ctx.materialize(m)
    before = host(m)
    bk_before = ctx.bookkeeping()
    ctx.fork(_i32([-1, 0]), _i32([1, 3]))    # both pairs out of range
    h, l, n, e = ctx.bookkeeping()
    assert e == 8 and (h, l, n) == bk_before[:3]
    ctx.materialize(m)
    assert np.array_equal(host(m), before)
    ctx.fork(_i32([0]), _i32([2]))           # a valid pair still works, error word was cleared
    h, l, n, e = ctx.bookkeeping()
    assert e == 0 and (h[2], l[2]) == (h[0], l[0])


def test_import_rejects_bad_headers():
    """A packed slot whose header an export could not have written (head outside [0, W), len
    outside [0, W], pending drafts) is not imported: the device error bit is set and the sequence
    keeps its state and bookkeeping; the valid slots of the same call are imported."""
    sh = wl.M2Shape(batch=4, nheads=2, ngroups=2, head_dim=16, d_state=16, window=4)
    prm = wl.m2_params(sh, 8)
    s0 = wl.m2_state0(sh, 8)
    ins = wl.m2_token_inputs(sh, 8, 0, ntok=3)
    d = m2_dev_tokens(sh, ins, 3)
    ctx = _m2_ctx(sh, prm)
    ctx.init_checkpoint(dev(s0))
    y = torch.empty(sh.batch, sh.nheads, 16, device="cuda")
    for t in range(3):
        ctx.decode_step(y, **_tok(d, t))
    nbytes = ctx.seq_state_bytes()
    buf = torch.zeros(4 * nbytes // 4, dtype=torch.float32, device="cuda")
    ctx.export(_i32([0, 0, 0, 0]), buf)      # four copies of sequence 0 (len 3)
    hdr = buf.view(torch.int32).view(4, nbytes // 4)
    hdr[0, 0] = sh.window                    # head out of range
    hdr[1, 1] = sh.window + 1                # len out of range
    hdr[2, 2] = 1                            # pending drafts
    ctx2 = _m2_ctx(sh, prm)
    ctx2.init_checkpoint(dev(wl.m2_state0(sh, 9)))
    m = torch.empty(s0.shape, device="cuda")
    ctx2.materialize(m)
    before = host(m).copy()
    ctx2.import_(_i32([0, 1, 2, 3]), buf)
    h, l, n, e = ctx2.bookkeeping()
    assert e == rb.RSSM_DEV_IMPORT_HEADER
    assert (h[:3], l[:3], n[:3]) == ([0, 0, 0], [0, 0, 0], [0, 0, 0]) and l[3] == 3
    ctx2.materialize(m)
    after = host(m)
    assert np.array_equal(after[:3], before[:3])
    ctx.materialize(m)
    assert np.array_equal(after[3], host(m)[0])


@pytest.mark.parametrize("dd,W", [(16, 4), (128, 16)])
def test_gdn_fork(dd, W):
    sh = wl.GDNShape(batch=3, nheads=2, d_k=dd, d_v=dd, window=W)
    s0 = wl.gdn_state0(sh, 7)
    ins = wl.gdn_token_inputs(sh, 7, 0, ntok=3 * W)
    d = gdn_dev_tokens(sh, ins, 3 * W)
    ctx = rb.Context("gdn", sh.batch, sh.nheads, dd, dd, W)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(sh.batch, sh.nheads, dd, device="cuda")
    ref = s0.astype(np.float64).copy()
    for t in range(W + 2):
        ctx.decode_step(o, **_tok(d, t))
        gdn_step(ins["q"][t], ins["k"][t], ins["v"][t], ins["beta"][t], ins["alpha"][t], ref)
    ctx.fork(_i32([1]), _i32([2]))
    perm = [0, 1, 1]
    ref = ref[perm].copy()
    for t in range(W + 2, 3 * W):
        ctx.decode_step(o, **_tok(d, t, perm))
        orf = gdn_step(ins["q"][t][perm], ins["k"][t][perm], ins["v"][t][perm], ins["beta"][t][perm],
                       ins["alpha"][t][perm], ref)
        oh = host(o)
        assert np.array_equal(oh[2], oh[1]), t
        assert normwise_err(oh, orf) < TOL, t
