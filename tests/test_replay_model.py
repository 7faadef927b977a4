"""Invariants that tie the CPU replay-form model (checkpoint + ring) to the conventional oracle,
and the integer bookkeeping model to a hand-derived trace. All CPU.

* replayed outputs equal conventional decoding up to floating point;
* a ring of length 1 reduces to the conventional step;
* the checkpoint after a fold equals the sequential state;
* rollback / commit of an accepted prefix equals recomputation from that prefix;
* outputs do not depend on the consolidation schedule (W);
* the bf16 read copy stays within its rounding bound and does not drift.
"""
import json
import os

import numpy as np
import pytest

import workloads as wl
from oracle import (Bookkeeping, GDNReplay, M2Replay, StateError, gdn_conventional, gdn_step,
                    gdn_wy_fold, m2_conventional, m2_spec_round, m2_step, normwise_err, token,
                    gdn_spec_round, gdn_replay_output)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c0(T=64, W=4, G=4, seed=0):
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=G, head_dim=16, d_state=16, window=W)
    prm = wl.m2_params(sh, seed)
    s0 = wl.m2_state0(sh, seed)
    ins = wl.m2_token_inputs(sh, seed, 0, ntok=T)
    return sh, prm, s0, ins


def _toks(ins):
    return [token(ins, t) for t in range(next(iter(ins.values())).shape[0])]


@pytest.mark.parametrize("G", [4, 2, 1])
def test_replay_equals_conventional(oracle_lib, G):
    sh, prm, s0, ins = _c0(G=G)
    y_ref, st_ref = m2_conventional(prm["A"], prm["D"], _toks(ins), s0)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, sh.window)
    y = np.stack([rp.decode(t) for t in _toks(ins)])
    assert normwise_err(y, y_ref) < 1e-12
    assert normwise_err(rp.materialize(), st_ref) < 1e-12


def test_window_one_is_conventional(oracle_lib):
    sh, prm, s0, ins = _c0(T=12, W=1)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 1)
    st = s0.astype(np.float64).copy()
    for t in _toks(ins):
        y = rp.decode(t)
        y_ref = m2_step(prm["A"], prm["D"], t["x"], t["B"], t["C"], t["dt"], st)
        assert int(rp.bk.len.max()) == 0
        assert np.max(np.abs(rp.S0 - st)) < 1e-14
        assert normwise_err(y, y_ref) < 1e-14


def test_fold_equals_sequential_steps(oracle_lib):
    sh, prm, s0, ins = _c0(T=20, W=4)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 4)
    st = s0.astype(np.float64).copy()
    for i, t in enumerate(_toks(ins)):
        rp.decode(t)
        m2_step(prm["A"], prm["D"], t["x"], t["B"], t["C"], t["dt"], st)
        assert normwise_err(rp.materialize(), st) < 1e-13
        if (i + 1) % 4 == 0:          # the step that fills the ring folds it into S0
            assert int(rp.bk.len.max()) == 0
            assert normwise_err(rp.S0, st) < 1e-13


@pytest.mark.parametrize("W", [1, 2, 3, 16, 65])
def test_schedule_invariance(oracle_lib, W):
    sh, prm, s0, ins = _c0(T=40, W=4)
    y_ref, _ = m2_conventional(prm["A"], prm["D"], _toks(ins), s0)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, W)
    y = np.stack([rp.decode(t) for t in _toks(ins)])
    assert normwise_err(y, y_ref) < 1e-12


def test_consolidate_partial(oracle_lib):
    sh, prm, s0, ins = _c0(T=7, W=4)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 4)
    st = s0.astype(np.float64).copy()
    for t in _toks(ins)[:6]:
        rp.decode(t)
        m2_step(prm["A"], prm["D"], t["x"], t["B"], t["C"], t["dt"], st)
    assert list(rp.bk.len) == [2, 2]
    rp.consolidate(2)
    assert list(rp.bk.len) == [0, 0] and list(rp.bk.head) == [2, 2]
    assert normwise_err(rp.S0, st) < 1e-13
    t = _toks(ins)[6]
    y = rp.decode(t)
    assert normwise_err(y, m2_step(prm["A"], prm["D"], t["x"], t["B"], t["C"], t["dt"], st)) < 1e-12


@pytest.mark.parametrize("W,K", [(4, 2), (6, 3), (16, 6)])
def test_rollback_equals_recompute(oracle_lib, W, K):
    sh = wl.M2Shape(batch=5, nheads=2, ngroups=2, head_dim=8, d_state=8, window=W, max_draft=K)
    prm = wl.m2_params(sh, 1)
    s0 = wl.m2_state0(sh, 1)
    rounds = 12
    acc = wl.spec_accepted(sh.batch, rounds, K, seed=1)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, W, max_draft=K)
    st = s0.astype(np.float64).copy()
    for r in range(rounds):
        d = wl.m2_token_inputs(sh, 1, r, ntok=K)
        y = rp.verify(d)
        y_ref = m2_spec_round(prm["A"], prm["D"], d, st, acc[r])
        assert normwise_err(y, y_ref) < 1e-12
        rp.commit(acc[r])
        assert normwise_err(rp.materialize(), st) < 1e-12
        assert int(rp.bk.len.max()) <= W
        # a normal decode step after the round also agrees
        t = token(wl.m2_token_inputs(sh, 1, 100 + r), 0)
        yd = rp.decode(t)
        assert normwise_err(yd, m2_step(prm["A"], prm["D"], t["x"], t["B"], t["C"], t["dt"], st)) < 1e-12
    assert rp.bk.read_err() == 0


def test_rollback_to_prefix_equals_shorter_run(oracle_lib):
    sh, prm, s0, ins = _c0(T=3, W=8)
    a = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 8)
    b = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 8)
    toks = _toks(ins)
    for t in toks:
        a.decode(t)
    a.rollback([1, 1])
    b.decode(toks[0])
    assert np.array_equal(a.materialize(), b.materialize())
    t2 = token(wl.m2_token_inputs(sh, 0, 9), 0)
    assert np.array_equal(a.decode(t2), b.decode(t2))


def test_bf16_read_bound_and_no_drift(oracle_lib):
    sh, prm, s0, ins = _c0(T=128, W=4)
    y_ref, _ = m2_conventional(prm["A"], prm["D"], _toks(ins), s0)
    rp = M2Replay(prm["A"], prm["D"], s0, sh.ngroups, 4, bf16_read=True)
    errs = []
    for i, t in enumerate(_toks(ins)):
        n = rp.bk.len.copy()
        S0 = rp.S0.copy()
        y = rp.decode(t)
        # per element: |dy| <= (window decay) 2^-8 sum_n |S0[p,n]| |C_n| + 1e-12 |y|max
        for b in range(2):
            if n[b] + 1 >= 4:
                continue          # the folding step reads the fresh fp32 checkpoint
            for h in range(4):
                m = n[b] + 1
                dts = [rp.rdt[b, h, (rp.bk.head[b] + j) % 4] for j in range(m - 1)] + [t["dt"][b, h]]
                lam = np.exp(np.sum(np.asarray(dts, dtype=np.float64)) * float(prm["A"][h]))
                bound = lam * 2.0 ** -8 * (np.abs(S0[b, h]) @ np.abs(t["C"][b, h].astype(np.float64)))
                assert np.all(np.abs(y[b, h] - y_ref[i, b, h]) <= bound + 1e-12 * np.max(np.abs(y_ref[i, b, h])))
        errs.append(normwise_err(y, y_ref[i]))
    assert max(errs) < 2e-2
    assert max(errs[-32:]) <= max(errs[:32])


# ---------------------------------------------------------------- Gated DeltaNet replay

def _gdn(T=40, W=4, d=16, seed=0):
    sh = wl.GDNShape(batch=2, nheads=3, d_k=d, d_v=d, window=W)
    return sh, wl.gdn_state0(sh, seed), wl.gdn_token_inputs(sh, seed, 0, ntok=T)


@pytest.mark.parametrize("W", [1, 4, 16])
def test_gdn_replay_equals_conventional(oracle_lib, W):
    sh, s0, ins = _gdn(W=W)
    o_ref, st_ref = gdn_conventional(_toks(ins), s0)
    rp = GDNReplay(s0, W)
    o = np.stack([rp.decode(t) for t in _toks(ins)])
    assert normwise_err(o, o_ref) < 1e-12
    assert normwise_err(rp.materialize(), st_ref) < 1e-12


def test_gdn_spec_round_pins(oracle_lib):
    """Each draft's output of the recomputed round equals the replay formula applied to the
    committed state with drafts 0..k as the only entries (a different formulation of the same
    state); all drafts accepted equals K conventional steps; none accepted leaves the state."""
    sh = wl.GDNShape(batch=3, nheads=2, d_k=8, d_v=6, window=8)
    s0 = wl.gdn_state0(sh, 3).astype(np.float64)
    K = 4
    d = wl.gdn_token_inputs(sh, 3, 0, ntok=K)
    st = s0.copy()
    acc = np.array([K, 0, 2])
    o = gdn_spec_round(d, st, acc)
    for b in range(sh.batch):
        for h in range(sh.nheads):
            for k in range(K):
                ref = gdn_replay_output(s0[b, h], d["k"][:k + 1, b, h], d["v"][:k + 1, b, h],
                                        d["beta"][:k + 1, b, h], d["alpha"][:k + 1, b, h],
                                        d["q"][k, b, h])
                assert np.abs(o[k, b, h] - ref).max() < 1e-12 * max(1.0, np.abs(ref).max())
    o_all, st_all = gdn_conventional(_toks(d), s0)
    assert np.array_equal(o, o_all)
    assert np.array_equal(st[0], st_all[0])           # all accepted
    assert np.array_equal(st[1], s0[1])               # none accepted
    o2, st2 = gdn_conventional(_toks({k: v[:2] for k, v in d.items()}), s0)
    assert np.array_equal(st[2], st2[2])              # two accepted


def test_gdn_wy_fold_equals_sequential(oracle_lib):
    sh, s0, ins = _gdn(T=16, W=16)
    st = s0.astype(np.float64).copy()
    for t in range(16):
        gdn_step(*(token(ins, t)[k] for k in ("q", "k", "v", "beta", "alpha")), st)
    S = gdn_wy_fold(s0[1, 2].astype(np.float64), ins["k"][:, 1, 2].astype(np.float64),
                    ins["v"][:, 1, 2].astype(np.float64), ins["beta"][:, 1, 2], ins["alpha"][:, 1, 2])
    assert normwise_err(S, st[1, 2]) < 1e-13


# ---------------------------------------------------------------- bookkeeping trace

def _run_trace(bk, ops):
    for op in ops:
        kind = op["op"]
        if kind == "init":
            bk.init()
        elif kind == "init_mask":
            bk.init(op["arg"])
        elif kind == "decode":
            bk.decode()
        elif kind == "verify":
            bk.verify(op["K"])
        elif kind == "commit":
            bk.commit(op["arg"])
        elif kind == "rollback":
            bk.rollback(op["arg"])
        elif kind == "consolidate":
            bk.consolidate(op["arg"])
        elif kind == "read_err":
            assert bk.read_err() == op["err"], op
            continue
        h, l, nd = bk.snapshot()
        assert list(h) == op["head"] and list(l) == op["len"] and list(nd) == op["ndraft"], op


def test_bookkeeping_golden_trace():
    g = json.load(open(os.path.join(GOLDEN, "bookkeeping_w4_k2.json")))
    _run_trace(Bookkeeping(g["batch"], g["window"], g["max_draft"]), g["ops"])


def test_bookkeeping_call_order():
    bk = Bookkeeping(2, 4, 2)
    with pytest.raises(StateError):
        bk.commit([0, 0])
    bk.verify(2)
    with pytest.raises(StateError):
        bk.decode()
    with pytest.raises(StateError):
        bk.verify(1)
    bk.rollback([0, 0])
    bk.decode()
    with pytest.raises(ValueError):
        bk.verify(3)


def test_replay_model_follows_golden_trace(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "bookkeeping_w4_k2.json")))
    sh = wl.M2Shape(batch=3, nheads=2, ngroups=2, head_dim=4, d_state=4, window=4, max_draft=2)
    prm = wl.m2_params(sh, 0)
    rp = M2Replay(prm["A"], prm["D"], wl.m2_state0(sh, 0), 2, 4, max_draft=2)
    for i, op in enumerate(g["ops"]):
        kind = op["op"]
        if kind == "init":
            rp.init(wl.m2_state0(sh, 0))
        elif kind == "init_mask":
            rp.init(wl.m2_state0(sh, 5), op["arg"])
        elif kind == "decode":
            rp.decode(token(wl.m2_token_inputs(sh, 0, i), 0))
        elif kind == "verify":
            rp.verify(wl.m2_token_inputs(sh, 0, i, ntok=op["K"]))
        elif kind == "commit":
            rp.commit(op["arg"])
        elif kind == "rollback":
            rp.rollback(op["arg"])
        elif kind == "consolidate":
            rp.consolidate(op["arg"])
        elif kind == "read_err":
            assert rp.bk.read_err() == op["err"]
            continue
        h, l, nd = rp.bk.snapshot()
        assert list(h) == op["head"] and list(l) == op["len"] and list(nd) == op["ndraft"], op


def test_cond_check_semantics():
    """A vector within the normwise tolerance passes whatever its bound; one over it passes only
    if every element is within its bound; the ratios say which element decided."""
    from oracle import cond_check
    ref = np.array([[[1.0, -2.0], [1e-4, 2e-4]]])          # [token, H=2, P=2]
    got = ref.copy()
    got[0, 1, 0] += 1e-6                                   # 5e-3 normwise on the small head
    bound = np.full(ref.shape, 2e-6)
    c = cond_check(got, ref, bound, 1e-5)
    assert c.n_over == 1 and abs(c.worst - 1e-6 / 2e-4) < 1e-12
    assert abs(c.ratio_over - 0.5) < 1e-12 and c.where == (0, 1) and c.ok
    c = cond_check(got, ref, bound / 4, 1e-5)              # same error, bound too small: fails
    assert not c.ok and abs(c.ratio_over - 2.0) < 1e-12
    got2 = ref.copy()
    got2[0, 0, 1] += 1e-6                                  # within 1e-5 of a large head: passes
    c = cond_check(got2, ref, bound / 100, 1e-5)
    assert c.ok and c.n_over == 0 and c.ratio_over == 0.0 and abs(c.ratio_all - 50.0) < 1e-6


def test_verify_launch_ring_slots_disjoint():
    """Ring slots touched by one speculative-verify launch, for every (W, K, head, len).

    The verify launch appends the K drafts at logical entries len_e .. len_e + K - 1 and, with B / C
    shared by a group of heads, only the group's first head writes the group's B rows, while every
    head of the group reads the committed entries 0 .. len_e - 1 in other workgroups of the same
    launch. With G < H the library folds sequences whose drafts do not fit (len + K > W) in a
    consolidation launch before the verify, so the verify launch sees len_e + K <= W; with G = H
    each workgroup reads and writes only its own head's rows, ordered by its own barrier. Under
    that plan the written slots never meet a slot read by another workgroup."""
    for W in range(1, 33):
        for K in range(1, W + 1):
            for head in range(W):
                for ln in range(W + 1):
                    # G < H: the consolidation launch folds first when the drafts do not fit
                    h_e, l_e = ((head + ln) % W, 0) if ln + K > W else (head, ln)
                    assert l_e + K <= W
                    reads = {(h_e + j) % W for j in range(l_e)}
                    writes = {(h_e + l_e + k) % W for k in range(K)}
                    assert len(writes) == K and not (reads & writes), (W, K, head, ln)
                    # the bookkeeping model lands on the same ring position
                    bk = Bookkeeping(1, W, K)
                    bk.head[0], bk.len[0] = head, ln
                    bk.verify(K)
                    assert (int(bk.head[0]), int(bk.len[0])) == (h_e, l_e)
