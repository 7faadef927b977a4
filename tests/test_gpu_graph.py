"""Decode steps captured in a HIP graph (a window of 2 W steps from an empty ring, so that it ends
at the ring position and bookkeeping buffer it started from) and replayed: every replay, with new
tokens copied into the captured input buffers and eager work between the replays, gives outputs,
states and bookkeeping bit-identical to the same steps run eagerly, and matches the oracle."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import gdn_step, kda_step, m2_step, normwise_err
from tests.gpu_helpers import dev, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5
REPLAYS = 3


def _setup(kind, bf16):
    if kind == "mamba2":
        sh = wl.M2Shape(batch=2, nheads=4, ngroups=2, head_dim=32, d_state=32, window=4)
        prm = wl.m2_params(sh, 0)
        s0 = wl.m2_state0(sh, 0)

        def make():
            c = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                           ngroups=sh.ngroups, bf16_read=bf16)
            c.set_params(dev(prm["A"]), dev(prm["D"]))
            return c

        def toks(seed, n):
            return wl.m2_token_inputs(sh, seed, 0, ntok=n)

        def oracle_step(ins, t, ref):
            return m2_step(prm["A"], prm["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t], ref)

        dv = sh.head_dim
    else:
        sh = wl.GDNShape(batch=2, nheads=4, d_k=64, d_v=64, window=4)
        kda = kind == "kda"
        s0 = (wl.kda_state0 if kda else wl.gdn_state0)(sh, 0)

        def make():
            return rb.Context(kind, sh.batch, sh.nheads, sh.d_v, sh.d_k, sh.window)

        def toks(seed, n):
            return (wl.kda_token_inputs if kda else wl.gdn_token_inputs)(sh, seed, 0, ntok=n)

        def oracle_step(ins, t, ref):
            return (kda_step if kda else gdn_step)(ins["q"][t], ins["k"][t], ins["v"][t],
                                                   ins["beta"][t], ins["alpha"][t], ref)

        dv = sh.d_v
    return sh, s0, make, toks, oracle_step, dv


@pytest.mark.parametrize("kind,bf16", [("mamba2", False), ("mamba2", True), ("gdn", False),
                                       ("kda", False)])
def test_graph_window_replays_match_eager(kind, bf16):
    sh, s0, make, toks, oracle_step, dv = _setup(kind, bf16)
    n = 2 * sh.window
    say(f"graph window {kind} bf16={bf16}: {n} steps, {REPLAYS} replays")
    cg, ce = make(), make()
    cg.init_checkpoint(dev(s0))
    ce.init_checkpoint(dev(s0))
    ref = s0.astype(np.float64).copy()
    first = toks(100, n)
    static = [{k: dev(v[t]) for k, v in first.items()} for t in range(n)]
    ys = [torch.empty(sh.batch, sh.nheads, dv, device="cuda") for _ in range(n)]
    ye = torch.empty(sh.batch, sh.nheads, dv, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for t in range(n):
            cg.decode_step(ys[t], **static[t])
    for r in range(REPLAYS):
        ins = toks(100 + r, n)
        for t in range(n):                       # new tokens into the captured buffers
            for k, v in ins.items():
                static[t][k].copy_(dev(v[t]))
        g.replay()
        torch.cuda.synchronize()
        for t in range(n):                       # the same steps, eagerly, on the other context
            ce.decode_step(ye, **{k: dev(v[t]) for k, v in ins.items()})
            yr = oracle_step(ins, t, ref)
            yg, yeh = host(ys[t]), host(ye)
            assert np.array_equal(yg, yeh), (r, t)
            tol = 2e-2 if bf16 else TOL
            assert normwise_err(yg.reshape(sh.batch, -1) if bf16 else yg,
                                yr.reshape(sh.batch, -1) if bf16 else yr) < tol, (r, t)
        mg = torch.empty(s0.shape, device="cuda")
        me = torch.empty(s0.shape, device="cuda")
        cg.materialize(mg)
        ce.materialize(me)
        assert np.array_equal(host(mg), host(me)), r
        assert cg.bookkeeping() == ce.bookkeeping(), r
        h, l, nd, e = cg.bookkeeping()
        assert l == [0] * sh.batch and e == 0
    del g
