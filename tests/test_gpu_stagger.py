"""GPU parity in the staggered serving state: every sequence at its own ring position, so every
decode launch mixes tiles that fold with tiles that replay. Continuous batching and speculative
commits leave a batch in that state (news.hamidun.com item "NVIDIA présente ReplaySSM...",
section "D'où vient le problème de l'état"). The state is reached by W-1 decode tokens and a
rollback of sequence b to b mod W entries; from there, 1/W of the sequences fold at every step.

Criteria as in the other Mamba-2 parity tests: per head vector normwise 1e-5 (fp32) or 2e-2 (bf16
read copy), else every element within its rounding bound (C_FP32 u32 kappa, plus
Lam u16 sum_n |S0[p,n]| |C_n| for a replayed output read from the bf16 copy); bookkeeping of every
sequence bit-exact after every call; the materialised state at the end."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import (C_FP32, U16, U32, Bookkeeping, cond_check, m2_kappa_step, m2_step,
                    normwise_err)
from tests.gpu_helpers import dev, host, m2_dev_tokens, say, tok0

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2


class _Sampled:
    """Oracle state of the sampled sequences: the fp64 state, its conditioning recurrence, the
    checkpoint the kernel reads (state at the sequence's last fold) and the step sizes of the
    entries buffered since then (for the bf16 read bound)."""

    def __init__(self, prm, s0_sub, hpg):
        self.prm, self.hpg = prm, hpg
        self.ref = s0_sub.astype(np.float64)
        self.M = np.abs(self.ref)
        self.ck = self.ref.copy()
        self.win = [[] for _ in range(s0_sub.shape[0])]

    def step(self, tok, folded):
        """One conventional token; `folded` [nsub] marks the sequences whose ring this token
        filled. Returns (y_ref, fp32 bound, bf16 read term or None per sequence)."""
        A = self.prm["A"].astype(np.float64)
        args = (tok["x"], tok["B"], tok["C"], tok["dt"])
        y = m2_step(self.prm["A"], self.prm["D"], *args, self.ref)
        kap = m2_kappa_step(self.prm["A"], self.prm["D"], *args, self.M)
        hh = np.arange(tok["x"].shape[1]) // self.hpg
        Cg = np.abs(tok["C"].astype(np.float64))[:, hh]
        bf = np.zeros_like(y)
        for i in range(y.shape[0]):
            self.win[i].append(tok["dt"][i].astype(np.float64))
            if folded[i]:           # output read from the fresh fp32 checkpoint
                self.ck[i] = self.ref[i]
                self.win[i] = []
            else:
                lam = np.exp(A * np.sum(self.win[i], axis=0))
                bf[i] = lam[:, None] * U16 * np.einsum("hpn,hn->hp", np.abs(self.ck[i]), Cg[i])
        return y, C_FP32 * U32 * kap, bf

    def rollback(self, states, Ms, lens, dts):
        """Sequence i keeps the first lens[i] buffered tokens: states / Ms are the oracle states
        after 0..W-1 tokens, dts the step sizes of those tokens."""
        for i, L in enumerate(lens):
            self.ref[i] = states[L][i]
            self.M[i] = Ms[L][i]
            self.win[i] = [dts[t][i] for t in range(L)]


def _run(sh, bf16, steps, sub, seed=0):
    say(f"stagger B={sh.batch} H={sh.nheads} G={sh.ngroups} {sh.head_dim}x{sh.d_state} "
        f"bf16={bf16} steps={steps}")
    W = sh.window
    prm = wl.m2_params(sh, seed)
    s0 = wl.m2_state0(sh, seed)
    ctx = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, W,
                     ngroups=sh.ngroups, bf16_read=bf16)
    A, D = dev(prm["A"]), dev(prm["D"])
    ctx.set_params(A, D)
    ctx.init_checkpoint(dev(s0))
    model = Bookkeeping(sh.batch, W)
    y = torch.empty(sh.batch, sh.nheads, sh.head_dim, device="cuda")
    orc = _Sampled(prm, s0[sub], sh.nheads // sh.ngroups)
    # W - 1 tokens, keeping the oracle states after 0..W-1 of them
    states, Ms, dts = [orc.ref.copy()], [orc.M.copy()], []
    for t in range(W - 1):
        ins = wl.m2_token_inputs(sh, seed, t)
        ctx.decode_step(y, **tok0(m2_dev_tokens(sh, ins, 1)))
        model.decode()
        s = {k: v[0][sub] for k, v in ins.items()}
        m2_step(prm["A"], prm["D"], s["x"], s["B"], s["C"], s["dt"], orc.ref)
        m2_kappa_step(prm["A"], prm["D"], s["x"], s["B"], s["C"], s["dt"], orc.M)
        states.append(orc.ref.copy())
        Ms.append(orc.M.copy())
        dts.append(s["dt"].astype(np.float64))
    new_len = (np.arange(sh.batch) % W).astype(np.int32)
    ctx.rollback(dev(new_len))
    model.rollback(new_len)
    orc.rollback(states, Ms, new_len[sub], dts)
    h, l, n, e = ctx.bookkeeping()
    assert l == list(model.len) and e == 0
    tol = TOL_BF16 if bf16 else TOL
    worst, n_over, ratio_all, ratio_over = 0.0, 0, 0.0, 0.0
    pool = [wl.m2_token_inputs(sh, seed, 100 + i) for i in range(min(steps, 16))]
    dpool = [tok0(m2_dev_tokens(sh, p, 1)) for p in pool]
    for t in range(steps):
        ins = pool[t % len(pool)]
        ctx.decode_step(y, **dpool[t % len(pool)])
        folded = model.decode()
        assert 0 < folded.sum() < sh.batch or sh.batch < W, t      # a mixed launch
        h, l, n, e = ctx.bookkeeping()
        mh, ml, mn = model.snapshot()
        assert h == list(mh) and l == list(ml) and n == list(mn) and e == 0, t
        y_ref, b32, bbf = orc.step({k: v[0][sub] for k, v in ins.items()}, folded[sub])
        c = cond_check(host(y)[sub], y_ref, b32 + (bbf if bf16 else 0.0), tol)
        assert c.ok and c.ratio_all <= 1.0, (t, c)
        worst, n_over = max(worst, c.worst), n_over + c.n_over
        ratio_all, ratio_over = max(ratio_all, c.ratio_all), max(ratio_over, c.ratio_over)
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    assert normwise_err(host(mat)[sub], orc.ref) < TOL
    say(f"  worst normwise {worst:.3e}, {n_over} head vectors over {tol:g} (worst |d|/bound "
        f"there {ratio_over:.3f}), worst |d|/bound {ratio_all:.3f}")


@pytest.mark.parametrize("P,N", [(64, 128), (64, 64), (32, 32), (128, 128)])
@pytest.mark.parametrize("bf16", [False, True])
def test_stagger_small(P, N, bf16):
    """Every sequence of a 32-sequence batch checked: 40 mixed steps (2.5 windows) at each head
    shape whose launches that may fold run their own thread map, grouped B/C."""
    sh = wl.M2Shape(batch=32, nheads=8, ngroups=4, head_dim=P, d_state=N, window=16)
    _run(sh, bf16, 40, np.arange(32))


@pytest.mark.parametrize("bf16", [False, True])
def test_stagger_serving_shape(bf16):
    """Batch 256, 128 heads, 64x128, W = 16: 48 mixed steps; sampled sequences cover every ring
    fill (0..15) and both ends of the batch."""
    sub = np.concatenate([np.arange(16), [100, 255]])
    _run(wl.M2_SERVE, bf16, 48, sub)
