"""Seeded random sequences of the library's operations on one context (Mamba-2 in fp32 and with the
bf16 read copy, Gated DeltaNet, Kimi Delta Attention), against the CPU oracle and
the bookkeeping model: decode steps, speculative rounds committed or discarded,
consolidation, masked re-initialisation, prefills, forks, and exports imported again later into
other slots. After every operation: every output it wrote and the bookkeeping; every few operations
and at the end: the materialised state of every sequence."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import (Bookkeeping, gdn_spec_round, gdn_step, kda_spec_round, kda_step, m2_spec_round,
                    m2_step, normwise_err)
from tests.gpu_helpers import dev, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5
TOL_BF16 = 2e-2
OPS = 120


class _Layer:
    """The layer under test: its context, inputs, oracle steps and fp64 reference state."""

    def __init__(self, kind, seed):
        self.bf16 = kind == "mamba2_bf16"
        kind = "mamba2" if self.bf16 else kind
        self.kind, self.seed = kind, seed
        if kind == "mamba2":
            self.sh = wl.M2Shape(batch=5, nheads=4, ngroups=2, head_dim=16, d_state=16, window=6,
                                 max_draft=3)
            self.prm = wl.m2_params(self.sh, seed)
            s0 = wl.m2_state0(self.sh, seed)
            self.ctx = rb.Context("mamba2", self.sh.batch, self.sh.nheads, 16, 16, self.sh.window,
                                  ngroups=self.sh.ngroups, max_draft=self.sh.max_draft,
                                  bf16_read=self.bf16)
            self.ctx.set_params(dev(self.prm["A"]), dev(self.prm["D"]))
            self.dv = 16
        else:
            self.sh = wl.GDNShape(batch=5, nheads=4, d_k=16, d_v=16, window=6, max_draft=3)
            s0 = (wl.kda_state0 if kind == "kda" else wl.gdn_state0)(self.sh, seed)
            self.ctx = rb.Context(kind, self.sh.batch, self.sh.nheads, 16, 16, self.sh.window,
                                  max_draft=self.sh.max_draft)
            self.dv = 16
        self.ctx.init_checkpoint(dev(s0))
        self.ref = s0.astype(np.float64).copy()
        self.model = Bookkeeping(self.sh.batch, self.sh.window, self.sh.max_draft)

    def inputs(self, slot, ntok):
        if self.kind == "mamba2":
            return wl.m2_token_inputs(self.sh, self.seed, slot, ntok=ntok)
        if self.kind == "kda":
            return wl.kda_token_inputs(self.sh, self.seed, slot, ntok=ntok)
        return wl.gdn_token_inputs(self.sh, self.seed, slot, ntok=ntok)

    def fresh_states(self, slot):
        gen = {"mamba2": wl.m2_state0, "gdn": wl.gdn_state0, "kda": wl.kda_state0}[self.kind]
        return gen(self.sh, 500 + slot)

    def spec_round(self, ins, accepted):
        """The oracle's conventional speculative round on the reference state."""
        if self.kind == "mamba2":
            return m2_spec_round(self.prm["A"], self.prm["D"], ins, self.ref, accepted)
        if self.kind == "kda":
            return kda_spec_round(ins, self.ref, accepted)
        return gdn_spec_round(ins, self.ref, accepted)

    def step(self, ins, t):
        """The oracle's conventional step t of `ins` on the reference state."""
        if self.kind == "mamba2":
            p = self.prm
            return m2_step(p["A"], p["D"], ins["x"][t], ins["B"][t], ins["C"][t], ins["dt"][t],
                           self.ref)
        step = kda_step if self.kind == "kda" else gdn_step
        return step(ins["q"][t], ins["k"][t], ins["v"][t], ins["beta"][t], ins["alpha"][t], self.ref)

    def out_err(self, got, ref):
        """fp32: per head vector; bf16 read copy: per sequence-token layer output."""
        if not self.bf16:
            return normwise_err(got, ref)
        b = self.sh.batch
        return normwise_err(np.asarray(got).reshape(*np.shape(got)[:-3], b, -1) if np.ndim(got) > 3
                            else np.asarray(got).reshape(b, -1),
                            np.asarray(ref).reshape(*np.shape(ref)[:-3], b, -1) if np.ndim(ref) > 3
                            else np.asarray(ref).reshape(b, -1))

    def check_bk(self, where):
        h, l, n, e = self.ctx.bookkeeping()
        m = self.model
        assert (h, l, n, e) == (list(m.head), list(m.len), list(m.ndraft), 0), (where, h, l, n, e)

    def check_state(self, where):
        mat = torch.empty(self.ref.shape, device="cuda")
        self.ctx.materialize(mat)
        err = normwise_err(host(mat), self.ref)
        assert err < TOL, (where, err)


def _i32(v):
    return torch.tensor(np.asarray(v, dtype=np.int32), device="cuda")


@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda", "mamba2_bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operation_sequences(kind, seed):
    rng = np.random.default_rng(9000 + seed)       # the schedule of operations, not method data
    L = _Layer(kind, seed)
    B = L.sh.batch
    tol = TOL_BF16 if L.bf16 else TOL
    ops = ["decode", "verify", "consolidate", "init", "prefill", "fork", "export", "import"]
    weights = [6, 3, 1, 1, 1, 1, 1, 1]
    p = np.asarray(weights, float) / sum(weights)
    buf = torch.empty(B * L.ctx.seq_state_bytes(), dtype=torch.uint8, device="cuda")
    snap = None                                    # (sequences, their ref rows, their bookkeeping)
    counts = {}
    for it in range(OPS):
        op = str(rng.choice(ops, p=p))
        counts[op] = counts.get(op, 0) + 1
        where = (it, op)
        if op == "decode":
            ins = L.inputs(it, 1)
            o = torch.empty(B, L.sh.nheads, L.dv, device="cuda")
            L.ctx.decode_step(o, **{k: dev(v[0]) for k, v in ins.items()})
            L.model.decode()
            assert L.out_err(host(o), L.step(ins, 0)) < tol, where
        elif op == "verify":
            K = int(rng.integers(1, L.sh.max_draft + 1))
            ins = L.inputs(it, K)
            yk = torch.empty(K, B, L.sh.nheads, L.dv, device="cuda")
            L.ctx.verify(yk, **{k: dev(v) for k, v in ins.items()})
            L.model.verify(K)
            L.check_bk(where)
            if rng.random() < 0.75:
                a = rng.integers(0, K + 1, size=B).astype(np.int32)
                L.ctx.commit(_i32(a))
                L.model.commit(a)
            else:                                   # discard every draft
                a = np.zeros(B, np.int32)
                L.ctx.rollback(_i32(L.model.len))
                L.model.rollback(L.model.len.copy())
            yr = L.spec_round(ins, a)
            assert L.out_err(host(yk), yr) < tol, where
        elif op == "consolidate":
            ml = int(rng.integers(1, L.sh.window + 1))
            L.ctx.consolidate(ml)
            L.model.consolidate(ml)
        elif op == "init":
            mask = (rng.random(B) < 0.4).astype(np.int32)
            fresh = L.fresh_states(it)
            L.ctx.init_checkpoint(dev(fresh), dev(mask))
            L.model.init(mask)
            L.ref[mask != 0] = fresh[mask != 0].astype(np.float64)
        elif op == "prefill":
            T = int(rng.integers(1, 40))
            ins = L.inputs(it, T)
            o = torch.empty(T, B, L.sh.nheads, L.dv, device="cuda")
            L.ctx.prefill(o, **{k: dev(v) for k, v in ins.items()})
            L.model.consolidate(1)                  # buffered entries fold first
            ref_o = np.stack([L.step(ins, t) for t in range(T)])
            assert L.out_err(host(o), ref_o) < tol, (where, T)
        elif op == "fork":
            perm = rng.permutation(B)
            n = int(rng.integers(1, 3))
            src, dst = perm[:n], perm[n:2 * n]
            L.ctx.fork(_i32(src), _i32(dst))
            for s_, d_ in zip(src, dst):
                L.ref[d_] = L.ref[s_]
                L.model.head[d_], L.model.len[d_] = L.model.head[s_], L.model.len[s_]
                L.model.ndraft[d_] = L.model.ndraft[s_]
        elif op == "export":
            n = int(rng.integers(1, B + 1))
            seqs = rng.permutation(B)[:n]
            L.ctx.export(_i32(seqs), buf)
            snap = (seqs, L.ref[seqs].copy(), L.model.head[seqs].copy(), L.model.len[seqs].copy(),
                    L.model.ndraft[seqs].copy())
        elif op == "import":
            if snap is None:
                continue
            seqs, rrows, hh, ll, nn = snap
            dst = rng.permutation(B)[:len(seqs)]
            L.ctx.import_(_i32(dst), buf)
            L.ref[dst] = rrows
            L.model.head[dst], L.model.len[dst], L.model.ndraft[dst] = hh, ll, nn
        L.check_bk(where)
        if it % 5 == 4:
            L.check_state(where)
    L.check_state("end")
    say(f"{kind} seed {seed}: {counts}")
