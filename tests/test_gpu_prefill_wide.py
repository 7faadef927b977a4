"""GPU parity of the prefills at shapes whose 16 token rows span more than 4 GiB, where the host
(Gated DeltaNet, Kimi Delta Attention) or the kernel (Mamba-2) takes the code with 64-bit row
offsets and predicated loads and stores; every other test runs the 32-bit-offset code. 128 x 128
delta-rule tiles at batch 4100 x 128 heads (524,800 tiles, 34 GB of state) and 64 x 128 Mamba-2
tiles at the same batch and heads; a 17-token prompt (one full chunk and a ragged one). Sequences
0, B/2 and B-1 (the last holds the largest offsets) against the oracle: every output and the
state the prompt leaves, normwise relative error 1e-5 per head vector, or for an output vector
over it its rounding bound C_FP32 u32 kappa element by element (kappa from the absolute-value
recurrence, as in the serving-shape tests). Inputs are drawn on the
device (torch's seeded generator), the sampled sequences copied to the host for the oracle."""
import gc

import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import (C_FP32, U32, cond_check, gdn_kappa_step, gdn_step, kda_kappa_step, kda_step,
                    m2_kappa_step, m2_step, normwise_err)
from tests.gpu_helpers import dev, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5
T = 17
B, H = 4100, 128


@pytest.mark.parametrize("kind,dv,dk", [("gdn", 128, 128), ("kda", 128, 128), ("mamba2", 64, 128)])
def test_prefill_rows_beyond_4gib(kind, dv, dk):
    assert B * H * max(dv, dk) * 4 * 16 > 2 ** 32          # the 64-bit-offset code
    say(f"{kind} prefill {dv}x{dk}, batch {B} x {H} heads, {T} tokens (rows beyond 4 GiB)")
    ins, s0 = wl.torch_prompt_inputs(kind, B, H, dv, dk, T, seed=21)
    seqs = [0, B // 2, B - 1]
    s0_h = {b: host(s0[b]).astype(np.float64) for b in seqs}
    ins_h = {b: {key: host(val[:, b]) for key, val in ins.items()} for b in seqs}
    ctx = rb.Context(kind, B, H, dv, dk, 1)
    if kind == "mamba2":
        prm = wl.m2_params(wl.M2Shape(batch=1, nheads=H, ngroups=H, head_dim=dv, d_state=dk,
                                      window=1), 21)
        A, D = dev(prm["A"]), dev(prm["D"])
        ctx.set_params(A, D)
    ctx.init_checkpoint(s0)
    del s0
    gc.collect()
    torch.cuda.empty_cache()
    y = torch.empty(T, B, H, dv, device="cuda")
    ctx.prefill(y, **ins)
    del ins
    gc.collect()
    torch.cuda.empty_cache()
    mat = torch.empty(B, H, dv, dk, device="cuda")
    ctx.materialize(mat)
    h, l, n, e = ctx.bookkeeping()
    assert e == 0 and max(l) == 0 and max(n) == 0
    for b in seqs:
        ref = s0_h[b][None].copy()
        M = np.abs(ref)
        x = ins_h[b]
        o_ref, kap = [], []
        for t in range(T):
            if kind == "mamba2":
                a = [prm["A"], prm["D"]] + [x[key][t][None] for key in ("x", "B", "C", "dt")]
                o_ref.append(m2_step(*a, ref))
                kap.append(m2_kappa_step(*a, M))
            else:
                a = [x[key][t][None] for key in ("q", "k", "v", "beta", "alpha")]
                o_ref.append((gdn_step if kind == "gdn" else kda_step)(*a, ref))
                kap.append((gdn_kappa_step if kind == "gdn" else kda_kappa_step)(*a, M))
        c = cond_check(host(y[:, b])[:, None], np.stack(o_ref), C_FP32 * U32 * np.stack(kap), TOL)
        say(f"  sequence {b}: outputs {c}")
        assert c.ok and c.ratio_all <= 1, (b, c)
        err = normwise_err(host(mat[b])[None], ref)
        say(f"  sequence {b}: state error {err:.2e}")
        assert err < TOL, (b, err)
    ctx.close()
    del ctx, y, mat
    gc.collect()
    torch.cuda.empty_cache()                 # the next tests need none of these 70 GB
