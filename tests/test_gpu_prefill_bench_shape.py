"""GPU parity of the three prefills (rssm_prefill, C ABI -> HIP matrix-core kernels) at the
workloads bench.py times: batch 256 with the benchmark's head shapes, a 512-token prompt whose
token t is pool slot t mod 32 of the decode inputs, from the benchmark's initial state. For
sampled sequences (every head, every prompt token) the outputs against the oracle, a head vector
over the normwise 1e-5 criterion passing only within its fp32 rounding bound C_FP32 u32 kappa
element by element; and the checkpoint the prompt leaves against the oracle's state."""
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
T, POOL = 512, 32
SUB = np.array([0, 255])


def _prompt(gen, sh):
    """The benchmark's prompt on the GPU ([T, ...] per input) and the sampled sequences' slot
    inputs on the host."""
    slots = [gen(sh, 0, s) for s in range(POOL)]
    pool = [{k: torch.from_numpy(v[0]).cuda() for k, v in sl.items()} for sl in slots]
    prompt = {k: torch.stack([pool[t % POOL][k] for t in range(T)]) for k in pool[0]}
    del pool
    hsub = [{k: v[0][SUB] for k, v in sl.items()} for sl in slots]
    return prompt, hsub


def _check(name, out, ctx, s0, step, kappa, keys, hsub):
    """Run the oracle over the prompt on the sampled sequences and compare."""
    sub_t = torch.from_numpy(SUB).cuda()
    osub = host(out.index_select(1, sub_t))
    mat = torch.empty(s0.shape, device="cuda")
    ctx.materialize(mat)
    msub = host(mat.index_select(0, sub_t))
    del mat
    ref = s0[SUB].astype(np.float64)
    M = np.abs(ref)
    o_ref, kref = [], []
    for t in range(T):
        a = [hsub[t % POOL][k] for k in keys]
        o_ref.append(step(*a, ref))
        kref.append(kappa(*a, M))
    c = cond_check(osub, np.stack(o_ref), C_FP32 * U32 * np.stack(kref), TOL)
    err = normwise_err(msub, ref)
    say(f"  {name}: outputs {c}; checkpoint normwise {err:.3e}")
    assert c.ok and c.ratio_all <= 1
    assert err < TOL


def test_m2_prefill_bench_shape():
    """Mamba-2, batch 256, 128 heads, 64 x 128 (per-head B and C), 512-token prompt."""
    sh = wl.M2_SERVE
    say("mamba-2 prefill at the benchmark's shape: generating inputs")
    prm = wl.m2_params(sh, 0)
    s0 = wl.m2_state0(sh, 0)
    prompt, hsub = _prompt(wl.m2_token_inputs, sh)
    ctx = rb.Context("mamba2", sh.batch, sh.nheads, sh.head_dim, sh.d_state, sh.window,
                     ngroups=sh.ngroups)
    ctx.set_params(dev(prm["A"]), dev(prm["D"]))
    ctx.init_checkpoint(dev(s0))
    y = torch.empty(T, sh.batch, sh.nheads, sh.head_dim, device="cuda")
    ctx.prefill(y, **prompt)
    del prompt
    _check("mamba-2", y, ctx, s0,
           lambda *a: m2_step(prm["A"], prm["D"], *a),
           lambda *a: m2_kappa_step(prm["A"], prm["D"], *a),
           ("x", "B", "C", "dt"), hsub)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_delta_prefill_bench_shape(kind):
    """Gated DeltaNet and Kimi Delta Attention, batch 256, 32 heads, 128 x 128, 512-token prompt."""
    sh = wl.GDN_SERVE if kind == "gdn" else wl.KDA_SERVE
    say(f"{kind} prefill at the benchmark's shape: generating inputs")
    s0 = (wl.gdn_state0 if kind == "gdn" else wl.kda_state0)(sh, 0)
    prompt, hsub = _prompt(wl.gdn_token_inputs if kind == "gdn" else wl.kda_token_inputs, sh)
    ctx = rb.Context(kind, sh.batch, sh.nheads, sh.d_v, sh.d_k, sh.window)
    ctx.init_checkpoint(dev(s0))
    o = torch.empty(T, sh.batch, sh.nheads, sh.d_v, device="cuda")
    ctx.prefill(o, **prompt)
    del prompt
    step, kappa = (gdn_step, gdn_kappa_step) if kind == "gdn" else (kda_step, kda_kappa_step)
    _check(kind, o, ctx, s0, step, kappa, ("q", "k", "v", "beta", "alpha"), hsub)
