"""The bf16 read copy, bit for bit: after every operation that writes the fp32 checkpoint (load,
the fold inside a decode step, consolidation, a verify that folds first, prefill) the copy holds
the round-to-nearest-even bf16 value of every fp32 checkpoint entry (the high-precision checkpoint
drives the recurrence, a lower-precision copy serves the reads: ia.goatify.app article "NVIDIA y
Princeton aceleran modelos híbridos...", paragraph "La precisión separa lectura y recurrencia").
Both arrays are read back with rssm_export, whose packed slot holds the checkpoint segment and
then the copy segment after a 16-byte header."""
import numpy as np
import pytest
import torch

import workloads as wl
from checkpoint_replay_buffer_amd import binding as rb
from oracle import round_bf16
from tests.gpu_helpers import dev, host, m2_dev_tokens, say, tok0

pytestmark = pytest.mark.gpu


def _check_copy(ctx, sh, what):
    """Export every sequence and compare the bf16 segment with RNE of the fp32 segment."""
    nbytes = ctx.seq_state_bytes()
    buf = torch.empty(sh.batch * nbytes // 4 + 4, dtype=torch.float32, device="cuda")
    ctx.export(torch.arange(sh.batch, dtype=torch.int32, device="cuda"), buf)
    raw = host(buf).view(np.uint8)[: sh.batch * nbytes].reshape(sh.batch, nbytes)
    tile = sh.nheads * sh.head_dim * sh.d_state
    f32 = raw[:, 16:16 + 4 * tile].copy().view(np.float32)
    off = 16 + (4 * tile + 15) // 16 * 16
    b16 = raw[:, off:off + 2 * tile].copy().view(np.uint16)
    want = (round_bf16(f32).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bad = int(np.count_nonzero(b16 != want))
    say(f"  {what}: {b16.size} copy entries, {bad} differ from RNE of the checkpoint")
    assert bad == 0, what
    return f32


@pytest.mark.parametrize("P,N", [(64, 128), (16, 16)])
def test_bf16_copy_is_rne_of_checkpoint(P, N):
    sh = wl.M2Shape(batch=4, nheads=4, ngroups=2, head_dim=P, d_state=N, window=8, max_draft=6)
    prm = wl.m2_params(sh, 12)
    s0 = wl.m2_state0(sh, 12)
    ctx = rb.Context("mamba2", sh.batch, sh.nheads, P, N, sh.window, ngroups=sh.ngroups,
                     max_draft=sh.max_draft, bf16_read=True)
    ctx.set_params(dev(prm["A"]), dev(prm["D"]))
    ctx.init_checkpoint(dev(s0))
    f32 = _check_copy(ctx, sh, "after init")
    assert np.array_equal(f32.reshape(s0.shape), s0)
    ins = wl.m2_token_inputs(sh, 12, 0, ntok=40)
    d = m2_dev_tokens(sh, ins, 40)
    y = torch.empty(sh.batch, sh.nheads, P, device="cuda")
    for t in range(sh.window):             # the W-th token folds inside the decode launch
        ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
    f32b = _check_copy(ctx, sh, "after the fold of a decode step")
    assert not np.array_equal(f32b, f32)
    for t in range(sh.window, sh.window + 5):
        ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
    ctx.consolidate(3)
    _check_copy(ctx, sh, "after consolidation")
    for t in range(sh.window + 5, sh.window + 11):
        ctx.decode_step(y, **{k: v[t] for k, v in d.items()})
    K = 6                                  # len 6 + K > W: the verify folds first
    dr = m2_dev_tokens(sh, wl.m2_token_inputs(sh, 12, 1, ntok=K), K)
    yk = torch.empty(K, sh.batch, sh.nheads, P, device="cuda")
    ctx.verify(yk, **dr)
    ctx.commit(dev(np.array([0, 1, 3, 6], np.int32)))
    _check_copy(ctx, sh, "after a verify that folds first")
    yp = torch.empty(20, sh.batch, sh.nheads, P, device="cuda")
    ctx.prefill(yp, **{k: v[:20] for k, v in d.items()})
    _check_copy(ctx, sh, "after prefill")
    h, l, n, e = ctx.bookkeeping()
    assert e == 0
