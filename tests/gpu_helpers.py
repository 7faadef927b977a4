"""Shared helpers of the GPU tests: host arrays -> device tensors with shape checks, and the
comparison routines. Every launch goes through the C ABI (checkpoint_replay_buffer_amd.binding)."""
import numpy as np
import pytest
import torch

import workloads as wl

gpu_available = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def m2_dev_tokens(sh: wl.M2Shape, ins: dict, ntok: int):
    """Device copies of token-major Mamba-2 inputs, shapes checked against the layer shape."""
    assert ins["x"].shape == (ntok, sh.batch, sh.nheads, sh.head_dim)
    assert ins["B"].shape == (ntok, sh.batch, sh.ngroups, sh.d_state)
    assert ins["C"].shape == (ntok, sh.batch, sh.ngroups, sh.d_state)
    assert ins["dt"].shape == (ntok, sh.batch, sh.nheads)
    return {k: dev(v) for k, v in ins.items()}


def gdn_dev_tokens(sh: wl.GDNShape, ins: dict, ntok: int):
    assert ins["q"].shape == (ntok, sh.batch, sh.nheads, sh.d_k)
    assert ins["k"].shape == (ntok, sh.batch, sh.nheads, sh.d_k)
    assert ins["v"].shape == (ntok, sh.batch, sh.nheads, sh.d_v)
    assert ins["beta"].shape == (ntok, sh.batch, sh.nheads)
    assert ins["alpha"].shape == (ntok, sh.batch, sh.nheads)
    return {k: dev(v) for k, v in ins.items()}


def kda_dev_tokens(sh: wl.GDNShape, ins: dict, ntok: int):
    """Device copies of token-major Kimi Delta Attention inputs (gate alpha [T,B,H,d_k])."""
    assert ins["q"].shape == (ntok, sh.batch, sh.nheads, sh.d_k)
    assert ins["k"].shape == (ntok, sh.batch, sh.nheads, sh.d_k)
    assert ins["v"].shape == (ntok, sh.batch, sh.nheads, sh.d_v)
    assert ins["beta"].shape == (ntok, sh.batch, sh.nheads)
    assert ins["alpha"].shape == (ntok, sh.batch, sh.nheads, sh.d_k)
    return {k: dev(v) for k, v in ins.items()}


def kda_kappa_torch(M, q, k, v, beta, alpha):
    """Kimi Delta Attention counterpart of gdn_kappa_torch (gate alpha [B,H,dk]):
    M <- alpha o M + beta s |k|^T + beta |v| |k|^T with s = (alpha o M) |k|; kappa = M |q|."""
    ka = k.abs()
    M.mul_(alpha[:, :, None, :])
    s = (M * ka[:, :, None, :]).sum(-1)
    be = beta[..., None, None]
    M.add_(be * s[..., None] * ka[:, :, None, :])
    M.add_(be * v.abs()[..., None] * ka[:, :, None, :])
    return (M * q.abs()[:, :, None, :]).sum(-1)


def tok0(d: dict) -> dict:
    """Single-token view (drop the leading token axis) of device inputs."""
    return {k: v[0] for k, v in d.items()}


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str):
    print(msg, flush=True)


# Conditioning of every sequence of a full batch, for rounding bounds between two GPU results
# (plain PyTorch on the device; the oracle's m2_kappa_step / gdn_kappa_step give the same scale
# for the sampled sequences compared against the oracle).

def m2_kappa_torch(M, A, D, x, Bm, C, dt):
    """M [B,H,P,N] fp32 (start at |S_0|) <- exp(dt A) M + dt |x| |B|^T in place; returns
    kappa [B,H,P] = sum_n M |C| + |D x| (the absolute-value recurrence, all terms >= 0)."""
    H, G = M.shape[1], Bm.shape[1]
    hmap = torch.arange(H, device=M.device) // (H // G)
    a = torch.exp(dt * A[None, :])
    Bh, Ch = Bm.abs()[:, hmap], C.abs()[:, hmap]
    M.mul_(a[..., None, None]).add_((dt[..., None] * x.abs())[..., None] * Bh[:, :, None, :])
    return (M * Ch[:, :, None, :]).sum(-1) + (D.abs()[None, :, None] * x.abs())


def gdn_kappa_torch(M, q, k, v, beta, alpha):
    """M [B,H,dv,dk] fp32 (start at |S_0|) <- alpha (M + beta s |k|^T) + beta |v| |k|^T with
    s = M |k|, in place; returns kappa [B,H,dv] = M |q|."""
    ka = k.abs()
    s = (M * ka[:, :, None, :]).sum(-1)
    be, al = beta[..., None, None], alpha[..., None, None]
    M.add_(be * s[..., None] * ka[:, :, None, :]).mul_(al)
    M.add_(be * v.abs()[..., None] * ka[:, :, None, :])
    return (M * q.abs()[:, :, None, :]).sum(-1)
