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


def tok0(d: dict) -> dict:
    """Single-token view (drop the leading token axis) of device inputs."""
    return {k: v[0] for k, v in d.items()}


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str):
    print(msg, flush=True)
