"""Seeded synthetic inputs for the ReplaySSM decode workloads.

This module only draws random numbers and shapes them into the input distributions of the
synthetic decode workloads. It holds none of the decode arithmetic, and both the CPU oracle and
the HIP path receive the very same arrays from it.

Every array is drawn in float64 and rounded once to float32. Each (seed, tensor, slot) triple has
its own Philox stream, so any slot can be regenerated on its own and in any order.

The pages (five short web articles on ReplaySSM) measure trained Nemotron 3 and Qwen3.5 hybrids;
neither weights nor activations are available, so these distributions stand in for the SSM
layer's activations at the decode shapes used by the tests and the bench:

Mamba-2 (per decode token)
    x ~ N(0, 1)                         [B, H, P]
    B, C ~ N(0, 1) / sqrt(N)            [B, G, N]
    dt = softplus(N(-2, 0.5))           [B, H]     (already positive; no bias, no clamp)
    A = -exp(U(0, ln 16))               [H]        (per head, in [-16, -1])
    D ~ N(0, 1)                         [H]
    initial state ~ N(0, 0.1)           [B, H, P, N]
Gated DeltaNet (per decode token)
    q, k ~ N(0, 1), then L2-normalised  [B, H, d_k]   (normalised in float64, then rounded)
    v ~ N(0, 1)                         [B, H, d_v]
    beta = sigmoid(N(0, 1))             [B, H]
    alpha = exp(-softplus(N(0, 1)))     [B, H]
    initial state ~ N(0, 0.1)           [B, H, d_v, d_k]
Kimi Delta Attention (per decode token; Gated DeltaNet with one forget gate per key channel)
    q, k ~ N(0, 1), then L2-normalised  [B, H, d_k]
    v ~ N(0, 1)                         [B, H, d_v]
    beta = sigmoid(N(0, 1))             [B, H]
    alpha = exp(-softplus(N(0, 1)))     [B, H, d_k]   (each key channel drawn on its own)
    initial state ~ N(0, 0.1)           [B, H, d_v, d_k]
Speculative decoding
    accepted = min(Geometric(0.35) failures before the first success, K)   [rounds, B] int32

N(mu, s) names the standard deviation s.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# One stream id per tensor kind; a stream is keyed by (seed, id, slot).
_TID = {
    "m2_A": 1, "m2_D": 2, "m2_state0": 3,
    "m2_x": 10, "m2_B": 11, "m2_C": 12, "m2_dt": 13,
    "gdn_state0": 20, "gdn_q": 21, "gdn_k": 22, "gdn_v": 23, "gdn_beta": 24, "gdn_alpha": 25,
    "accepted": 30,
    "kda_state0": 40, "kda_q": 41, "kda_k": 42, "kda_v": 43, "kda_beta": 44, "kda_alpha": 45,
}


def _rng(seed: int, name: str, slot: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), _TID[name], int(slot)])
    return np.random.Generator(np.random.Philox(ss))


def _normal(seed, name, slot, shape, loc=0.0, scale=1.0) -> np.ndarray:
    z = _rng(seed, name, slot).standard_normal(size=shape, dtype=np.float64)
    if scale != 1.0:
        z *= scale
    if loc != 0.0:
        z += loc
    return z


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


@dataclasses.dataclass(frozen=True)
class M2Shape:
    """Mamba-2 decode layer shape: batch B, heads H, B/C groups G, head_dim P, d_state N, ring W."""
    batch: int
    nheads: int
    ngroups: int
    head_dim: int
    d_state: int
    window: int
    max_draft: int = 0

    @property
    def state_elems(self) -> int:
        return self.batch * self.nheads * self.head_dim * self.d_state


@dataclasses.dataclass(frozen=True)
class GDNShape:
    """Gated DeltaNet decode layer shape: batch B, heads H, d_k, d_v, ring W."""
    batch: int
    nheads: int
    d_k: int
    d_v: int
    window: int
    max_draft: int = 0


def m2_params(shape: M2Shape, seed: int = 0) -> dict:
    u = _rng(seed, "m2_A").uniform(0.0, math.log(16.0), size=(shape.nheads,))
    A = (-np.exp(u)).astype(np.float32)
    D = _normal(seed, "m2_D", 0, (shape.nheads,)).astype(np.float32)
    return {"A": A, "D": D}


def m2_state0(shape: M2Shape, seed: int = 0) -> np.ndarray:
    s = shape
    return _normal(seed, "m2_state0", 0, (s.batch, s.nheads, s.head_dim, s.d_state),
                   scale=0.1).astype(np.float32)


def m2_token_inputs(shape: M2Shape, seed: int, slot: int, ntok: int = 1) -> dict:
    """Inputs of `ntok` consecutive tokens stored in pool slot `slot`.

    Shapes carry a leading token axis: x [T,B,H,P], B and C [T,B,G,N], dt [T,B,H].
    """
    s = shape
    T, Bt, H, G, P, N = ntok, s.batch, s.nheads, s.ngroups, s.head_dim, s.d_state
    x = _normal(seed, "m2_x", slot, (T, Bt, H, P)).astype(np.float32)
    Bm = _normal(seed, "m2_B", slot, (T, Bt, G, N), scale=1.0 / math.sqrt(N)).astype(np.float32)
    C = _normal(seed, "m2_C", slot, (T, Bt, G, N), scale=1.0 / math.sqrt(N)).astype(np.float32)
    dt = _softplus(_normal(seed, "m2_dt", slot, (T, Bt, H), loc=-2.0, scale=0.5)).astype(np.float32)
    return {"x": x, "B": Bm, "C": C, "dt": dt}


def gdn_state0(shape: GDNShape, seed: int = 0) -> np.ndarray:
    s = shape
    return _normal(seed, "gdn_state0", 0, (s.batch, s.nheads, s.d_v, s.d_k),
                   scale=0.1).astype(np.float32)


def _l2n(z: np.ndarray) -> np.ndarray:
    return z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True))


def gdn_token_inputs(shape: GDNShape, seed: int, slot: int, ntok: int = 1) -> dict:
    """Inputs of `ntok` tokens: q, k [T,B,H,d_k], v [T,B,H,d_v], beta, alpha [T,B,H]."""
    s = shape
    T, Bt, H = ntok, s.batch, s.nheads
    q = _l2n(_normal(seed, "gdn_q", slot, (T, Bt, H, s.d_k))).astype(np.float32)
    k = _l2n(_normal(seed, "gdn_k", slot, (T, Bt, H, s.d_k))).astype(np.float32)
    v = _normal(seed, "gdn_v", slot, (T, Bt, H, s.d_v)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-_normal(seed, "gdn_beta", slot, (T, Bt, H))))).astype(np.float32)
    alpha = np.exp(-_softplus(_normal(seed, "gdn_alpha", slot, (T, Bt, H)))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "beta": beta, "alpha": alpha}


def kda_state0(shape: GDNShape, seed: int = 0) -> np.ndarray:
    s = shape
    return _normal(seed, "kda_state0", 0, (s.batch, s.nheads, s.d_v, s.d_k),
                   scale=0.1).astype(np.float32)


def kda_token_inputs(shape: GDNShape, seed: int, slot: int, ntok: int = 1) -> dict:
    """Inputs of `ntok` Kimi Delta Attention tokens: q, k [T,B,H,d_k], v [T,B,H,d_v],
    beta [T,B,H], alpha [T,B,H,d_k] (one gate per key channel)."""
    s = shape
    T, Bt, H = ntok, s.batch, s.nheads
    q = _l2n(_normal(seed, "kda_q", slot, (T, Bt, H, s.d_k))).astype(np.float32)
    k = _l2n(_normal(seed, "kda_k", slot, (T, Bt, H, s.d_k))).astype(np.float32)
    v = _normal(seed, "kda_v", slot, (T, Bt, H, s.d_v)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-_normal(seed, "kda_beta", slot, (T, Bt, H))))).astype(np.float32)
    alpha = np.exp(-_softplus(_normal(seed, "kda_alpha", slot, (T, Bt, H, s.d_k)))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "beta": beta, "alpha": alpha}


def spec_accepted(batch: int, rounds: int, max_accept: int, p: float = 0.35,
                  seed: int = 0) -> np.ndarray:
    """Accepted draft counts [rounds, batch]: failures before the first success, capped at K."""
    g = _rng(seed, "accepted").geometric(p, size=(rounds, batch)) - 1
    return np.minimum(g, max_accept).astype(np.int32)


# Named workloads (tests and the bench refer to them by these names).
M2_TINY = M2Shape(batch=2, nheads=4, ngroups=4, head_dim=16, d_state=16, window=4)
M2_SERVE = M2Shape(batch=256, nheads=128, ngroups=128, head_dim=64, d_state=128, window=16)
M2_SPEC = M2Shape(batch=512, nheads=128, ngroups=128, head_dim=64, d_state=128, window=16,
                  max_draft=6)
GDN_SERVE = GDNShape(batch=256, nheads=32, d_k=128, d_v=128, window=16)
KDA_SERVE = GDNShape(batch=256, nheads=32, d_k=128, d_v=128, window=16)


def torch_prompt_inputs(kind: str, batch: int, nheads: int, dim_v: int, dim_k: int, ntok: int,
                        seed: int, device="cuda"):
    """Prompt inputs and an initial state drawn on the device with torch's seeded generator, in
    float32, for shapes too large to draw on the host; the distributions are the ones above
    (Mamba-2 with one B/C group per head). Token-major like the *_token_inputs functions. Returns
    (inputs, state0); Mamba-2's A and D come from m2_params."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))

    def nrm(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)

    T, B, H = ntok, batch, nheads
    if kind == "mamba2":
        x = nrm(T, B, H, dim_v)
        Bm = nrm(T, B, H, dim_k).mul_(1.0 / math.sqrt(dim_k))
        C = nrm(T, B, H, dim_k).mul_(1.0 / math.sqrt(dim_k))
        dt = torch.nn.functional.softplus(nrm(T, B, H).mul_(0.5).add_(-2.0))
        ins = {"x": x, "B": Bm, "C": C, "dt": dt}
    else:
        q = nrm(T, B, H, dim_k)
        q.div_(q.norm(dim=-1, keepdim=True))
        k = nrm(T, B, H, dim_k)
        k.div_(k.norm(dim=-1, keepdim=True))
        v = nrm(T, B, H, dim_v)
        beta = torch.sigmoid(nrm(T, B, H))
        ga = nrm(T, B, H, dim_k) if kind == "kda" else nrm(T, B, H)
        alpha = torch.exp(-torch.nn.functional.softplus(ga))
        ins = {"q": q, "k": k, "v": v, "beta": beta, "alpha": alpha}
    return ins, nrm(B, H, dim_v, dim_k).mul_(0.1)
