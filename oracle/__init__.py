"""CPU oracle for the ReplaySSM decode path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The decode library (C ABI + HIP kernels) shares no code with it, and its Python
binding never imports it.

Contents
--------
* ``m2_step`` / ``gdn_step``: one conventional decode token (plain C, fp64, ``oracle.c``).
* ``m2_conventional`` / ``gdn_conventional``: those steps run over a token schedule.
* ``Bookkeeping``: the integer model of the ring pointers (head, len, ndraft) and of the
  commit / rollback rules, which the device bookkeeping must match bit for bit.
* ``kda_step`` and friends: the Kimi Delta Attention counterparts (a per key channel gate; the
  pages name the layer type without a formula, so the step is the reading stated in ``oracle.c``).
* ``M2Replay`` / ``GDNReplay`` / ``KDAReplay``: fp64 numpy models of the checkpoint + ring-buffer form itself
  (append, replay output, consolidation, speculative verify, commit, rollback). They exist so that
  the invariants the pages fix -- replayed outputs equal conventional decoding, consolidation equals
  the sequential steps, rollback equals recomputation from the accepted prefix -- can be checked on
  the CPU, and they carry the bookkeeping rules for the GPU comparison.

The method (five short web articles describing ReplaySSM):
* the state of an SSM layer is kept as a checkpoint plus a short buffer of recent inputs
  (ia.goatify.app article, paragraph "ReplaySSM cambia qué se almacena"; newsverum.com item,
  lede);
* a normal step appends its inputs to the buffer and computes the output from the checkpoint; the
  checkpoint is consolidated only when the buffer is full (ia.goatify.app, "El checkpoint reduce
  escrituras de estado");
* speculative decoding keeps the drafts' inputs and accepts a prefix by moving a pointer to the
  last accepted token, with no per-draft state copy (ia.goatify.app, "El retroceso usa un puntero
  del búfer"; fagnersouza.tech post, "O que muda para quem desenvolve");
* an optional lower-precision copy of the checkpoint serves reads while the recurrence stays in
  high precision (ia.goatify.app, "La precisión separa lectura y recurrencia").

Readings adopted where the pages are silent (each also listed in the design notes):
R1 per-head B and C by default (groups G = H); R2 dt arrives positive; R3 Mamba-2 update
``S <- exp(dt A) S + dt x B^T``, output ``y = S C + D x`` from the post-update state; R6 eager
consolidation in the step whose entry fills the buffer, and before a verify whose drafts would not
fit; R7 logical entry j lives in ring slot ``(head + j) mod W``, a fold of n entries moves head by
n; R11 the decay weight of entry j is the product of the later entries' per-step decays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RSSM_ORACLE_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer
# (the process must then preload libasan, e.g. LD_PRELOAD=$(gcc -print-file-name=libasan.so)).
_SANITIZE = os.environ.get("RSSM_ORACLE_SANITIZE") == "1"
_SO = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (fp64, no contraction, OpenMP)."""
    if force or not os.path.exists(_SO):
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-g"] if _SANITIZE else []
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", *san,
               "-shared", os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        fp = ctypes.c_void_p
        i = ctypes.c_int
        lib.orc_m2_step.argtypes = [i, i, i, i, i, fp, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_m2_step.restype = None
        lib.orc_gdn_step.argtypes = [i, i, i, i, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_gdn_step.restype = None
        lib.orc_m2_step_f32.argtypes = [i, i, i, i, i, fp, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_m2_step_f32.restype = None
        lib.orc_gdn_kappa_step.argtypes = [i, i, i, i, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_gdn_kappa_step.restype = None
        lib.orc_kda_step.argtypes = [i, i, i, i, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_kda_step.restype = None
        lib.orc_kda_kappa_step.argtypes = [i, i, i, i, fp, fp, fp, fp, fp, fp, fp]
        lib.orc_kda_kappa_step.restype = None
        lib.orc_set_threads.argtypes = [i]
        lib.orc_set_threads.restype = i
        _lib = lib
    return _lib


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (n <= 0 keeps it); returns the count in use."""
    return _load().orc_set_threads(int(n))


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data


def _chk64(a):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ----------------------------------------------------------------------------------------------
# Conventional recurrences (the definition)
# ----------------------------------------------------------------------------------------------

def m2_step(A, D, x, Bm, C, dt, state: np.ndarray) -> np.ndarray:
    """One conventional Mamba-2 token. ``state`` [B,H,P,N] float64 is updated in place.

    x [B,H,P], Bm and C [B,G,N], dt [B,H], A and D [H] (float32). Returns y [B,H,P] float64.
    """
    nb, nh, P, N = state.shape
    ng = Bm.shape[1]
    assert nh % ng == 0 and x.shape == (nb, nh, P) and Bm.shape == (nb, ng, N)
    assert C.shape == (nb, ng, N) and dt.shape == (nb, nh)
    keep = [_f32(v) for v in (A, D, x, Bm, C, dt)]
    y = np.empty((nb, nh, P), dtype=np.float64)
    _load().orc_m2_step(nb, nh, ng, P, N, *[k[1] for k in keep], _chk64(state), _chk64(y))
    return y


def m2_step_f32(A, D, x, Bm, C, dt, state32: np.ndarray) -> np.ndarray:
    """One conventional Mamba-2 token in fp32 arithmetic (``oracle.c``: orc_m2_step_f32).
    ``state32`` [B,H,P,N] float32 is updated in place; returns y [B,H,P] float32. It measures how
    far fp32 conventional decoding itself lands from the fp64 definition on given inputs."""
    nb, nh, P, N = state32.shape
    ng = Bm.shape[1]
    assert nh % ng == 0 and x.shape == (nb, nh, P) and Bm.shape == (nb, ng, N)
    assert C.shape == (nb, ng, N) and dt.shape == (nb, nh)
    assert state32.dtype == np.float32 and state32.flags["C_CONTIGUOUS"]
    keep = [_f32(v) for v in (A, D, x, Bm, C, dt)]
    y = np.empty((nb, nh, P), dtype=np.float32)
    _load().orc_m2_step_f32(nb, nh, ng, P, N, *[k[1] for k in keep], state32.ctypes.data,
                            y.ctypes.data)
    return y


def m2_kappa_step(A, D, x, Bm, C, dt, M: np.ndarray) -> np.ndarray:
    """Conditioning of one Mamba-2 token: the recurrence on absolute values. ``M`` [B,H,P,N]
    float64 (start it at |S_0|) is updated in place to
        M <- exp(dt A) M + dt |x| |B|^T
    (dt > 0, so every coefficient is non-negative and M bounds entry by entry the absolute value
    of every partial sum of the state's terms, in any evaluation order), and the return value
        kappa[p] = sum_n M[p,n] |C_n| + |D x_p|
    bounds the terms of the output y = S C + D x. A relative perturbation e of every term moves
    y_p by at most e kappa_p. It is the conventional step run on |x|, |B|, |C|, |D|."""
    ab = lambda a: np.abs(np.asarray(a, dtype=np.float32))
    return m2_step(A, ab(D), ab(x), ab(Bm), ab(C), dt, M)


def gdn_kappa_step(q, k, v, beta, alpha, M: np.ndarray) -> np.ndarray:
    """Conditioning of one Gated DeltaNet token (``oracle.c``: orc_gdn_kappa_step). ``M``
    [B,H,dv,dk] float64, start at |S_0|, updated in place; returns kappa [B,H,dv]."""
    nb, nh, dv, dk = M.shape
    keep = [_f32(a) for a in (q, k, v, beta, alpha)]
    kap = np.empty((nb, nh, dv), dtype=np.float64)
    _load().orc_gdn_kappa_step(nb, nh, dk, dv, *[kk[1] for kk in keep], _chk64(M), _chk64(kap))
    return kap


def gdn_step(q, k, v, beta, alpha, state: np.ndarray) -> np.ndarray:
    """One conventional Gated DeltaNet token. ``state`` [B,H,dv,dk] float64, updated in place."""
    nb, nh, dv, dk = state.shape
    assert q.shape == (nb, nh, dk) and k.shape == (nb, nh, dk) and v.shape == (nb, nh, dv)
    assert beta.shape == (nb, nh) and alpha.shape == (nb, nh)
    keep = [_f32(a) for a in (q, k, v, beta, alpha)]
    o = np.empty((nb, nh, dv), dtype=np.float64)
    _load().orc_gdn_step(nb, nh, dk, dv, *[kk[1] for kk in keep], _chk64(state), _chk64(o))
    return o


def kda_step(q, k, v, beta, a, state: np.ndarray) -> np.ndarray:
    """One conventional Kimi Delta Attention token (``oracle.c``: orc_kda_step): per key channel
    gate a [B,H,dk]; ``state`` [B,H,dv,dk] float64, updated in place; returns o [B,H,dv]."""
    nb, nh, dv, dk = state.shape
    assert q.shape == (nb, nh, dk) and k.shape == (nb, nh, dk) and v.shape == (nb, nh, dv)
    assert beta.shape == (nb, nh) and a.shape == (nb, nh, dk)
    keep = [_f32(x) for x in (q, k, v, beta, a)]
    o = np.empty((nb, nh, dv), dtype=np.float64)
    _load().orc_kda_step(nb, nh, dk, dv, *[kk[1] for kk in keep], _chk64(state), _chk64(o))
    return o


def kda_kappa_step(q, k, v, beta, a, M: np.ndarray) -> np.ndarray:
    """Conditioning of one Kimi Delta Attention token (``oracle.c``: orc_kda_kappa_step). ``M``
    [B,H,dv,dk] float64, start at |S_0|, updated in place; returns kappa [B,H,dv]."""
    nb, nh, dv, dk = M.shape
    keep = [_f32(x) for x in (q, k, v, beta, a)]
    kap = np.empty((nb, nh, dv), dtype=np.float64)
    _load().orc_kda_kappa_step(nb, nh, dk, dv, *[kk[1] for kk in keep], _chk64(M), _chk64(kap))
    return kap


def m2_conventional(A, D, tokens, state0) -> tuple[np.ndarray, np.ndarray]:
    """Run conventional decoding over ``tokens`` (an iterable of dicts with x, B, C, dt, one token
    each). Returns (y [T,B,H,P] float64, final state float64)."""
    state = np.array(state0, dtype=np.float64, order="C", copy=True)
    ys = [m2_step(A, D, t["x"], t["B"], t["C"], t["dt"], state) for t in tokens]
    return np.stack(ys), state


def gdn_conventional(tokens, state0) -> tuple[np.ndarray, np.ndarray]:
    state = np.array(state0, dtype=np.float64, order="C", copy=True)
    os_ = [gdn_step(t["q"], t["k"], t["v"], t["beta"], t["alpha"], state) for t in tokens]
    return np.stack(os_), state


def m2_spec_round(A, D, drafts: dict, state: np.ndarray, accepted) -> np.ndarray:
    """One speculative round by recomputation: from the committed ``state`` run the K drafts
    conventionally (y_1..y_K), then keep, per sequence b, the state after ``accepted[b]`` drafts
    (the committed state itself when it is 0). ``state`` is updated in place; returns y [K,B,H,P].
    This is the conventional reading of a rollback: a state snapshot after every draft."""
    K = drafts["x"].shape[0]
    acc = np.asarray(accepted)
    work = state.copy()
    keep = state.copy()
    ys = []
    for k in range(K):
        ys.append(m2_step(A, D, drafts["x"][k], drafts["B"][k], drafts["C"][k], drafts["dt"][k],
                          work))
        sel = acc == k + 1
        keep[sel] = work[sel]
    state[...] = keep
    return np.stack(ys)


def m2_spec_kappa(A, D, drafts: dict, M: np.ndarray, accepted) -> np.ndarray:
    """Conditioning (m2_kappa_step) of the K draft outputs of a speculative round, with ``M``
    [B,H,P,N] kept, per sequence, after ``accepted[b]`` drafts, as m2_spec_round keeps the state.
    Returns kappa [K,B,H,P]."""
    K = drafts["x"].shape[0]
    acc = np.asarray(accepted)
    work = M.copy()
    keep = M.copy()
    ks = []
    for k in range(K):
        ks.append(m2_kappa_step(A, D, drafts["x"][k], drafts["B"][k], drafts["C"][k],
                                drafts["dt"][k], work))
        sel = acc == k + 1
        keep[sel] = work[sel]
    M[...] = keep
    return np.stack(ks)


def gdn_spec_round(drafts: dict, state: np.ndarray, accepted) -> np.ndarray:
    """Gated DeltaNet counterpart of m2_spec_round: from the committed ``state`` [B,H,dv,dk] run
    the K drafts (q, k, v, beta, alpha with a leading K axis) conventionally, keep per sequence b
    the state after ``accepted[b]`` drafts; ``state`` is updated in place; returns o [K,B,H,dv]."""
    K = drafts["q"].shape[0]
    acc = np.asarray(accepted)
    work = state.copy()
    keep = state.copy()
    os_ = []
    for k in range(K):
        os_.append(gdn_step(drafts["q"][k], drafts["k"][k], drafts["v"][k], drafts["beta"][k],
                            drafts["alpha"][k], work))
        sel = acc == k + 1
        keep[sel] = work[sel]
    state[...] = keep
    return np.stack(os_)


def kda_conventional(tokens, state0) -> tuple[np.ndarray, np.ndarray]:
    state = np.array(state0, dtype=np.float64, order="C", copy=True)
    os_ = [kda_step(t["q"], t["k"], t["v"], t["beta"], t["alpha"], state) for t in tokens]
    return np.stack(os_), state


def kda_spec_round(drafts: dict, state: np.ndarray, accepted) -> np.ndarray:
    """Kimi Delta Attention counterpart of m2_spec_round (drafts q, k, v, beta, alpha with a
    leading K axis; alpha [K,B,H,dk]); ``state`` is updated in place; returns o [K,B,H,dv]."""
    K = drafts["q"].shape[0]
    acc = np.asarray(accepted)
    work = state.copy()
    keep = state.copy()
    os_ = []
    for k in range(K):
        os_.append(kda_step(drafts["q"][k], drafts["k"][k], drafts["v"][k], drafts["beta"][k],
                            drafts["alpha"][k], work))
        sel = acc == k + 1
        keep[sel] = work[sel]
    state[...] = keep
    return np.stack(os_)


def kda_spec_kappa(drafts: dict, M: np.ndarray, accepted) -> np.ndarray:
    """Conditioning (kda_kappa_step) of the K draft outputs of a speculative round, ``M`` kept per
    sequence after ``accepted[b]`` drafts. Returns kappa [K,B,H,dv]."""
    K = drafts["q"].shape[0]
    acc = np.asarray(accepted)
    work = M.copy()
    keep = M.copy()
    ks = []
    for k in range(K):
        ks.append(kda_kappa_step(drafts["q"][k], drafts["k"][k], drafts["v"][k],
                                 drafts["beta"][k], drafts["alpha"][k], work))
        sel = acc == k + 1
        keep[sel] = work[sel]
    M[...] = keep
    return np.stack(ks)


def token(inputs: dict, t: int) -> dict:
    """Token ``t`` of a dict of arrays with a leading token axis."""
    return {k: v[t] for k, v in inputs.items()}


# ----------------------------------------------------------------------------------------------
# Integer bookkeeping model (ring pointers, commit / rollback)
# ----------------------------------------------------------------------------------------------

COMMIT_RANGE = 1     # device error bit: accepted[b] outside [0, ndraft[b]]
ROLLBACK_RANGE = 2   # device error bit: new_len[b] outside [0, len[b]]


class StateError(Exception):
    """Call-order misuse that the host can see (mirrors the library's RSSM_E_STATE)."""


class Bookkeeping:
    """head / len / ndraft per sequence and the rules every entry point applies to them.

    * decode: the token becomes logical entry ``len``; with ``m = len + 1`` entries, if ``m >= W``
      the whole buffer (ring entries plus this token) is folded: ``head <- (head + m) mod W``,
      ``len <- 0``; otherwise ``len <- m``. Needs no pending drafts.
    * verify(K): if ``len + K > W`` the committed entries are folded first
      (``head <- (head + len) mod W``, ``len <- 0``); the K drafts become entries
      ``len .. len+K-1``; ``ndraft <- K``.
    * commit(a): ``len <- len + a`` if ``0 <= a <= ndraft``, else the COMMIT_RANGE bit;
      ``ndraft <- 0`` either way.
    * rollback(L): ``len <- L`` if ``0 <= L <= len``, else the ROLLBACK_RANGE bit; ``ndraft <- 0``.
    * consolidate(min_len): sequences with ``len >= max(min_len, 1)`` fold their entries.
    """

    def __init__(self, batch: int, window: int, max_draft: int = 0):
        self.W = int(window)
        self.K = int(max_draft)
        self.head = np.zeros(batch, dtype=np.int64)
        self.len = np.zeros(batch, dtype=np.int64)
        self.ndraft = np.zeros(batch, dtype=np.int64)
        self.err = 0
        self.pending = False

    def init(self, mask=None):
        sel = slice(None) if mask is None else np.asarray(mask) != 0
        self.head[sel] = 0
        self.len[sel] = 0
        self.ndraft[sel] = 0
        if mask is None:
            self.err = 0
        self.pending = False

    def decode(self) -> np.ndarray:
        """Returns the boolean mask of sequences folded in this step."""
        if self.pending:
            raise StateError("decode with pending drafts")
        m = self.len + 1
        fold = m >= self.W
        self.head = np.where(fold, (self.head + m) % self.W, self.head)
        self.len = np.where(fold, 0, m)
        return fold

    def consolidate(self, min_len: int) -> np.ndarray:
        if self.pending:
            raise StateError("consolidate with pending drafts")
        fold = self.len >= max(int(min_len), 1)
        self.head = np.where(fold, (self.head + self.len) % self.W, self.head)
        self.len = np.where(fold, 0, self.len)
        return fold

    def verify(self, K: int) -> np.ndarray:
        if self.pending:
            raise StateError("verify with pending drafts")
        if K < 1 or K > self.W or K > self.K:
            raise ValueError("bad draft count")
        fold = self.len + K > self.W
        self.head = np.where(fold, (self.head + self.len) % self.W, self.head)
        self.len = np.where(fold, 0, self.len)
        self.ndraft[:] = K
        self.pending = True
        return fold

    def commit(self, accepted):
        if not self.pending:
            raise StateError("commit without a verify")
        a = np.asarray(accepted, dtype=np.int64)
        ok = (a >= 0) & (a <= self.ndraft)
        if not ok.all():
            self.err |= COMMIT_RANGE
        self.len = np.where(ok, self.len + a, self.len)
        self.ndraft[:] = 0
        self.pending = False

    def rollback(self, new_len):
        nl = np.asarray(new_len, dtype=np.int64)
        ok = (nl >= 0) & (nl <= self.len)
        if not ok.all():
            self.err |= ROLLBACK_RANGE
        self.len = np.where(ok, nl, self.len)
        self.ndraft[:] = 0
        self.pending = False

    def read_err(self) -> int:
        e, self.err = self.err, 0
        return e

    def snapshot(self):
        return self.head.copy(), self.len.copy(), self.ndraft.copy()


# ----------------------------------------------------------------------------------------------
# bf16 read copy (round to nearest even from the fp32 value)
# ----------------------------------------------------------------------------------------------

def round_bf16(a: np.ndarray) -> np.ndarray:
    """Value of bf16(fp32(a)) with round-to-nearest-even, returned as float64 (finite inputs)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Mamba-2 checkpoint + ring replay model (fp64)
# ----------------------------------------------------------------------------------------------

def _m2_decay(dts: np.ndarray, A: float):
    """For entries with step sizes dts[0..m-1] (oldest first): the decay of the whole window,
    prod_i exp(dt_i A), and each entry's weight w_j = dt_j * prod_{i>j} exp(dt_i A)."""
    a = np.exp(dts.astype(np.float64) * float(A))
    m = len(dts)
    w = np.empty(m)
    later = 1.0
    for j in range(m - 1, -1, -1):
        w[j] = float(dts[j]) * later
        later *= a[j]
    return later, w


class M2Replay:
    """Checkpoint S0 (fp64 here) + ring of the last W tokens' (x, B, C, dt) per sequence.

    A normal step never writes S0; S0 changes only when entries are folded (consolidation).
    With ``bf16_read`` the checkpoint term of a replayed output reads bf16(fp32(S0)), refreshed
    at init and at every fold, while folds keep using the full-precision S0.
    """

    def __init__(self, A, D, state0, ngroups: int, window: int, max_draft: int = 0,
                 bf16_read: bool = False):
        nb, nh, P, N = state0.shape
        self.A = np.asarray(A, dtype=np.float32)
        self.D = np.asarray(D, dtype=np.float32)
        self.G, self.W, self.bf16 = int(ngroups), int(window), bool(bf16_read)
        self.hpg = nh // self.G
        self.nb, self.nh, self.P, self.N = nb, nh, P, N
        self.bk = Bookkeeping(nb, window, max_draft)
        self.S0 = np.array(state0, dtype=np.float64, copy=True)
        self.rx = np.zeros((nb, nh, window, P))
        self.rB = np.zeros((nb, self.G, window, N))
        self.rC = np.zeros((nb, self.G, window, N))
        self.rdt = np.zeros((nb, nh, window), dtype=np.float32)
        self._refresh()

    def _refresh(self, b=None):
        if self.bf16:
            if b is None:
                self.S0r = round_bf16(self.S0)
            else:
                self.S0r[b] = round_bf16(self.S0[b])
        else:
            self.S0r = self.S0

    # entries of sequence b, head h, in logical order: ring[0..n-1] then the extra tokens
    def _entries(self, b, h, n, extra):
        W, g, hd = self.W, h // self.hpg, int(self.bk.head[b])
        xs = [self.rx[b, h, (hd + j) % W] for j in range(n)]
        Bs = [self.rB[b, g, (hd + j) % W] for j in range(n)]
        dts = [self.rdt[b, h, (hd + j) % W] for j in range(n)]
        for e in extra:
            xs.append(e["x"][b, h].astype(np.float64))
            Bs.append(e["B"][b, g].astype(np.float64))
            dts.append(e["dt"][b, h])
        return np.array(xs).reshape(-1, self.P), np.array(Bs).reshape(-1, self.N), \
            np.array(dts, dtype=np.float32)

    def _fold(self, b, n, extra=()):
        """S0[b] <- (window decay) S0[b] + sum_j w_j x_j B_j^T over the first n ring entries and the
        extra tokens."""
        for h in range(self.nh):
            X, Bm, dts = self._entries(b, h, n, extra)
            if len(dts) == 0:
                continue
            lam, w = _m2_decay(dts, self.A[h])
            self.S0[b, h] = lam * self.S0[b, h] + (X * w[:, None]).T @ Bm

    def _append(self, b, pos, tok):
        slot = (int(self.bk.head[b]) + pos) % self.W
        self.rx[b, :, slot] = tok["x"][b]
        self.rdt[b, :, slot] = tok["dt"][b]
        self.rB[b, :, slot] = tok["B"][b]
        self.rC[b, :, slot] = tok["C"][b]

    def _replay_out(self, b, n, extra, C):
        """Output of the newest entry: ring entries [0, n) then the extra tokens (newest last)."""
        y = np.empty((self.nh, self.P))
        for h in range(self.nh):
            g = h // self.hpg
            X, Bm, dts = self._entries(b, h, n, extra)
            lam, w = _m2_decay(dts, self.A[h])
            c = C[b, g].astype(np.float64)
            z = self.S0r[b, h] @ c
            s = Bm @ c
            y[h] = lam * z + (w * s) @ X + float(self.D[h]) * extra[-1]["x"][b, h].astype(np.float64)
        return y

    def init(self, state, mask=None):
        sel = range(self.nb) if mask is None else [b for b in range(self.nb) if mask[b]]
        for b in sel:
            self.S0[b] = state[b]
        self._refresh()
        self.bk.init(mask)

    def decode(self, tok) -> np.ndarray:
        """tok: dict x [B,H,P], B, C [B,G,N], dt [B,H]. Returns y [B,H,P]."""
        if self.bk.pending:
            raise StateError("decode with pending drafts")
        y = np.empty((self.nb, self.nh, self.P))
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n + 1 >= self.W:
                self._fold(b, n, [tok])
                self._refresh(b)
                for h in range(self.nh):
                    g = h // self.hpg
                    y[b, h] = self.S0[b, h] @ tok["C"][b, g].astype(np.float64) \
                        + float(self.D[h]) * tok["x"][b, h].astype(np.float64)
            else:
                y[b] = self._replay_out(b, n, [tok], tok["C"])
                self._append(b, n, tok)
        self.bk.decode()
        return y

    def consolidate(self, min_len: int):
        if self.bk.pending:
            raise StateError("consolidate with pending drafts")
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n >= max(int(min_len), 1):
                self._fold(b, n)
                self._refresh(b)
        self.bk.consolidate(min_len)

    def verify(self, drafts: dict) -> np.ndarray:
        """drafts: dict with a leading token axis K. Returns y [K,B,H,P] (causal)."""
        K = drafts["x"].shape[0]
        if self.bk.pending:
            raise StateError("verify with pending drafts")
        toks = [token(drafts, k) for k in range(K)]
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n + K > self.W:
                self._fold(b, n)
                self._refresh(b)
        self.bk.verify(K)
        y = np.empty((K, self.nb, self.nh, self.P))
        for b in range(self.nb):
            n = int(self.bk.len[b])
            for k in range(K):
                y[k, b] = self._replay_out(b, n, toks[:k + 1], toks[k]["C"])
            for k in range(K):
                self._append(b, n + k, toks[k])
        return y

    def commit(self, accepted):
        self.bk.commit(accepted)

    def rollback(self, new_len):
        self.bk.rollback(new_len)

    def materialize(self) -> np.ndarray:
        """The current state (S0 folded with the committed entries); nothing is modified."""
        out = np.empty_like(self.S0)
        for b in range(self.nb):
            n = int(self.bk.len[b])
            for h in range(self.nh):
                X, Bm, dts = self._entries(b, h, n, ())
                if len(dts) == 0:
                    out[b, h] = self.S0[b, h]
                    continue
                lam, w = _m2_decay(dts, self.A[h])
                out[b, h] = lam * self.S0[b, h] + (X * w[:, None]).T @ Bm
        return out


# ----------------------------------------------------------------------------------------------
# Gated DeltaNet checkpoint + ring replay model (fp64)
# ----------------------------------------------------------------------------------------------

def gdn_replay_output(S0, ks, vs, betas, alphas, q):
    """Output of the newest of m buffered entries from checkpoint S0 (d_v x d_k).

    The state after the entries is S0 M_1 ... M_m + sum_j beta_j v_j k_j^T M_{j+1} ... M_m with
    M_i = alpha_i (I - beta_i k_i k_i^T). Applying it to q right to left: keep r (initially q),
    and for j = m..1 take c_j = k_j . r, add (prod_{i>j} alpha_i) beta_j c_j v_j to the output and
    replace r by r - beta_j c_j k_j; finally add (prod_i alpha_i) S0 r.
    """
    # every operand in fp64: a float32 array times a Python float stays float32 under NumPy's
    # promotion rules
    S0 = np.asarray(S0, dtype=np.float64)
    ks = np.asarray(ks, dtype=np.float64)
    vs = np.asarray(vs, dtype=np.float64)
    r = np.array(q, dtype=np.float64)
    acc = np.zeros(S0.shape[0])
    later = 1.0
    for j in range(len(betas) - 1, -1, -1):
        c = float(np.dot(ks[j], r))
        acc += later * float(betas[j]) * c * vs[j]
        r = r - float(betas[j]) * c * ks[j]
        later *= float(alphas[j])
    return later * (S0 @ r) + acc


def gdn_wy_fold(S0, ks, vs, betas, alphas):
    """Fold m entries into S0 using the WY form of the product of the m rank-1 corrections.

    With gamma_t = prod_{i<=t} alpha_i:
      y_t = beta_t (k_t - sum_{i<t} y_i (k_i . k_t))         (prod_t (I - beta_t k_t k_t^T) = I - Y^T K)
      u_t = beta_t (v_t - sum_{i<t} (gamma_t / gamma_i) u_i (k_i . k_t))
      S   = gamma_m S0 + (U^T diag(gamma_m / gamma_t) - gamma_m S0 Y^T) K
    """
    K = np.array(ks, dtype=np.float64)
    V = np.array(vs, dtype=np.float64)
    m = K.shape[0]
    gam = np.cumprod(np.asarray(alphas, dtype=np.float64))
    gram = K @ K.T
    Y = np.zeros_like(K)
    U = np.zeros_like(V)
    for t in range(m):
        Y[t] = float(betas[t]) * (K[t] - gram[:t, t] @ Y[:t])
        U[t] = float(betas[t]) * (V[t] - (gram[:t, t] * (gam[t] / gam[:t])) @ U[:t])
    gm = gam[-1]
    return gm * S0 + (U.T * (gm / gam)[None, :] - gm * (S0 @ Y.T)) @ K


class GDNReplay:
    """Gated DeltaNet checkpoint + ring of the last W tokens' (k, v, beta, alpha) per (b, h)."""

    def __init__(self, state0, window: int):
        nb, nh, dv, dk = state0.shape
        self.nb, self.nh, self.dv, self.dk, self.W = nb, nh, dv, dk, int(window)
        self.bk = Bookkeeping(nb, window, 0)
        self.S0 = np.array(state0, dtype=np.float64, copy=True)
        self.rk = np.zeros((nb, nh, window, dk))
        self.rv = np.zeros((nb, nh, window, dv))
        self.rbeta = np.zeros((nb, nh, window), dtype=np.float32)
        self.ralpha = np.zeros((nb, nh, window), dtype=np.float32)

    def _entries(self, b, h, n, tok=None):
        W, hd = self.W, int(self.bk.head[b])
        sl = [(hd + j) % W for j in range(n)]
        ks = [self.rk[b, h, s] for s in sl]
        vs = [self.rv[b, h, s] for s in sl]
        be = [self.rbeta[b, h, s] for s in sl]
        al = [self.ralpha[b, h, s] for s in sl]
        if tok is not None:
            ks.append(tok["k"][b, h].astype(np.float64))
            vs.append(tok["v"][b, h].astype(np.float64))
            be.append(tok["beta"][b, h])
            al.append(tok["alpha"][b, h])
        return ks, vs, be, al

    def decode(self, tok) -> np.ndarray:
        o = np.empty((self.nb, self.nh, self.dv))
        for b in range(self.nb):
            n = int(self.bk.len[b])
            for h in range(self.nh):
                ks, vs, be, al = self._entries(b, h, n, tok)
                q = tok["q"][b, h].astype(np.float64)
                if n + 1 >= self.W:
                    self.S0[b, h] = gdn_wy_fold(self.S0[b, h], ks, vs, be, al)
                    o[b, h] = self.S0[b, h] @ q
                else:
                    o[b, h] = gdn_replay_output(self.S0[b, h], ks, vs, be, al, q)
            if n + 1 < self.W:
                s = (int(self.bk.head[b]) + n) % self.W
                self.rk[b, :, s] = tok["k"][b]
                self.rv[b, :, s] = tok["v"][b]
                self.rbeta[b, :, s] = tok["beta"][b]
                self.ralpha[b, :, s] = tok["alpha"][b]
        self.bk.decode()
        return o

    def consolidate(self, min_len: int):
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n >= max(int(min_len), 1):
                for h in range(self.nh):
                    ks, vs, be, al = self._entries(b, h, n)
                    self.S0[b, h] = gdn_wy_fold(self.S0[b, h], ks, vs, be, al)
        self.bk.consolidate(min_len)

    def materialize(self) -> np.ndarray:
        out = self.S0.copy()
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n:
                for h in range(self.nh):
                    ks, vs, be, al = self._entries(b, h, n)
                    out[b, h] = gdn_wy_fold(self.S0[b, h], ks, vs, be, al)
        return out


# ----------------------------------------------------------------------------------------------
# Kimi Delta Attention checkpoint + ring replay model (fp64)
# ----------------------------------------------------------------------------------------------

def kda_replay_output(S0, ks, vs, betas, alphas, q):
    """Output of the newest of m buffered entries from checkpoint S0 (d_v x d_k), entry j with key
    k_j, value v_j, beta_j and per-channel gate a_j (oldest first).

    The state after the entries is S0 M_1 ... M_m + sum_j beta_j v_j k_j^T M_{j+1} ... M_m with
    M_i = diag(a_i) (I - beta_i k_i k_i^T). Applying it to q right to left: keep r (initially q);
    for j = m..1 take c_j = k_j . r, add beta_j c_j v_j to the output and replace r by
    a_j o (r - beta_j c_j k_j); finally add S0 r. The gates act on r channel by channel, so no
    decay factor multiplies the checkpoint term or the value sum.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    r = np.array(q, dtype=np.float64)
    acc = np.zeros(S0.shape[0])
    for j in range(len(betas) - 1, -1, -1):
        kj = np.asarray(ks[j], dtype=np.float64)
        c = float(np.dot(kj, r))
        acc += float(betas[j]) * c * np.asarray(vs[j], dtype=np.float64)
        r = np.asarray(alphas[j], dtype=np.float64) * (r - float(betas[j]) * c * kj)
    return S0 @ r + acc


def kda_fold(S0, ks, vs, betas, alphas):
    """Fold m entries into S0: the entries' updates applied in order (the consolidation)."""
    S = np.array(S0, dtype=np.float64)
    for j in range(len(betas)):
        kj = np.asarray(ks[j], dtype=np.float64)
        S = S * np.asarray(alphas[j], dtype=np.float64)[None, :]
        S = S + float(betas[j]) * np.outer(np.asarray(vs[j], dtype=np.float64) - S @ kj, kj)
    return S


class KDAReplay:
    """Kimi Delta Attention checkpoint + ring of the last W tokens' (k, v, beta, gate vector)."""

    def __init__(self, state0, window: int, max_draft: int = 0):
        nb, nh, dv, dk = state0.shape
        self.nb, self.nh, self.dv, self.dk, self.W = nb, nh, dv, dk, int(window)
        self.bk = Bookkeeping(nb, window, max_draft)
        self.S0 = np.array(state0, dtype=np.float64, copy=True)
        self.rk = np.zeros((nb, nh, window, dk))
        self.rv = np.zeros((nb, nh, window, dv))
        self.rbeta = np.zeros((nb, nh, window), dtype=np.float32)
        self.ralpha = np.zeros((nb, nh, window, dk), dtype=np.float32)

    def _entries(self, b, h, n, extra=()):
        W, hd = self.W, int(self.bk.head[b])
        sl = [(hd + j) % W for j in range(n)]
        ks = [self.rk[b, h, s] for s in sl]
        vs = [self.rv[b, h, s] for s in sl]
        be = [self.rbeta[b, h, s] for s in sl]
        al = [self.ralpha[b, h, s] for s in sl]
        for e in extra:
            ks.append(e["k"][b, h].astype(np.float64))
            vs.append(e["v"][b, h].astype(np.float64))
            be.append(e["beta"][b, h])
            al.append(e["alpha"][b, h])
        return ks, vs, be, al

    def _append(self, b, pos, tok):
        s = (int(self.bk.head[b]) + pos) % self.W
        self.rk[b, :, s] = tok["k"][b]
        self.rv[b, :, s] = tok["v"][b]
        self.rbeta[b, :, s] = tok["beta"][b]
        self.ralpha[b, :, s] = tok["alpha"][b]

    def decode(self, tok) -> np.ndarray:
        if self.bk.pending:
            raise StateError("decode with pending drafts")
        o = np.empty((self.nb, self.nh, self.dv))
        for b in range(self.nb):
            n = int(self.bk.len[b])
            for h in range(self.nh):
                ks, vs, be, al = self._entries(b, h, n, [tok])
                q = tok["q"][b, h].astype(np.float64)
                if n + 1 >= self.W:
                    self.S0[b, h] = kda_fold(self.S0[b, h], ks, vs, be, al)
                    o[b, h] = self.S0[b, h] @ q
                else:
                    o[b, h] = kda_replay_output(self.S0[b, h], ks, vs, be, al, q)
            if n + 1 < self.W:
                self._append(b, n, tok)
        self.bk.decode()
        return o

    def consolidate(self, min_len: int):
        if self.bk.pending:
            raise StateError("consolidate with pending drafts")
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n >= max(int(min_len), 1):
                for h in range(self.nh):
                    self.S0[b, h] = kda_fold(self.S0[b, h], *self._entries(b, h, n))
        self.bk.consolidate(min_len)

    def verify(self, drafts: dict) -> np.ndarray:
        K = drafts["q"].shape[0]
        if self.bk.pending:
            raise StateError("verify with pending drafts")
        toks = [token(drafts, k) for k in range(K)]
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n + K > self.W:
                for h in range(self.nh):
                    self.S0[b, h] = kda_fold(self.S0[b, h], *self._entries(b, h, n))
        self.bk.verify(K)
        o = np.empty((K, self.nb, self.nh, self.dv))
        for b in range(self.nb):
            n = int(self.bk.len[b])
            for k in range(K):
                for h in range(self.nh):
                    ks, vs, be, al = self._entries(b, h, n, toks[:k + 1])
                    o[k, b, h] = kda_replay_output(self.S0[b, h], ks, vs, be, al,
                                                   toks[k]["q"][b, h])
            for k in range(K):
                self._append(b, n + k, toks[k])
        return o

    def commit(self, accepted):
        self.bk.commit(accepted)

    def rollback(self, new_len):
        self.bk.rollback(new_len)

    def materialize(self) -> np.ndarray:
        out = self.S0.copy()
        for b in range(self.nb):
            n = int(self.bk.len[b])
            if n:
                for h in range(self.nh):
                    out[b, h] = kda_fold(self.S0[b, h], *self._entries(b, h, n))
        return out


# ----------------------------------------------------------------------------------------------
# Comparison metric
# ----------------------------------------------------------------------------------------------

def normwise_err(got, ref) -> float:
    """max over output vectors (last axis) of max|got - ref| / max|ref| (0 for an empty array)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


# Unit roundoff of fp32 and of bf16 (round to nearest).
U32 = 2.0 ** -24
U16 = 2.0 ** -8
# Rounding-error constant of the fp32 paths. A term of an output passes through at most about
# N + 2W + 8 roundings that the decay does not damp (the d_state products and their sum, the W
# buffered entries of the newest window and one fold's scale and sum; 168 at d_state 128, W 16);
# the worst-case bound of a sum evaluated in any order is then that many unit roundoffs of the
# sum of the absolute values of its terms (kappa). 256 covers it with room for the errors carried
# in the checkpoint from earlier windows, which each window's decay shrinks.
C_FP32 = 256


class Cond:
    """Result of ``cond_check``: the worst unfloored normwise error over the output vectors, how
    many vectors exceed the tolerance, the worst ratio |got - ref| / bound over the elements of
    those vectors (0 if there are none) and over all elements."""

    def __init__(self, worst, n_over, ratio_over, ratio_all, where):
        self.worst, self.n_over = worst, n_over
        self.ratio_over, self.ratio_all, self.where = ratio_over, ratio_all, where

    @property
    def ok(self) -> bool:
        """Every vector within the tolerance or, element by element, within its bound."""
        return self.ratio_over <= 1.0

    def __repr__(self):
        return (f"normwise {self.worst:.3e} ({self.n_over} vectors over tolerance, worst "
                f"|d|/bound there {self.ratio_over:.3f} at {self.where}); "
                f"worst |d|/bound over all elements {self.ratio_all:.3f}")


def cond_check(got, ref, bound, tol) -> Cond:
    """Per output vector (last axis): it passes when its normwise error max|d| / max|ref| is within
    ``tol``, or else when every element satisfies |d| <= ``bound`` (broadcast to ref's shape: the
    rounding-error bound of that element, e.g. C_FP32 * U32 * kappa)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), ref.shape)
    d = np.abs(got - ref)
    den = np.max(np.abs(ref), axis=-1)
    nw = np.max(d, axis=-1) / np.where(den == 0, 1.0, den)
    over = nw > tol
    r = np.max(d / np.where(bound > 0, bound, np.inf), axis=-1) if d.size else np.zeros(nw.shape)
    ratio_all = float(np.max(r)) if r.size else 0.0
    ratio_over, where = 0.0, None
    if over.any():
        ro = np.where(over, r, 0.0)
        idx = np.unravel_index(int(np.argmax(ro)), ro.shape)
        ratio_over, where = float(ro[idx]), tuple(int(v) for v in idx)
    worst = float(np.max(nw)) if nw.size else 0.0
    return Cond(worst, int(over.sum()), ratio_over, ratio_all, where)
