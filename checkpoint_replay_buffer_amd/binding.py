"""ctypes binding of librssm.so (the C ABI declared in include/rssm.h).

Argument marshalling only: every step of the decode path runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and streams. The module-level functions carry the C
names; ``Context`` bundles a context with its torch-allocated workspace.

Loading fails loudly when the library is not built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librssm.so")

RSSM_OK = 0
STATUS = {0: "RSSM_OK", -1: "RSSM_E_ARG", -2: "RSSM_E_SHAPE", -3: "RSSM_E_SPACE",
          -4: "RSSM_E_STATE", -5: "RSSM_E_DEVICE", -6: "RSSM_E_UNSUPPORTED"}
RSSM_DEV_COMMIT_RANGE = 1
RSSM_DEV_ROLLBACK_RANGE = 2
RSSM_DEV_INDEX_RANGE = 8
RSSM_DEV_IMPORT_HEADER = 16
RSSM_MAMBA2 = 1
RSSM_GDN = 2
RSSM_KDA = 3
RSSM_F_BF16_READ = 1
RSSM_F_STORE_C = 2

EXPORTS = ("rssm_workspace_bytes", "rssm_create", "rssm_destroy", "rssm_set_params",
           "rssm_init_checkpoint", "rssm_decode_step", "rssm_consolidate", "rssm_prefill", "rssm_verify",
           "rssm_verify_commit", "rssm_rollback", "rssm_step_baseline", "rssm_step_baseline_seqs",
           "rssm_step_baseline_spec",
           "rssm_baseline_commit", "rssm_seq_state_bytes", "rssm_fork", "rssm_export", "rssm_import",
           "rssm_materialize", "rssm_read_bookkeeping", "rssm_status_str")


class RssmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_str(status)})")


class rssm_config(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("nheads", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("dim_v", ctypes.c_int32), ("dim_k", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_draft", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class rssm_inputs(ctypes.Structure):
    _fields_ = [("ntok", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("dt", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("alpha", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librssm.so. torch is imported first so that the process has a single HIP runtime
    (the library's libamdhip64.so.7 dependency resolves to the one torch already loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m checkpoint_replay_buffer_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    cfgp = ctypes.POINTER(rssm_config)
    inp = ctypes.POINTER(rssm_inputs)
    sig = {
        "rssm_workspace_bytes": (I32, [cfgp, ctypes.POINTER(SZ)]),
        "rssm_create": (I32, [cfgp, P, SZ, ctypes.POINTER(P)]),
        "rssm_destroy": (None, [P]),
        "rssm_set_params": (I32, [P, P, P]),
        "rssm_init_checkpoint": (I32, [P, P, P, P]),
        "rssm_decode_step": (I32, [P, inp, P, P]),
        "rssm_consolidate": (I32, [P, I32, P]),
        "rssm_prefill": (I32, [P, inp, P, P]),
        "rssm_verify": (I32, [P, inp, P, P]),
        "rssm_verify_commit": (I32, [P, P, P]),
        "rssm_rollback": (I32, [P, P, P]),
        "rssm_step_baseline": (I32, [cfgp, P, inp, P, P, P, P, P]),
        "rssm_step_baseline_seqs": (I32, [cfgp, P, inp, P, P, P, P, P]),
        "rssm_step_baseline_spec": (I32, [cfgp, P, P, inp, P, P, P, P]),
        "rssm_baseline_commit": (I32, [cfgp, P, P, I32, P]),
        "rssm_seq_state_bytes": (I32, [cfgp, ctypes.POINTER(SZ)]),
        "rssm_fork": (I32, [P, P, P, I32, P]),
        "rssm_export": (I32, [P, P, I32, P, P]),
        "rssm_import": (I32, [P, P, I32, P, P]),
        "rssm_materialize": (I32, [P, P, P]),
        "rssm_read_bookkeeping": (I32, [P, P, P, P, ctypes.POINTER(U32), P]),
        "rssm_status_str": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _chk(fn: str, st: int):
    if st != RSSM_OK:
        raise RssmError(fn, st)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_str(st: int) -> str:
    return load_library().rssm_status_str(int(st)).decode()


def make_config(kind, batch, nheads, ngroups, dim_v, dim_k, window, max_draft=0,
                flags=0) -> rssm_config:
    return rssm_config(int(kind), int(batch), int(nheads), int(ngroups), int(dim_v), int(dim_k),
                       int(window), int(max_draft), int(flags))


def make_inputs(ntok=1, x=None, B=None, C=None, dt=None, q=None, k=None, v=None, beta=None,
                alpha=None) -> rssm_inputs:
    return rssm_inputs(int(ntok), *[_ptr(t) for t in (x, B, C, dt, q, k, v, beta, alpha)])


# ---- the C ABI, one Python function per entry point -------------------------------------------

def rssm_workspace_bytes(cfg: rssm_config) -> int:
    n = ctypes.c_size_t(0)
    _chk("rssm_workspace_bytes", load_library().rssm_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def rssm_create(cfg: rssm_config, dev_ws: int, nbytes: int) -> int:
    h = ctypes.c_void_p(0)
    _chk("rssm_create", load_library().rssm_create(ctypes.byref(cfg), dev_ws, nbytes, ctypes.byref(h)))
    return h.value


def rssm_destroy(ctx: int) -> None:
    load_library().rssm_destroy(ctx)


def rssm_set_params(ctx: int, A, D) -> None:
    _chk("rssm_set_params", load_library().rssm_set_params(ctx, _ptr(A), _ptr(D)))


def rssm_init_checkpoint(ctx: int, state, seq_mask=None, stream=None) -> None:
    _chk("rssm_init_checkpoint",
         load_library().rssm_init_checkpoint(ctx, _ptr(state), _ptr(seq_mask), _stream(stream)))


def rssm_decode_step(ctx: int, inputs: rssm_inputs, y, stream=None) -> None:
    _chk("rssm_decode_step",
         load_library().rssm_decode_step(ctx, ctypes.byref(inputs), _ptr(y), _stream(stream)))


def rssm_consolidate(ctx: int, min_len: int, stream=None) -> None:
    _chk("rssm_consolidate", load_library().rssm_consolidate(ctx, int(min_len), _stream(stream)))


def rssm_prefill(ctx: int, inputs: rssm_inputs, y, stream=None) -> None:
    _chk("rssm_prefill", load_library().rssm_prefill(ctx, ctypes.byref(inputs), _ptr(y), _stream(stream)))


def rssm_verify(ctx: int, inputs: rssm_inputs, y, stream=None) -> None:
    _chk("rssm_verify", load_library().rssm_verify(ctx, ctypes.byref(inputs), _ptr(y), _stream(stream)))


def rssm_verify_commit(ctx: int, accepted, stream=None) -> None:
    _chk("rssm_verify_commit", load_library().rssm_verify_commit(ctx, _ptr(accepted), _stream(stream)))


def rssm_rollback(ctx: int, new_len, stream=None) -> None:
    _chk("rssm_rollback", load_library().rssm_rollback(ctx, _ptr(new_len), _stream(stream)))


def rssm_step_baseline(cfg: rssm_config, state, inputs: rssm_inputs, A, D, y, snapshots=None,
                       stream=None) -> None:
    _chk("rssm_step_baseline",
         load_library().rssm_step_baseline(ctypes.byref(cfg), _ptr(state), ctypes.byref(inputs),
                                           _ptr(A), _ptr(D), _ptr(y), _ptr(snapshots),
                                           _stream(stream)))


def rssm_step_baseline_seqs(cfg: rssm_config, seq_ptrs, inputs: rssm_inputs, A, D, y,
                            snapshots=None, stream=None) -> None:
    """seq_ptrs: int64 CUDA tensor [B] of device addresses of per-sequence [H,dim_v,dim_k] states."""
    _chk("rssm_step_baseline_seqs",
         load_library().rssm_step_baseline_seqs(ctypes.byref(cfg), _ptr(seq_ptrs),
                                                ctypes.byref(inputs), _ptr(A), _ptr(D), _ptr(y),
                                                _ptr(snapshots), _stream(stream)))


def rssm_step_baseline_spec(cfg: rssm_config, pool, slot_of, inputs: rssm_inputs, A, D, y,
                            stream=None) -> None:
    _chk("rssm_step_baseline_spec",
         load_library().rssm_step_baseline_spec(ctypes.byref(cfg), _ptr(pool), _ptr(slot_of),
                                                ctypes.byref(inputs), _ptr(A), _ptr(D), _ptr(y),
                                                _stream(stream)))


def rssm_baseline_commit(cfg: rssm_config, slot_of, accepted, ndraft: int, stream=None) -> None:
    _chk("rssm_baseline_commit",
         load_library().rssm_baseline_commit(ctypes.byref(cfg), _ptr(slot_of), _ptr(accepted),
                                             int(ndraft), _stream(stream)))


def rssm_seq_state_bytes(cfg: rssm_config) -> int:
    n = ctypes.c_size_t(0)
    _chk("rssm_seq_state_bytes", load_library().rssm_seq_state_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def rssm_fork(ctx: int, src, dst, n: int, stream=None) -> None:
    _chk("rssm_fork", load_library().rssm_fork(ctx, _ptr(src), _ptr(dst), int(n), _stream(stream)))


def rssm_export(ctx: int, seq, n: int, buf, stream=None) -> None:
    _chk("rssm_export", load_library().rssm_export(ctx, _ptr(seq), int(n), _ptr(buf), _stream(stream)))


def rssm_import(ctx: int, seq, n: int, buf, stream=None) -> None:
    _chk("rssm_import", load_library().rssm_import(ctx, _ptr(seq), int(n), _ptr(buf), _stream(stream)))


def rssm_materialize(ctx: int, state_out, stream=None) -> None:
    _chk("rssm_materialize", load_library().rssm_materialize(ctx, _ptr(state_out), _stream(stream)))


def rssm_read_bookkeeping(ctx: int, batch: int, stream=None):
    """Returns (head, len, ndraft, err) as Python lists / int; synchronises the stream."""
    arr = ctypes.c_int32 * batch
    h, l, n = arr(), arr(), arr()
    e = ctypes.c_uint32(0)
    _chk("rssm_read_bookkeeping",
         load_library().rssm_read_bookkeeping(ctx, h, l, n, ctypes.byref(e), _stream(stream)))
    return list(h), list(l), list(n), e.value


# ---- convenience wrapper ------------------------------------------------------------------------

def _f32(t, name):
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    return t


class Context:
    """A ReplaySSM context and its device workspace (a torch uint8 tensor it owns).

    kind 'mamba2', 'gdn' or 'kda'; dim_v / dim_k are (head_dim, d_state) for Mamba-2 and
    (d_v, d_k) for Gated DeltaNet and Kimi Delta Attention (whose alpha inputs carry one gate per
    key channel, [..., d_k]).
    """

    def __init__(self, kind: str, batch: int, nheads: int, dim_v: int, dim_k: int, window: int,
                 ngroups: int | None = None, max_draft: int = 0, bf16_read: bool = False,
                 store_c: bool = True, device="cuda"):
        k = {"mamba2": RSSM_MAMBA2, "gdn": RSSM_GDN, "kda": RSSM_KDA}[kind]
        flags = (RSSM_F_BF16_READ if bf16_read else 0) | \
                (RSSM_F_STORE_C if (store_c and k == RSSM_MAMBA2) else 0)
        self.kind = kind
        self.cfg = make_config(k, batch, nheads, ngroups or nheads, dim_v, dim_k, window,
                               max_draft, flags)
        self.nbytes = rssm_workspace_bytes(self.cfg)
        self._ws = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        base = self._ws.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        self.handle = rssm_create(self.cfg, self.ws_ptr, self.nbytes)
        self._keep = []

    @property
    def batch(self) -> int:
        return self.cfg.batch

    def set_params(self, A, D):
        self._keep = [_f32(A, "A"), _f32(D, "D")]
        rssm_set_params(self.handle, A, D)

    def init_checkpoint(self, state, seq_mask=None, stream=None):
        _f32(state, "state")
        rssm_init_checkpoint(self.handle, state, seq_mask, stream)

    def _inputs(self, ntok, **kw) -> rssm_inputs:
        for name, t in kw.items():
            _f32(t, name)
        return make_inputs(ntok, **kw)

    def decode_step(self, y, stream=None, **kw):
        rssm_decode_step(self.handle, self._inputs(1, **kw), _f32(y, "y"), stream)

    def prefill(self, y, stream=None, **kw):
        """T prompt tokens (token-major inputs, leading dimension T) into the checkpoint."""
        ntok = next(iter(kw.values())).shape[0]
        rssm_prefill(self.handle, self._inputs(ntok, **kw), _f32(y, "y"), stream)

    def verify(self, y, stream=None, **kw):
        ntok = next(iter(kw.values())).shape[0]
        rssm_verify(self.handle, self._inputs(ntok, **kw), _f32(y, "y"), stream)

    def commit(self, accepted, stream=None):
        rssm_verify_commit(self.handle, accepted, stream)

    def rollback(self, new_len, stream=None):
        rssm_rollback(self.handle, new_len, stream)

    def consolidate(self, min_len: int, stream=None):
        rssm_consolidate(self.handle, min_len, stream)

    def seq_state_bytes(self) -> int:
        return rssm_seq_state_bytes(self.cfg)

    def fork(self, src, dst, stream=None):
        """Sequence dst[i] becomes a copy of sequence src[i] (int32 device tensors)."""
        rssm_fork(self.handle, src, dst, src.numel(), stream)

    def export(self, seq, buf, stream=None):
        """Packed state of sequences seq (int32 device tensor) into buf (uint8 device tensor)."""
        rssm_export(self.handle, seq, seq.numel(), buf, stream)

    def import_(self, seq, buf, stream=None):
        rssm_import(self.handle, seq, seq.numel(), buf, stream)

    def materialize(self, out, stream=None):
        rssm_materialize(self.handle, _f32(out, "out"), stream)

    def bookkeeping(self, stream=None):
        return rssm_read_bookkeeping(self.handle, self.cfg.batch, stream)

    def close(self):
        if self.handle:
            rssm_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def step_baseline_spec(cfg: rssm_config, pool, slot_of, y, A=None, D=None, stream=None, **kw):
    """Conventional speculative round over the drafts in kw (leading token axis K): snapshots into
    the slot pool [2K+1, B, H, dim_v, dim_k] from each sequence's committed slot (A and D: Mamba-2
    only)."""
    ntok = next(iter(kw.values())).shape[0]
    rssm_step_baseline_spec(cfg, pool, slot_of, make_inputs(ntok, **kw), A, D, y, stream)


def step_baseline_seqs(cfg: rssm_config, seq_ptrs, y, A=None, D=None, snapshots=None, stream=None,
                       **kw):
    """Conventional decode over per-sequence state tiles (seq_ptrs: [B] int64 device addresses)."""
    ntok = next(iter(kw.values())).shape[0]
    rssm_step_baseline_seqs(cfg, seq_ptrs, make_inputs(ntok, **kw), A, D, y, snapshots, stream)


def step_baseline(cfg: rssm_config, state, y, A=None, D=None, snapshots=None, stream=None, **kw):
    """Conventional read-modify-write decode over the tokens in kw (leading token axis)."""
    ntok = next(iter(kw.values())).shape[0]
    rssm_step_baseline(cfg, state, make_inputs(ntok, **kw), A, D, y, snapshots, stream)
