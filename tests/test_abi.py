"""librssm loads, exports every entry point include/rssm.h declares, and rejects bad arguments and
call-order misuse on the host, before any device work. No GPU needed."""
import ctypes
import os
import re

import pytest

import checkpoint_replay_buffer_amd.binding as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rssm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rb.LIB_PATH):
        from checkpoint_replay_buffer_amd import build
        build.build()
    return rb.load_library()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rssm_[a-z_]+)\s*\(", src)))


def test_exports_match_header(lib):
    names = _declared()
    assert set(names) == set(rb.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in range(0, -7, -1):
        assert rb.status_str(st) not in ("", "unknown status")
    assert rb.status_str(-99) == "unknown status"


def _cfg(**kw):
    base = dict(kind=rb.RSSM_MAMBA2, batch=256, nheads=128, ngroups=128, dim_v=64, dim_k=128,
                window=16, max_draft=6, flags=rb.RSSM_F_STORE_C)
    base.update(kw)
    return rb.make_config(**base)


def _up(v):
    return (v + 255) // 256 * 256


def test_workspace_layout(lib):
    B, H, G, P, N, W = 256, 128, 128, 64, 128, 16
    want = _up(2 * 3 * B * 4) + _up(4) + _up(B * H * P * N * 4) + _up(B * H * W * P * 4) \
        + 2 * _up(B * G * W * N * 4) + _up(B * H * W * 4)
    assert rb.rssm_workspace_bytes(_cfg()) == want
    # bf16 read copy adds B*H*P*N*2; no stored C removes one B/C ring
    assert rb.rssm_workspace_bytes(_cfg(flags=rb.RSSM_F_STORE_C | rb.RSSM_F_BF16_READ)) == \
        want + _up(B * H * P * N * 2)
    assert rb.rssm_workspace_bytes(_cfg(flags=0)) == want - _up(B * G * W * N * 4)


@pytest.mark.parametrize("kw,status", [
    (dict(kind=4), -1),
    (dict(window=0), -2),
    (dict(window=33), -2),
    (dict(max_draft=17), -2),
    (dict(max_draft=-1), -2),
    (dict(ngroups=3), -2),
    (dict(batch=0), -2),
    (dict(flags=8), -1),
    (dict(dim_v=48), -6),
    (dict(dim_k=96), -6),
    (dict(kind=rb.RSSM_GDN, dim_v=128, dim_k=128, ngroups=64), -2),
    (dict(kind=rb.RSSM_GDN, dim_v=128, dim_k=128, flags=rb.RSSM_F_BF16_READ), -6),
    (dict(kind=rb.RSSM_KDA, dim_v=128, dim_k=128, ngroups=64), -2),
    (dict(kind=rb.RSSM_KDA, dim_v=128, dim_k=128, flags=rb.RSSM_F_BF16_READ), -6),
    (dict(kind=rb.RSSM_KDA, dim_v=64, dim_k=128), -6),
    (dict(kind=rb.RSSM_KDA, dim_v=128, dim_k=128, window=32, max_draft=32), -6),   # LDS
])
def test_config_errors(lib, kw, status):
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_workspace_bytes(_cfg(**kw))
    assert e.value.status == status


FAKE_WS = 1 << 40     # an aligned address; creation never dereferences it


def test_create_checks(lib):
    cfg = _cfg()
    n = rb.rssm_workspace_bytes(cfg)
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_create(cfg, FAKE_WS + 16, n)
    assert e.value.status == -1
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_create(cfg, FAKE_WS, n - 1)
    assert e.value.status == -3
    h = rb.rssm_create(cfg, FAKE_WS, n)
    rb.rssm_destroy(h)


def test_call_order_checked_on_host(lib):
    cfg = _cfg(batch=2, nheads=4, ngroups=4, dim_v=16, dim_k=16, window=4, max_draft=2)
    h = rb.rssm_create(cfg, FAKE_WS, rb.rssm_workspace_bytes(cfg))
    try:
        tok = rb.make_inputs(1, x=FAKE_WS, B=FAKE_WS, C=FAKE_WS, dt=FAKE_WS)
        # nothing loaded yet
        for call in (lambda: rb.rssm_decode_step(h, tok, FAKE_WS, stream=0),
                     lambda: rb.rssm_consolidate(h, 1, stream=0),
                     lambda: rb.rssm_verify(h, tok, FAKE_WS, stream=0),
                     lambda: rb.rssm_verify_commit(h, FAKE_WS, stream=0),
                     lambda: rb.rssm_rollback(h, FAKE_WS, stream=0),
                     lambda: rb.rssm_materialize(h, FAKE_WS, stream=0),
                     lambda: rb.rssm_prefill(h, tok, FAKE_WS, stream=0),
                     lambda: rb.rssm_fork(h, FAKE_WS, FAKE_WS, 1, stream=0),
                     lambda: rb.rssm_export(h, FAKE_WS, 1, FAKE_WS, stream=0),
                     lambda: rb.rssm_import(h, FAKE_WS, 1, FAKE_WS, stream=0),
                     lambda: rb.rssm_init_checkpoint(h, FAKE_WS, FAKE_WS, stream=0)):
            with pytest.raises(rb.RssmError) as e:
                call()
            assert e.value.status == -4
        # null / misaligned arguments
        with pytest.raises(rb.RssmError) as e:
            rb.rssm_init_checkpoint(h, FAKE_WS + 4, None, stream=0)
        assert e.value.status == -1
        with pytest.raises(rb.RssmError) as e:
            rb.rssm_set_params(h, None, FAKE_WS)
        assert e.value.status == -1
    finally:
        rb.rssm_destroy(h)


def test_baseline_argument_checks(lib):
    cfg = _cfg(batch=2, nheads=4, ngroups=4, dim_v=16, dim_k=16, window=4, max_draft=0)
    bad = rb.make_inputs(1, x=FAKE_WS + 8, B=FAKE_WS, C=FAKE_WS, dt=FAKE_WS)
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_step_baseline(cfg, FAKE_WS, bad, FAKE_WS, FAKE_WS, FAKE_WS, stream=0)
    assert e.value.status == -1
    zero = rb.make_inputs(0, x=FAKE_WS, B=FAKE_WS, C=FAKE_WS, dt=FAKE_WS)
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_step_baseline(cfg, FAKE_WS, zero, FAKE_WS, FAKE_WS, FAKE_WS, stream=0)
    assert e.value.status == -1
    with pytest.raises(rb.RssmError) as e:
        rb.rssm_step_baseline(cfg, FAKE_WS, rb.make_inputs(1, x=FAKE_WS, B=FAKE_WS, C=FAKE_WS,
                                                           dt=FAKE_WS),
                              None, FAKE_WS, FAKE_WS, stream=0)
    assert e.value.status == -1


@pytest.mark.parametrize("kind,flags,dims", [
    (rb.RSSM_MAMBA2, 0, (3, 4, 2, 16, 16, 5)),
    (rb.RSSM_MAMBA2, rb.RSSM_F_BF16_READ | rb.RSSM_F_STORE_C, (2, 128, 128, 64, 128, 16)),
    (rb.RSSM_GDN, 0, (2, 3, 3, 64, 64, 7)),
    (rb.RSSM_KDA, 0, (2, 3, 3, 64, 64, 7)),
])
def test_seq_state_bytes(lib, kind, flags, dims):
    """A packed sequence slot: a 16-byte header (head, len, ndraft) and each state array's share of
    one sequence, padded to 16 bytes, in the order checkpoint, read copy, ring arrays."""
    B, H, G, V, K, W = dims
    cfg = rb.make_config(kind, B, H, G, V, K, W, 0, flags)
    pad = lambda n: (n + 15) // 16 * 16
    segs = [H * V * K * 4]
    if flags & rb.RSSM_F_BF16_READ:
        segs.append(H * V * K * 2)
    if kind == rb.RSSM_MAMBA2:
        segs += [H * W * V * 4, G * W * K * 4]
        if flags & rb.RSSM_F_STORE_C:
            segs.append(G * W * K * 4)
        segs.append(H * W * 4)
    else:
        gate = K if kind == rb.RSSM_KDA else 1          # Kimi Delta Attention: a gate per key channel
        segs += [H * W * K * 4, H * W * V * 4, H * W * 4, H * W * gate * 4]
    assert rb.rssm_seq_state_bytes(cfg) == 16 + sum(pad(n) for n in segs)


def test_kda_workspace_and_prefill(lib):
    """Kimi Delta Attention rings: k, v, beta and a gate row of d_k per entry; prefill before any
    checkpoint is loaded is a state error."""
    B, H, V, K, W = 4, 3, 64, 64, 8
    cfg = rb.make_config(rb.RSSM_KDA, B, H, H, V, K, W, 4, 0)
    want = _up(2 * 3 * B * 4) + _up(4) + _up(B * H * V * K * 4) + _up(B * H * W * K * 4) \
        + _up(B * H * W * V * 4) + _up(B * H * W * 4) + _up(B * H * W * K * 4)
    n = rb.rssm_workspace_bytes(cfg)
    assert n == want
    h = rb.rssm_create(cfg, FAKE_WS, n)
    try:
        tok = rb.make_inputs(3, q=FAKE_WS, k=FAKE_WS, v=FAKE_WS, beta=FAKE_WS, alpha=FAKE_WS)
        with pytest.raises(rb.RssmError) as e:
            rb.rssm_prefill(h, tok, FAKE_WS, stream=0)
        assert e.value.status == -4             # nothing loaded yet
    finally:
        rb.rssm_destroy(h)
