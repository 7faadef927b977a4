"""Pins of the oracle's precision tools to facts other than themselves: the bf16 rounding used for
the read copy (round to nearest, ties to even, decided by exact rational comparison), the fp32
instantiation of the conventional Mamba-2 step (exact where fp32 arithmetic is exact, within the
worst-case rounding bound elsewhere), and the conditioning recurrences that scale the rounding
bounds of the GPU criteria."""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl
from oracle import (C_FP32, U32, cond_check, gdn_kappa_step, gdn_step, m2_kappa_step, m2_step,
                    m2_step_f32, normwise_err, round_bf16)


# ------------------------------------------------------------------------ bf16 read-copy rounding

def _bits(u32):
    return np.array([u32], dtype=np.uint32).view(np.float32)


def _bf16_exact(f32_bits: int) -> float:
    """Nearest bf16 value (8 significant bits) to a finite fp32 value, by exact rational distance;
    on a tie the candidate whose last significand bit is 0. Candidates: the fp32 value truncated
    to its upper 16 bits and the next bf16 value away from zero."""
    x = Fraction(float(_bits(f32_bits)[0]))
    lo_bits = f32_bits & 0xFFFF0000
    hi_bits = lo_bits + 0x10000
    lo = Fraction(float(_bits(lo_bits)[0]))
    hi = Fraction(float(_bits(hi_bits)[0])) if (hi_bits & 0x7F800000) != 0x7F800000 else None
    if hi is None or abs(x - lo) < abs(hi - x):
        return float(lo)
    if abs(x - lo) > abs(hi - x):
        return float(hi)
    return float(lo) if ((lo_bits >> 16) & 1) == 0 else float(hi)


@pytest.mark.parametrize("bits,expect", [
    (0x3F808000, 0x3F800000),   # 1 + 2^-8: halfway between 1 and 1 + 2^-7, tie to even (down)
    (0x3F818000, 0x3F820000),   # halfway above an odd significand: tie to even (up)
    (0x3F808001, 0x3F810000),   # just above halfway: up
    (0x3F807FFF, 0x3F800000),   # just below halfway: down
    (0x3FFF8000, 0x40000000),   # tie above an odd all-ones significand: carry into the exponent
    (0x3FFF7FFF, 0x3FFF0000),   # just below that tie: no carry
    (0xBF808000, 0xBF800000),   # negative tie: to even, magnitude down
    (0xBF818000, 0xBF820000),   # negative tie: to even, magnitude up
    (0x00008000, 0x00000000),   # subnormal tie at zero: even
    (0x00018000, 0x00020000),   # subnormal tie above an odd significand
    (0x007F8000, 0x00800000),   # largest subnormals round up into the smallest normal
    (0x7F7F7FFF, 0x7F7F0000),   # near the largest finite value, below the tie: stays finite
])
def test_round_bf16_ties_and_carries(bits, expect):
    got = round_bf16(_bits(bits))[0]
    assert got == float(_bits(expect)[0])
    assert got == _bf16_exact(bits)


def test_round_bf16_matches_exact_nearest_even():
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force a quarter of them onto exact ties (lower 16 bits = 0x8000)
    raw[: raw.size // 4] = (raw[: raw.size // 4] & 0xFFFF0000) | 0x8000
    raw = raw[(raw & 0x7F800000) != 0x7F800000]               # finite values only
    raw = raw[(raw & 0x7FFFFFFF) < 0x7F7F8000]                # that do not round past the range
    got = round_bf16(raw.view(np.float32))
    want = np.array([_bf16_exact(int(b)) for b in raw])
    assert np.array_equal(got, want)
    # every result is a bf16 value: its lower 16 fp32 bits are zero
    assert np.all((got.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)


# ------------------------------------------------------------------ fp32 conventional Mamba-2 step

def test_m2_f32_exact_where_fp32_is_exact(oracle_lib):
    """A = 0 (decay exp(0) = 1 exactly), dt = 1/2 and small dyadic inputs: every product and sum is
    exact in fp32, so the fp32 step equals the fp64 definition bit for bit over many tokens. A
    dropped or misplaced term, a wrong index or group map would show."""
    rng = np.random.default_rng(1)
    B, H, G, P, N, T = 2, 4, 2, 5, 6, 9
    A = np.zeros(H, np.float32)
    D = (rng.integers(-4, 5, size=H) / 4).astype(np.float32)
    s64 = (rng.integers(-8, 9, size=(B, H, P, N)) / 8).astype(np.float64)
    s32 = s64.astype(np.float32)
    for t in range(T):
        x = (rng.integers(-4, 5, size=(B, H, P)) / 2).astype(np.float32)
        Bm = (rng.integers(-4, 5, size=(B, G, N)) / 4).astype(np.float32)
        C = (rng.integers(-4, 5, size=(B, G, N)) / 4).astype(np.float32)
        dt = np.full((B, H), 0.5, np.float32)
        y64 = m2_step(A, D, x, Bm, C, dt, s64)
        y32 = m2_step_f32(A, D, x, Bm, C, dt, s32)
        assert np.array_equal(y32.astype(np.float64), y64), t
        assert np.array_equal(s32.astype(np.float64), s64), t


def test_m2_f32_within_worst_case_bound(oracle_lib):
    """Random workload inputs over T tokens: every fp32 output is within the worst-case a priori
    bound gamma_L kappa of the fp64 definition, L = 14 T + N + 6 (per token at most 12 unit
    roundoffs in the decay exp(dt A) with |dt A| < 10, one for its product and one for the sum;
    N + 1 for the output sum and its terms), gamma_L = L u / (1 - L u). The fp32 recurrence is
    the same computation as the fp64 one."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=2, head_dim=8, d_state=16, window=4)
    prm = wl.m2_params(sh, 3)
    s0 = wl.m2_state0(sh, 3)
    T = 24
    ins = wl.m2_token_inputs(sh, 3, 0, ntok=T)
    assert np.max(np.abs(ins["dt"] * prm["A"][None, None, :])) < 10
    s64 = s0.astype(np.float64)
    s32 = s0.copy()
    M = np.abs(s0).astype(np.float64)
    L = 14 * T + sh.d_state + 6
    gam = L * U32 / (1 - L * U32)
    worst = 0.0
    for t in range(T):
        a = [ins[k][t] for k in ("x", "B", "C", "dt")]
        y64 = m2_step(prm["A"], prm["D"], *a, s64)
        y32 = m2_step_f32(prm["A"], prm["D"], *a, s32)
        kap = m2_kappa_step(prm["A"], prm["D"], *a, M)
        r = np.max(np.abs(y32 - y64) / (gam * kap))
        worst = max(worst, r)
        assert r <= 1.0, t
    assert worst > 0       # the fp32 step does round


def test_m2_kappa_is_the_output_for_nonnegative_inputs(oracle_lib):
    """With non-negative x, B, C, D and initial state, every term of the recurrence is already
    non-negative, so kappa equals the output itself, token after token; with signed inputs it
    bounds |y| from above."""
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=4, head_dim=6, d_state=8, window=4)
    prm = wl.m2_params(sh, 4)
    s0 = np.abs(wl.m2_state0(sh, 4))
    ins = wl.m2_token_inputs(sh, 4, 0, ntok=10)
    pos = {k: np.abs(v) for k, v in ins.items()}
    Dp = np.abs(prm["D"])
    st = s0.astype(np.float64)
    M = s0.astype(np.float64)
    for t in range(10):
        a = [pos[k][t] for k in ("x", "B", "C", "dt")]
        y = m2_step(prm["A"], Dp, *a, st)
        kap = m2_kappa_step(prm["A"], prm["D"], *a, M)    # |D| inside
        assert np.array_equal(y, kap), t
        assert np.array_equal(st, M), t
    st = wl.m2_state0(sh, 4).astype(np.float64)
    M = np.abs(st)
    for t in range(10):
        a = [ins[k][t] for k in ("x", "B", "C", "dt")]
        y = m2_step(prm["A"], prm["D"], *a, st)
        kap = m2_kappa_step(prm["A"], prm["D"], *a, M)
        assert np.all(np.abs(y) <= kap * (1 + 1e-12)), t


def test_gdn_kappa_pins(oracle_lib):
    """beta = 0 leaves the pure decay: with non-negative state and query kappa equals the output
    exactly. A unit key e_i with beta = alpha = 1 adds, in row r, s_r = M[r][i] and |v_r| to
    column i only (M[r][i] -> 2 M[r][i] + |v_r|). With signed inputs kappa bounds |o|."""
    rng = np.random.default_rng(2)
    B, H, d = 1, 2, 4
    S = np.abs(rng.standard_normal((B, H, d, d)))
    q = np.abs(rng.standard_normal((B, H, d))).astype(np.float32)
    k = rng.standard_normal((B, H, d)).astype(np.float32)
    v = rng.standard_normal((B, H, d)).astype(np.float32)
    al = np.full((B, H), 0.75, np.float32)
    st, M = S.copy(), S.copy()
    o = gdn_step(q, k, v, np.zeros((B, H), np.float32), al, st)
    kap = gdn_kappa_step(q, k, v, np.zeros((B, H), np.float32), al, M)
    assert np.array_equal(o, kap) and np.array_equal(st, M)
    M = S.copy()
    e = np.zeros((B, H, d), np.float32)
    e[..., 2] = 1.0
    one = np.ones((B, H), np.float32)
    gdn_kappa_step(q, e, v, one, one, M)
    want = S.copy()
    want[..., :, 2] = 2 * S[..., :, 2] + np.abs(v.astype(np.float64))
    assert np.array_equal(M, want)
    sh = wl.GDNShape(batch=2, nheads=3, d_k=8, d_v=8, window=4)
    s0 = wl.gdn_state0(sh, 1).astype(np.float64)
    ins = wl.gdn_token_inputs(sh, 1, 0, ntok=12)
    M = np.abs(s0)
    for t in range(12):
        a = [ins[kk][t] for kk in ("q", "k", "v", "beta", "alpha")]
        o = gdn_step(*a, s0)
        kap = gdn_kappa_step(*a, M)
        assert np.all(np.abs(o) <= kap * (1 + 1e-12)), t


def test_fp32_conventional_misses_1e5_on_a_near_cancelling_head(oracle_lib):
    """Conventional decoding in fp32 is itself not within 1e-5 normwise of the exact recurrence
    on a head whose output nearly cancels. The 64-token prompt of the Mamba-2 serving-shape
    prefill test (seed 0, slot 100; batch 256, 128 heads, 64 x 128): at token 25, sequence 17,
    head 12 has max|y| = 6.2e-4 against a conditioning kappa over a thousand times larger; the
    fp32 recurrence misses 1e-5 there, and stays within the fp32 rounding bound C_FP32 u kappa
    (as on every other head of that sequence)."""
    sh = wl.M2_SERVE
    prm = wl.m2_params(sh, 0)
    T = 26
    ins = wl.m2_token_inputs(sh, 0, 100, ntok=T)          # the first 26 tokens of the prompt
    b = 17
    s0 = wl.m2_state0(sh, 0)[b:b + 1]
    s64 = s0.astype(np.float64)
    s32 = s0.copy()
    M = np.abs(s0).astype(np.float64)
    for t in range(T):
        a = [ins[k][t][b:b + 1] for k in ("x", "B", "C", "dt")]
        y64 = m2_step(prm["A"], prm["D"], *a, s64)
        y32 = m2_step_f32(prm["A"], prm["D"], *a, s32)
        kap = m2_kappa_step(prm["A"], prm["D"], *a, M)
        c = cond_check(y32, y64, C_FP32 * U32 * kap, 1e-5)
        assert c.ok and c.ratio_all <= 1.0, (t, c)
    head = (0, 12)
    assert np.max(np.abs(y64[head])) < 1e-3
    assert np.max(kap[head]) > 1000 * np.max(np.abs(y64[head]))
    assert normwise_err(y32[head], y64[head]) > 1e-5


def test_torch_kappa_helpers_match_the_oracle(oracle_lib):
    """The device-side conditioning used for full-batch GPU-vs-GPU checks (plain PyTorch, here on
    the CPU) equals the oracle's to fp32 rounding: all its terms are non-negative."""
    import torch
    from tests.gpu_helpers import gdn_kappa_torch, m2_kappa_torch
    sh = wl.M2Shape(batch=2, nheads=4, ngroups=2, head_dim=8, d_state=16, window=4)
    prm = wl.m2_params(sh, 6)
    s0 = wl.m2_state0(sh, 6)
    ins = wl.m2_token_inputs(sh, 6, 0, ntok=12)
    M = np.abs(s0).astype(np.float64)
    Mt = torch.from_numpy(np.abs(s0))
    A, D = torch.from_numpy(prm["A"]), torch.from_numpy(prm["D"])
    for t in range(12):
        a = [ins[k][t] for k in ("x", "B", "C", "dt")]
        k64 = m2_kappa_step(prm["A"], prm["D"], *a, M)
        k32 = m2_kappa_torch(Mt, A, D, *[torch.from_numpy(v) for v in a]).numpy()
        assert np.max(np.abs(k32 - k64) / k64) < 1e-5, t
    gs = wl.GDNShape(batch=2, nheads=3, d_k=16, d_v=8, window=4)
    g0 = wl.gdn_state0(gs, 6)
    gin = wl.gdn_token_inputs(gs, 6, 0, ntok=12)
    M = np.abs(g0).astype(np.float64)
    Mt = torch.from_numpy(np.abs(g0))
    for t in range(12):
        a = [gin[k][t] for k in ("q", "k", "v", "beta", "alpha")]
        k64 = gdn_kappa_step(*a, M)
        k32 = gdn_kappa_torch(Mt, *[torch.from_numpy(v) for v in a]).numpy()
        assert np.max(np.abs(k32 - k64) / k64) < 1e-5, t


def test_torch_kda_kappa_helper_matches_the_oracle(oracle_lib):
    import torch
    from oracle import kda_kappa_step
    from tests.gpu_helpers import kda_kappa_torch
    gs = wl.GDNShape(batch=2, nheads=3, d_k=16, d_v=8, window=4)
    g0 = wl.kda_state0(gs, 6)
    gin = wl.kda_token_inputs(gs, 6, 0, ntok=12)
    M = np.abs(g0).astype(np.float64)
    Mt = torch.from_numpy(np.abs(g0))
    for t in range(12):
        a = [gin[k][t] for k in ("q", "k", "v", "beta", "alpha")]
        k64 = kda_kappa_step(*a, M)
        k32 = kda_kappa_torch(Mt, *[torch.from_numpy(v) for v in a]).numpy()
        assert np.max(np.abs(k32 - k64) / k64) < 1e-5, t
