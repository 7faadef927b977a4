#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode hot path on one MI355X.

Default workload: Mamba-2 decode of one SSM layer at serving shape -- batch 256, 128 heads,
head_dim 64, d_state 128 (4 MiB fp32 state per sequence, 1 GiB per layer), ring W = 16, fp32
state. One step = one decode token for every sequence (one rssm_decode_step launch, the fold of
a full ring included in the launch that fills it). Inputs come from a pool of 32 pre-generated
seeded token slots (step t uses slot t mod 32) resident in HBM before timing starts.

Printed: one JSON line. `value` is the algorithmic HBM traffic of the replay decode per second
(GB/s), the bytes the method must move (checkpoint reads, the fold's read+write, ring reads and
appends, inputs, outputs) divided by the timed wall time. Also reported: SSM-layer tokens/s, the
speedup over the conventional read-modify-write kernel on the same input schedule, the roofline
of the dominant kernel, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (1e9 bytes)
METRIC = "SSM decode state GB/s (% of HBM peak) + tokens/s vs conventional, batch 256 W=16"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "checkpoint_replay_buffer_amd", "csrc", "mamba2.hip")


# ------------------------------------------------------------------------------------------
# algorithmic byte model (per (sequence, head) pair and per launch)
# ------------------------------------------------------------------------------------------

def m2_replay_bytes(P, N, W, gr, length, store_c=True, bf16=False) -> float:
    """HBM bytes one decode launch must move for one (b, h) pair whose ring holds `length`
    committed entries before the token. gr = G / H (B and C rows are shared by a group)."""
    f = 4
    inputs = (P + 1) * f + 2 * N * f * gr          # x, dt, B, C of the token
    ring_rd = length * ((P + 1) * f + N * f * gr)  # x, dt, B of the buffered entries
    y = P * f
    if length + 1 >= W:                            # the token fills the ring: fold
        s0 = 2 * P * N * f + (P * N * 2 if bf16 else 0)
        return s0 + inputs + ring_rd + y
    s0 = P * N * (2 if bf16 else f)
    append = (P + 1) * f + N * f * gr * (2 if store_c else 1)
    return s0 + inputs + ring_rd + append + y


def m2_rmw_bytes(P, N, gr) -> float:
    f = 4
    return 2 * P * N * f + (P + 1) * f + 2 * N * f * gr + P * f


# ------------------------------------------------------------------------------------------

def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _repeat_ms(torch, first_ms, reps, restart, step, K):
    """The timed region repeated: `first_ms` is the first run; each further run restarts the
    context (`restart`, untimed) and times the same K steps. Returns median, min and max of the
    runs in ms per step."""
    runs = [first_ms]
    for _ in range(reps - 1):
        restart()
        torch.cuda.synchronize()
        ev = _events(torch, 2)
        ev[0].record()
        for t in range(K):
            step(t)
        ev[1].record()
        torch.cuda.synchronize()
        runs.append(ev[0].elapsed_time(ev[1]))
    per = sorted(r / K for r in runs)
    return {"n": len(runs), "median": round(per[len(per) // 2], 5), "min": round(per[0], 5),
            "max": round(per[-1], 5)}


def measure_copy_gbs(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate on this machine ((read + write) bytes / time): the practical ceiling
    the HBM-bound legs are also quoted against."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms / 1e3) / 1e9


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _src_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(os.path.dirname(KERNEL_SRC), f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_fields(kernel_key: str) -> dict:
    """The measured HBM bytes per launch of a kernel (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
    plain copy's counters) beside the byte model of the same profiled launches and their ratio.
    The profiled launches follow their own schedule, so `traffic` is compared with
    `traffic_alg_bytes_per_launch`, not with this run's `alg_bytes_per_launch`. None when the
    counters were taken on other kernel sources."""
    try:
        t = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        t = {}
    e = t.get(kernel_key)
    if not e or e.get("src_hash") != _src_hash(e.get("files", ())):
        return {"traffic": None}
    out = {"traffic": e.get("bytes_per_launch"),
           "traffic_alg_bytes_per_launch": e.get("alg_bytes_per_launch")}
    if out["traffic"] and out["traffic_alg_bytes_per_launch"]:
        out["traffic_ratio"] = round(out["traffic"] / out["traffic_alg_bytes_per_launch"], 4)
    return out


def _graph_time(torch, nsteps, step, reps_warm, reps):
    """Capture `nsteps` consecutive calls step(t) into one HIP graph (torch's capture stream; the
    library launches on torch's current stream), replay it reps_warm times, then time `reps`
    replays between two events. Returns the timed milliseconds."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for t in range(nsteps):
            step(t)
    for _ in range(reps_warm):
        g.replay()
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for _ in range(reps):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    del g
    return ms


def run_m2(args, torch, rb, wl):
    """Mamba-2 decode at the serving shape. Lock-step (default): every sequence starts from an
    empty ring, so all of them fold in the same launch, one launch in W. --stagger: W - 1 tokens and
    a rollback of sequence b to b mod W entries before every timed pass (untimed), so every
    sequence sits at its own ring position and every timed launch mixes tiles that fold (1 / W of
    them) with tiles that replay, the state continuous batching and speculative commits leave."""
    bf16 = args.workload == "m2_serve_bf16"
    batch = args.batch or 256
    sh = wl.M2Shape(batch=batch, nheads=128, ngroups=args.groups or 128, head_dim=64, d_state=128,
                    window=16)
    P, N, W, H, B = sh.head_dim, sh.d_state, sh.window, sh.nheads, sh.batch
    gr = sh.ngroups / sh.nheads
    pool_n = 32
    t0 = time.time()
    prm = wl.m2_params(sh, 0)
    s0 = torch.from_numpy(wl.m2_state0(sh, 0)).cuda()
    host_pool, pool = [], []
    for s in range(pool_n):
        ins = wl.m2_token_inputs(sh, 0, s)
        host_pool.append({k: v[0] for k, v in ins.items()})
        pool.append({k: torch.from_numpy(v[0]).cuda() for k, v in ins.items()})
    A = torch.from_numpy(prm["A"]).cuda()
    D = torch.from_numpy(prm["D"]).cuda()
    gen_s = time.time() - t0

    ctx = rb.Context("mamba2", B, H, P, N, W, ngroups=sh.ngroups, bf16_read=bf16, store_c=True)
    ctx.set_params(A, D)
    y = torch.empty(B, H, P, device="cuda")
    K, Wm = args.steps, args.warmup
    # lock-step: the timed steps start at ring fill `pre`, so that K steps hold ceil(K / W) folds
    # (never fewer than the steady state's K / W when K is not a multiple of W)
    pre = 0 if args.stagger or args.graph else (W - K % W) % W
    start_len = np.arange(B) % W if args.stagger else np.full(B, pre, dtype=np.int64)
    new_len = torch.from_numpy(start_len.astype(np.int32)).cuda()

    def restart():
        """Back to the checkpoint; then (untimed) to ring fill b mod W with --stagger, or to the
        common fill `pre`."""
        ctx.init_checkpoint(s0)
        if args.stagger:
            for t in range(W - 1):
                ctx.decode_step(y, **pool[(pool_n - 1 - t) % pool_n])
            ctx.rollback(new_len)
        else:
            for t in range(pre):
                ctx.decode_step(y, **pool[(pool_n - 1 - t) % pool_n])

    # warm-up, then restart so the timed steps see the schedule from its start
    restart()
    for t in range(Wm):
        ctx.decode_step(y, **pool[t % pool_n])
    restart()
    torch.cuda.synchronize()

    # timed region: K steps bracketed by events only (wall time of the whole job)
    reps = None
    if not args.graph:
        ev = _events(torch, 2)
        ev[0].record()
        for t in range(K):
            ctx.decode_step(y, **pool[t % pool_n])
        ev[1].record()
        torch.cuda.synchronize()
        total_ms = ev[0].elapsed_time(ev[1])
        h, l, n, e = ctx.bookkeeping()
        assert e == 0 and list(l) == [int(v) for v in (start_len + K) % W], \
            "unexpected bookkeeping after the timed steps"
        reps = _repeat_ms(torch, total_ms, args.reps, restart,
                          lambda t: ctx.decode_step(y, **pool[t % pool_n]), K)

    # the same K steps again with an event pair around every launch (per-kernel durations on the
    # stream the kernels run on)
    restart()
    torch.cuda.synchronize()
    evl = _events(torch, 2 * K)
    for t in range(K):
        evl[2 * t].record()
        ctx.decode_step(y, **pool[t % pool_n])
        evl[2 * t + 1].record()
    torch.cuda.synchronize()
    launch_ms = [evl[2 * t].elapsed_time(evl[2 * t + 1]) for t in range(K)]

    if args.graph:
        # the timed steps as replays of one captured window of pool_n = 2 W decode steps from an
        # empty ring (the window ends where it started: same ring position, same bookkeeping buffer)
        ctx.init_checkpoint(s0)
        total_ms = _graph_time(torch, pool_n, lambda t: ctx.decode_step(y, **pool[t]), 1,
                               K // pool_n)
        h, l, n, e = ctx.bookkeeping()
        assert e == 0 and l[0] == 0, "unexpected bookkeeping after the graph replays"

    # algorithmic bytes of every launch: sequence b holds (start_len[b] + t) mod W entries at
    # step t; the state-only part is the checkpoint read (and, when folding, its write)
    def launch_bytes(t):
        ls = (start_len + t) % W
        counts = np.bincount(ls, minlength=W)
        alg = sum(int(c) * m2_replay_bytes(P, N, W, gr, l, True, bf16) for l, c in enumerate(counts))
        st = sum(int(c) * (2 * P * N * 4 + (P * N * 2 if bf16 else 0) if l == W - 1
                           else P * N * (2 if bf16 else 4)) for l, c in enumerate(counts))
        return alg * H, st * H
    per = [launch_bytes(t) for t in range(K)]
    alg_bytes = sum(p[0] for p in per)
    state_bytes = sum(p[1] for p in per)
    replay_s = total_ms / 1e3

    # conventional read-modify-write on the same schedule
    rmw_s = None
    if not args.no_rmw:
        cfg = rb.make_config(rb.RSSM_MAMBA2, B, H, sh.ngroups, P, N, W)
        st = s0.clone()
        y1 = torch.empty(1, B, H, P, device="cuda")
        pool1 = [{k: v.unsqueeze(0) for k, v in pool[t].items()} for t in range(pool_n)]
        for t in range(Wm):
            rb.step_baseline(cfg, st, y1, A, D, **pool1[t % pool_n])
        st.copy_(s0)
        torch.cuda.synchronize()
        if args.graph:
            rmw_s = _graph_time(torch, pool_n, lambda t: rb.step_baseline(cfg, st, y1, A, D, **pool1[t]),
                                1, K // pool_n) / 1e3
        else:
            ev2 = _events(torch, 2)
            ev2[0].record()
            for t in range(K):
                rb.step_baseline(cfg, st, y1, A, D, **pool1[t % pool_n])
            ev2[1].record()
            torch.cuda.synchronize()
            rmw_s = ev2[0].elapsed_time(ev2[1]) / 1e3
        del st

    # dominant kernel. Lock-step: the replay-only launches (no sequence folds); the launches whose
    # token fills every ring run the folding variant and are reported beside it. Staggered: every
    # launch is the variant that may fold, with a mix of folding and replaying tiles.
    if args.stagger:
        rep, fol = list(range(K)), []
        kname = f"k_m2_decode<64,128,{'true' if bf16 else 'false'},kMayFold> (mixed: 1/{W} of the tiles fold)"
        tkey = "decode_stagger_bf16" if bf16 else "decode_stagger"
    else:
        rep = [t for t in range(K) if (pre + t) % W != W - 1]
        fol = [t for t in range(K) if (pre + t) % W == W - 1]
        kname = f"k_m2_decode<64,128,{'true' if bf16 else 'false'},kUniform> (steps that replay)"
        tkey = "decode_replay_bf16" if bf16 else "decode_replay"
    rep_bytes = sum(per[t][0] for t in rep)
    fol_bytes = sum(per[t][0] for t in fol)
    rep_s = sum(launch_ms[t] for t in rep) / 1e3
    fol_s = sum(launch_ms[t] for t in fol) / 1e3
    achieved = rep_bytes / rep_s / 1e9
    roof = {
        "bound": "hbm",
        "kernel": kname,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "alg_bytes_per_launch": round(rep_bytes / len(rep)),
        "avg_launch_us": round(1e6 * rep_s / len(rep), 2),
        "launches": len(rep),
    }
    roof.update(_traffic_fields(tkey))
    line = {
        "metric": METRIC,
        "value": round(alg_bytes / replay_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-read/fp32" if bf16 else "fp32",
        "data": "synthetic (seeded N(0,1) x, N(0,1)/sqrt(N) B and C, softplus(N(-2,0.5)) dt)",
        "config": {"workload": f"mamba2_decode_b{B}_h{H}_p{P}_n{N}_w{W}"
                               + (f"_g{sh.ngroups}" if sh.ngroups != H else "") + ("_bf16read" if bf16 else "")
                               + ("_stagger" if args.stagger else "") + ("_graph" if args.graph else ""),
                   "batch": B, "heads": H, "head_dim": P, "d_state": N, "window": W,
                   "groups": sh.ngroups, "input_pool_slots": pool_n,
                   "ring_fill": "staggered: sequence b starts at b mod W entries" if args.stagger
                   else f"lock-step: every sequence starts at {pre} entries "
                        f"({sum(1 for t in range(K) if (pre + t) % W == W - 1)} folding steps in {K})",
                   "launch": "hip graph of 2 W steps, replayed" if args.graph else "eager"},
        "value_is": "alg_gbs: every byte the method moves per step (checkpoint reads, the fold's "
                    "read + write, ring reads and appends, inputs, outputs) / wall time",
        "alg_gbs": round(alg_bytes / replay_s / 1e9, 1),
        "state_gbs": round(state_bytes / replay_s / 1e9, 1),
        "state_gbs_is": "checkpoint bytes only (its reads, and the fold's write) / wall time",
        "pct_hbm_peak": round(100 * alg_bytes / replay_s / 1e9 / HBM_PEAK_GBS, 2),
        "ms_per_step_reps": reps,
        "tokens_per_s": round(B * K / replay_s, 1),
        "rmw_ms_per_step": round(rmw_s * 1e3 / K, 5) if rmw_s else None,
        "rmw_gbs": round(m2_rmw_bytes(P, N, gr) * B * H * K / rmw_s / 1e9, 1) if rmw_s else None,
        "speedup_vs_rmw": round(rmw_s / replay_s, 3) if rmw_s else None,
        "roofline": roof,
        "decode_all_launches_gbs": round(alg_bytes / (sum(launch_ms) / 1e3) / 1e9, 1),
        "input_gen_s": round(gen_s, 1),
    }
    if fol:
        line["fold_steps"] = {
            "kernel": f"k_m2_decode<64,128,{'true' if bf16 else 'false'},kAllFold> (the step that fills every ring)",
            "achieved_gbs": round(fol_bytes / fol_s / 1e9, 1),
            "alg_bytes_per_launch": round(fol_bytes / len(fol)),
            "avg_launch_us": round(1e6 * fol_s / len(fol), 2),
            "launches": len(fol),
            **_traffic_fields("decode_fold_bf16" if bf16 else "decode_fold"),
        }
    return line, (sh, prm, host_pool)


def m2_verify_bytes(P, N, W, gr, K, length, store_c=True) -> tuple[float, bool]:
    """HBM bytes of one verify for one (b, h) pair with `length` committed entries, and whether it
    folds them first (length + K > W). With B / C shared by groups (gr < 1) that fold is a
    consolidation launch of its own, after which the verify reads the new checkpoint again."""
    f = 4
    drafts = K * ((P + 1) * f + 2 * N * f * gr)
    ring = length * ((P + 1) * f + N * f * gr)
    outs = K * P * f
    append = K * ((P + 1) * f + N * f * gr * (2 if store_c else 1))
    fold = length + K > W
    s0 = ((3 if gr < 1 else 2) if fold else 1) * P * N * f
    return s0 + ring + drafts + outs + append, fold


def run_m2_spec(args, torch, rb, wl):
    """Speculative decoding: K = 6 drafts per round into the W = 16 ring, verify (outputs of all
    drafts, checkpoint streamed once) then a pointer commit of the seeded accepted prefix, against
    the conventional round (state read once, one snapshot written per draft, pointer commit)."""
    sh = wl.M2_SPEC if not args.groups else wl.M2Shape(batch=512, nheads=128, ngroups=args.groups,
                                                       head_dim=64, d_state=128, window=16, max_draft=6)
    P, N, W, H, B, K = sh.head_dim, sh.d_state, sh.window, sh.nheads, sh.batch, sh.max_draft
    gr = sh.ngroups / sh.nheads
    rounds, Wm, S = args.steps or 256, args.warmup, 4
    t0 = time.time()
    prm = wl.m2_params(sh, 0)
    s0 = torch.from_numpy(wl.m2_state0(sh, 0)).cuda()
    pool = []
    for s in range(S):
        ins = wl.m2_token_inputs(sh, 0, s, ntok=K)
        pool.append({k: torch.from_numpy(v).cuda() for k, v in ins.items()})
    acc_h = wl.spec_accepted(B, rounds + Wm, K, p=0.35, seed=0)
    acc = torch.from_numpy(acc_h).cuda()
    A = torch.from_numpy(prm["A"]).cuda()
    D = torch.from_numpy(prm["D"]).cuda()
    gen_s = time.time() - t0

    ctx = rb.Context("mamba2", B, H, P, N, W, ngroups=sh.ngroups, max_draft=K, store_c=True)
    ctx.set_params(A, D)
    yk = torch.empty(K, B, H, P, device="cuda")
    ctx.init_checkpoint(s0)
    for r in range(Wm):
        ctx.verify(yk, **pool[r % S])
        ctx.commit(acc[rounds + r])
    ctx.init_checkpoint(s0)
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for r in range(rounds):
        ctx.verify(yk, **pool[r % S])
        ctx.commit(acc[r])
    ev[1].record()
    torch.cuda.synchronize()
    replay_s = ev[0].elapsed_time(ev[1]) / 1e3
    h, l, n, e = ctx.bookkeeping()
    assert e == 0
    # per-launch durations of the verify kernel (second pass)
    ctx.init_checkpoint(s0)
    torch.cuda.synchronize()
    evl = _events(torch, 2 * rounds)
    for r in range(rounds):
        evl[2 * r].record()
        ctx.verify(yk, **pool[r % S])
        evl[2 * r + 1].record()
        ctx.commit(acc[r])
    torch.cuda.synchronize()
    verify_ms = [evl[2 * r].elapsed_time(evl[2 * r + 1]) for r in range(rounds)]
    del ctx

    # exact algorithmic bytes from the ring lengths the rounds produce
    L = np.zeros(B, dtype=np.int64)
    vbytes, folds = 0.0, 0
    for r in range(rounds):
        per = [m2_verify_bytes(P, N, W, gr, int(x), K) for x in L]
        vbytes += sum(p[0] for p in per) * H
        fold = L + K > W
        folds += int(fold.sum())
        L = np.where(fold, 0, L) + acc_h[r]
    cbytes = 3 * 4 * B * 2 * rounds + B * 4 * rounds          # commits
    alg_bytes = vbytes + cbytes

    # conventional comparator: snapshots into a 2K+1 slot pool, pointer commit
    cfg = rb.make_config(rb.RSSM_MAMBA2, B, H, sh.ngroups, P, N, W, K)
    spool = torch.empty((2 * K + 1, B, H, P, N), device="cuda")
    slot_of = torch.empty(B, dtype=torch.int32, device="cuda")

    def conv_round(r, a_row):
        rb.step_baseline_spec(cfg, spool, slot_of, yk, A, D, **pool[r % S])
        rb.rssm_baseline_commit(cfg, slot_of, a_row, K)

    spool[2 * K].copy_(s0)
    slot_of.fill_(2 * K)
    for r in range(Wm):
        conv_round(r, acc[rounds + r])
    spool[2 * K].copy_(s0)
    slot_of.fill_(2 * K)
    torch.cuda.synchronize()
    ev2 = _events(torch, 2)
    ev2[0].record()
    for r in range(rounds):
        conv_round(r, acc[r])
    ev2[1].record()
    torch.cuda.synchronize()
    conv_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    del spool
    conv_bytes = (P * N * 4 * (1 + K) + K * ((P + 1) * 4 + 2 * N * 4 * gr) + K * P * 4) * B * H * rounds

    vk_s = sum(verify_ms) / 1e3
    achieved = vbytes / vk_s / 1e9
    accepted = int(acc_h[:rounds].sum())
    return {
        "metric": "speculative verify+commit state GB/s (% of HBM peak) + accepted tokens/s vs "
                  "conventional per-draft snapshots, batch 512 K=6 W=16",
        "value": round(alg_bytes / replay_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": rounds, "warmup": Wm,
        "ms_per_step": round(replay_s * 1e3 / rounds, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded drafts; accepted ~ min(Geometric(0.35) failures, 6))",
        "config": {"workload": f"mamba2_spec_b{B}_h{H}_p{P}_n{N}_w{W}_k{K}"
                               + (f"_g{sh.ngroups}" if sh.ngroups != H else ""), "batch": B,
                   "groups": sh.ngroups,
                   "heads": H, "head_dim": P, "d_state": N, "window": W, "drafts": K,
                   "rounds": rounds, "draft_pool_slots": S},
        "pct_hbm_peak": round(100 * alg_bytes / replay_s / 1e9 / HBM_PEAK_GBS, 2),
        "accepted_tokens_per_s": round(accepted / replay_s, 1),
        "mean_accepted": round(accepted / (rounds * B), 3),
        "fold_fraction": round(folds / (rounds * B), 4),
        "conv_ms_per_round": round(conv_s * 1e3 / rounds, 5),
        "conv_gbs": round(conv_bytes / conv_s / 1e9, 1),
        "speedup_vs_conventional": round(conv_s / replay_s, 3),
        "roofline": {"bound": "hbm", "kernel": "k_m2_verify<64,128,false>" + (
                         "" if sh.ngroups == H else " (with the consolidation launch queued before it "
                         "in rounds where a sequence's drafts do not fit)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     **_traffic_fields("verify"),
                     "alg_bytes_per_launch": round(vbytes / rounds),
                     "avg_launch_us": round(1e6 * vk_s / rounds, 2), "launches": rounds},
        "input_gen_s": round(gen_s, 1),
    }, (sh, prm)


def gdn_verify_bytes(DV, DK, W, K, length, ga=1) -> tuple[float, bool]:
    """HBM bytes of one delta-rule verify launch for one (b, h) pair with `length` committed
    entries (ga gate floats per entry), and whether it folds them first (length + K > W)."""
    f = 4
    entry = (DK + DV + 1 + ga) * f
    drafts = K * (entry + DK * f)
    ring = length * entry
    outs = K * DV * f
    append = K * entry
    fold = length + K > W
    s0 = (2 if fold else 1) * DV * DK * f
    return s0 + ring + drafts + outs + append, fold


DELTA = {
    "gdn": {"name": "Gated DeltaNet", "tag": "gdn", "state0": "gdn_state0", "inputs": "gdn_token_inputs",
            "kind": "RSSM_GDN", "step": "gdn_step", "spec": "gdn_spec_round",
            "data": "synthetic (seeded; q, k L2-normalised N(0,1), v N(0,1), beta sigmoid, alpha exp(-softplus))"},
    "kda": {"name": "Kimi Delta Attention", "tag": "kda", "state0": "kda_state0",
            "inputs": "kda_token_inputs", "kind": "RSSM_KDA", "step": "kda_step",
            "spec": "kda_spec_round",
            "data": "synthetic (seeded; q, k L2-normalised N(0,1), v N(0,1), beta sigmoid, one gate "
                    "exp(-softplus(N(0,1))) per key channel)"},
}


def run_gdn_spec(args, torch, rb, wl, layer="gdn"):
    """Delta-rule speculative decoding (Gated DeltaNet, or Kimi Delta Attention with layer="kda"):
    K = 6 drafts per round into the W = 16 ring (batch 512, 32 heads, 128 x 128), verify then a
    pointer commit of the seeded accepted prefix, against the conventional round (state read once,
    one snapshot written per draft, pointer commit)."""
    L = DELTA[layer]
    sh = wl.GDNShape(batch=args.batch or 512, nheads=32, d_k=128, d_v=128, window=16, max_draft=6)
    DV, DK, W, H, B, K = sh.d_v, sh.d_k, sh.window, sh.nheads, sh.batch, sh.max_draft
    ga = DK if layer == "kda" else 1
    rounds, Wm, S = args.steps or 256, args.warmup, 4
    t0 = time.time()
    s0 = torch.from_numpy(getattr(wl, L["state0"])(sh, 0)).cuda()
    pool = [{k: torch.from_numpy(v).cuda() for k, v in getattr(wl, L["inputs"])(sh, 0, s, ntok=K).items()}
            for s in range(S)]
    acc_h = wl.spec_accepted(B, rounds + Wm, K, p=0.35, seed=0)
    acc = torch.from_numpy(acc_h).cuda()
    gen_s = time.time() - t0

    ctx = rb.Context(layer, B, H, DV, DK, W, max_draft=K)
    ok = torch.empty(K, B, H, DV, device="cuda")
    ctx.init_checkpoint(s0)
    for r in range(Wm):
        ctx.verify(ok, **pool[r % S])
        ctx.commit(acc[rounds + r])
    ctx.init_checkpoint(s0)
    torch.cuda.synchronize()
    ev = _events(torch, 2)
    ev[0].record()
    for r in range(rounds):
        ctx.verify(ok, **pool[r % S])
        ctx.commit(acc[r])
    ev[1].record()
    torch.cuda.synchronize()
    replay_s = ev[0].elapsed_time(ev[1]) / 1e3
    h, l, n, e = ctx.bookkeeping()
    assert e == 0
    ctx.init_checkpoint(s0)
    torch.cuda.synchronize()
    evl = _events(torch, 2 * rounds)
    for r in range(rounds):
        evl[2 * r].record()
        ctx.verify(ok, **pool[r % S])
        evl[2 * r + 1].record()
        ctx.commit(acc[r])
    torch.cuda.synchronize()
    verify_ms = [evl[2 * r].elapsed_time(evl[2 * r + 1]) for r in range(rounds)]
    del ctx

    lens = np.zeros(B, dtype=np.int64)
    vbytes, folds = 0.0, 0
    for r in range(rounds):
        vbytes += sum(gdn_verify_bytes(DV, DK, W, K, int(x), ga)[0] for x in lens) * H
        fold = lens + K > W
        folds += int(fold.sum())
        lens = np.where(fold, 0, lens) + acc_h[r]
    cbytes = 3 * 4 * B * 2 * rounds + B * 4 * rounds          # commits
    alg_bytes = vbytes + cbytes

    cfg = rb.make_config(getattr(rb, L["kind"]), B, H, H, DV, DK, W, K)
    spool = torch.empty((2 * K + 1, B, H, DV, DK), device="cuda")
    slot_of = torch.empty(B, dtype=torch.int32, device="cuda")

    def conv_round(r, a_row):
        rb.step_baseline_spec(cfg, spool, slot_of, ok, **pool[r % S])
        rb.rssm_baseline_commit(cfg, slot_of, a_row, K)

    spool[2 * K].copy_(s0)
    slot_of.fill_(2 * K)
    for r in range(Wm):
        conv_round(r, acc[rounds + r])
    spool[2 * K].copy_(s0)
    slot_of.fill_(2 * K)
    torch.cuda.synchronize()
    ev2 = _events(torch, 2)
    ev2[0].record()
    for r in range(rounds):
        conv_round(r, acc[r])
    ev2[1].record()
    torch.cuda.synchronize()
    conv_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    del spool
    conv_bytes = (DV * DK * 4 * (1 + K) + K * (2 * DK + DV + 1 + ga) * 4 + K * DV * 4) * B * H * rounds

    vk_s = sum(verify_ms) / 1e3
    achieved = vbytes / vk_s / 1e9
    accepted = int(acc_h[:rounds].sum())
    return {
        "metric": "speculative verify+commit state GB/s (% of HBM peak) + accepted tokens/s vs "
                  f"conventional per-draft snapshots, {L['name']} batch 512 K=6 W=16",
        "value": round(alg_bytes / replay_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": rounds, "warmup": Wm,
        "ms_per_step": round(replay_s * 1e3 / rounds, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded drafts; accepted ~ min(Geometric(0.35) failures, 6))",
        "config": {"workload": f"{layer}_spec_b{B}_h{H}_dk{DK}_dv{DV}_w{W}_k{K}", "batch": B,
                   "heads": H, "d_k": DK, "d_v": DV, "window": W, "drafts": K,
                   "rounds": rounds, "draft_pool_slots": S},
        "pct_hbm_peak": round(100 * alg_bytes / replay_s / 1e9 / HBM_PEAK_GBS, 2),
        "accepted_tokens_per_s": round(accepted / replay_s, 1),
        "mean_accepted": round(accepted / (rounds * B), 3),
        "fold_fraction": round(folds / (rounds * B), 4),
        "conv_ms_per_round": round(conv_s * 1e3 / rounds, 5),
        "conv_gbs": round(conv_bytes / conv_s / 1e9, 1),
        "speedup_vs_conventional": round(conv_s / replay_s, 3),
        "roofline": {"bound": "hbm", "kernel": "k_gdn_verify<128,128,1>" if layer == "gdn" else
                     "k_kda_verify<128,128>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     **_traffic_fields(f"{layer}_verify"),
                     "alg_bytes_per_launch": round(vbytes / rounds),
                     "avg_launch_us": round(1e6 * vk_s / rounds, 2), "launches": rounds},
        "input_gen_s": round(gen_s, 1),
    }, sh


def cpu_baseline_gdn_spec(sh, wl, budget_s=8.0, layer="gdn"):
    import oracle
    L = DELTA[layer]
    spec = getattr(oracle, L["spec"])
    cores = oracle.set_threads(0)
    nseq = 64
    K = sh.max_draft
    state = getattr(wl, L["state0"])(sh, 0)[:nseq].astype(np.float64)
    drafts = [{k: np.ascontiguousarray(v[:, :nseq])
               for k, v in getattr(wl, L["inputs"])(sh, 0, s, ntok=K).items()} for s in range(2)]
    acc = wl.spec_accepted(sh.batch, 512, K, seed=0)[:, :nseq]
    t0 = time.perf_counter()
    spec(drafts[0], state, acc[0])
    one = time.perf_counter() - t0
    rounds = max(2, min(256, int(budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    for r in range(rounds):
        spec(drafts[r % 2], state, acc[r])
    el = time.perf_counter() - t0
    return {"value": round(int(acc[:rounds].sum()) / el, 1), "unit": "accepted tokens/s",
            "cores": cores, "kind": "oracle",
            "sample": f"first {rounds} rounds of sequences 0..{nseq - 1} (all heads), conventional fp64 "
                      f"recurrence with a state copy per draft, {el:.1f} s"}


def gdn_bytes(DV, DK, W, length, ga=1) -> float:
    """HBM bytes of one decode launch for one (b, h) pair of a delta-rule layer whose ring holds
    `length` entries; ga = gate floats per entry (1 for Gated DeltaNet, d_k for Kimi Delta
    Attention)."""
    f = 4
    entry = (DK + DV + 1 + ga) * f                 # k, v, beta, gate of one entry
    token = entry + DK * f                         # and q
    ring = length * entry
    o = DV * f
    if length + 1 >= W:
        return 2 * DV * DK * f + token + ring + o
    return DV * DK * f + token + ring + entry + o


MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix


def m2_prefill_bytes(P, N, gr, T) -> float:
    """HBM bytes of one prefill of T tokens for one (b, h) pair: the checkpoint read and written
    once, every token's x, dt, B, C read, every output written."""
    f = 4
    return 2 * P * N * f + T * ((P + 1) * f + 2 * N * f * gr) + T * P * f


def m2_prefill_flops(P, N, T) -> float:
    """Matrix-core flops of one prefill for one (b, h) pair, per 16-token chunk: S C^T and the
    rank-16 update (2 * 16 * P * N each), C B^T (2 * 16 * 16 * N) and M X (2 * 16 * 16 * P)."""
    chunks = (T + 15) // 16
    return chunks * (2 * 2 * 16 * P * N + 2 * 16 * 16 * N + 2 * 16 * 16 * P)


def run_m2_prefill(args, torch, rb, wl):
    """Prefill: a T-token prompt per sequence into the checkpoint (batch 256, 128 heads, 64 x 128),
    against the conventional sequential scan (state read once, the T updates applied in order in
    registers, state written once)."""
    T = args.prompt
    sh = wl.M2Shape(batch=args.batch or 256, nheads=128, ngroups=args.groups or 128, head_dim=64,
                    d_state=128, window=16)
    P, N, W, H, B = sh.head_dim, sh.d_state, sh.window, sh.nheads, sh.batch
    gr = sh.ngroups / sh.nheads
    K, Wm, S = args.steps, args.warmup, 32
    t0 = time.time()
    prm = wl.m2_params(sh, 0)
    s0 = torch.from_numpy(wl.m2_state0(sh, 0)).cuda()
    pool = [{k: torch.from_numpy(v[0]).cuda() for k, v in wl.m2_token_inputs(sh, 0, s).items()}
            for s in range(S)]
    prompt = {k: torch.stack([pool[t % S][k] for t in range(T)]) for k in pool[0]}
    del pool
    A = torch.from_numpy(prm["A"]).cuda()
    D = torch.from_numpy(prm["D"]).cuda()
    gen_s = time.time() - t0
    ctx = rb.Context("mamba2", B, H, P, N, W, ngroups=sh.ngroups)
    ctx.set_params(A, D)
    y = torch.empty(T, B, H, P, device="cuda")
    ctx.init_checkpoint(s0)
    for _ in range(Wm):
        ctx.prefill(y, **prompt)
    torch.cuda.synchronize()
    ev = _events(torch, 2 * K)
    for k in range(K):
        ev[2 * k].record()
        ctx.prefill(y, **prompt)
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    ms = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(K)]
    pre_s = sum(ms) / 1e3
    # conventional sequential scan on the same prompt
    cfg = rb.make_config(rb.RSSM_MAMBA2, B, H, sh.ngroups, P, N, W)
    st = s0.clone()
    for _ in range(Wm):
        rb.step_baseline(cfg, st, y, A, D, **prompt)
    torch.cuda.synchronize()
    ev2 = _events(torch, 2)
    ev2[0].record()
    for _ in range(K):
        rb.step_baseline(cfg, st, y, A, D, **prompt)
    ev2[1].record()
    torch.cuda.synchronize()
    conv_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    bytes_call = m2_prefill_bytes(P, N, gr, T) * B * H
    flops_call = m2_prefill_flops(P, N, T) * B * H
    gbs = bytes_call * K / pre_s / 1e9
    tfl = flops_call * K / pre_s / 1e12
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tfl / MFMA_FP32_PEAK_TFLOPS
    bound_hbm = hbm_frac >= mfma_frac
    return {
        "metric": "SSM prefill tokens/s (prompt into the checkpoint) vs the conventional sequential scan",
        "value": round(B * T * K / pre_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": round(1e3 * pre_s / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded; prompt token t is pool slot t mod 32 of the decode inputs)",
        "config": {"workload": f"mamba2_prefill_b{B}_h{H}_p{P}_n{N}_t{T}"
                               + (f"_g{sh.ngroups}" if sh.ngroups != H else ""),
                   "batch": B, "heads": H, "head_dim": P, "d_state": N, "prompt": T,
                   "groups": sh.ngroups},
        "alg_gbs": round(gbs, 1), "mfma_tflops": round(tfl, 2),
        "conventional_ms": round(1e3 * conv_s / K, 4),
        "speedup_vs_conventional": round(conv_s / pre_s, 3),
        "roofline": {"bound": "hbm" if bound_hbm else "mfma", "kernel": "k_m2_prefill<64,128,false>",
                     "achieved": round(gbs if bound_hbm else tfl, 2),
                     "peak": HBM_PEAK_GBS if bound_hbm else MFMA_FP32_PEAK_TFLOPS,
                     "unit": "GB/s" if bound_hbm else "TFLOP/s",
                     "frac": round(hbm_frac if bound_hbm else mfma_frac, 4),
                     "other": {"hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4)},
                     **_traffic_fields("prefill"), "alg_bytes_per_launch": round(bytes_call),
                     "flops_per_launch": round(flops_call),
                     "avg_launch_us": round(1e6 * pre_s / K, 2), "launches": K},
        "input_gen_s": round(gen_s, 1),
    }, (sh, prm)


def gdn_prefill_bytes(DV, DK, T) -> float:
    """HBM bytes of one Gated DeltaNet prefill of T tokens for one (b, h) pair: the checkpoint read
    and written once, every token's q, k, v, beta, alpha read, every output written."""
    f = 4
    return 2 * DV * DK * f + T * (2 * DK + DV + 2) * f + T * DV * f


def gdn_prefill_flops(DV, DK, T) -> float:
    """Matrix-core flops of one Gated DeltaNet prefill for one (b, h) pair, per 16-token chunk:
    K S^T, Q S^T and the rank-16 update (2 * 16 * DV * DK each), K K^T and Q K^T (2 * 16 * 16 * DK
    each), U = A T (2 * 16^3), U F, (U o R) V and T Z (2 * 16 * 16 * DV each)."""
    chunks = (T + 15) // 16
    return chunks * (3 * 2 * 16 * DV * DK + 2 * 2 * 256 * DK + 2 * 4096 + 3 * 2 * 256 * DV)


def kda_prefill_bytes(DV, DK, T) -> float:
    """HBM bytes of one Kimi Delta Attention prefill of T tokens for one (b, h) pair: the
    checkpoint read and written once, every token's q, k, gate row, v and beta read, every output
    written."""
    f = 4
    return 2 * DV * DK * f + T * (3 * DK + DV + 1) * f + T * DV * f


def kda_prefill_flops(DV, DK, T) -> float:
    """Matrix-core flops of one Kimi Delta Attention prefill for one (b, h) pair, per 16-token
    chunk of the chunk form: Kh S^T, Qh S^T and the rank-16 update (2 * 16 * DV * DK each), the
    A and M blocks (2 * 16 * 16 * DK each), M T (2 * 16^3), (M T) Z and T Z (2 * 16 * 16 * DV
    each). Chunks that take the token path (a gate product below 2^-64) do not occur in these
    inputs."""
    chunks = (T + 15) // 16
    return chunks * (3 * 2 * 16 * DV * DK + 2 * 2 * 256 * DK + 2 * 4096 + 2 * 2 * 256 * DV)


def run_kda_prefill(args, torch, rb, wl):
    """Kimi Delta Attention prefill: a T-token prompt per sequence into the checkpoint (batch 256,
    32 heads, 128 x 128) in 16-token chunks on the matrix cores, against the conventional
    sequential scan on the row-major state."""
    T = args.prompt
    sh = wl.GDNShape(batch=args.batch or 256, nheads=32, d_k=128, d_v=128, window=16)
    DV, DK, W, H, B = sh.d_v, sh.d_k, sh.window, sh.nheads, sh.batch
    K, Wm, S = args.steps, args.warmup, 32
    t0 = time.time()
    s0 = torch.from_numpy(wl.kda_state0(sh, 0)).cuda()
    pool = [{k: torch.from_numpy(v[0]).cuda() for k, v in wl.kda_token_inputs(sh, 0, s).items()}
            for s in range(S)]
    prompt = {k: torch.stack([pool[t % S][k] for t in range(T)]) for k in pool[0]}
    del pool
    gen_s = time.time() - t0
    ctx = rb.Context("kda", B, H, DV, DK, W)
    o = torch.empty(T, B, H, DV, device="cuda")
    ctx.init_checkpoint(s0)
    for _ in range(Wm):
        ctx.prefill(o, **prompt)
    torch.cuda.synchronize()
    ev = _events(torch, 2 * K)
    for k in range(K):
        ev[2 * k].record()
        ctx.prefill(o, **prompt)
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    pre_s = sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(K)) / 1e3
    cfg = rb.make_config(rb.RSSM_KDA, B, H, H, DV, DK, W)
    st = s0.clone()
    for _ in range(Wm):
        rb.step_baseline(cfg, st, o, **prompt)
    torch.cuda.synchronize()
    ev2 = _events(torch, 2)
    ev2[0].record()
    for _ in range(K):
        rb.step_baseline(cfg, st, o, **prompt)
    ev2[1].record()
    torch.cuda.synchronize()
    conv_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    bytes_call = kda_prefill_bytes(DV, DK, T) * B * H
    flops_call = kda_prefill_flops(DV, DK, T) * B * H
    gbs = bytes_call * K / pre_s / 1e9
    tfl = flops_call * K / pre_s / 1e12
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tfl / MFMA_FP32_PEAK_TFLOPS
    bound_hbm = hbm_frac >= mfma_frac
    return {
        "metric": "SSM prefill tokens/s (prompt into the checkpoint) vs the conventional sequential scan",
        "value": round(B * T * K / pre_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": round(1e3 * pre_s / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded; prompt token t is pool slot t mod 32 of the decode inputs)",
        "config": {"workload": f"kda_prefill_b{B}_h{H}_dk{DK}_dv{DV}_t{T}",
                   "batch": B, "heads": H, "d_k": DK, "d_v": DV, "prompt": T},
        "alg_gbs": round(gbs, 1), "mfma_tflops": round(tfl, 2),
        "conventional_ms": round(1e3 * conv_s / K, 4),
        "speedup_vs_conventional": round(conv_s / pre_s, 3),
        "roofline": {"bound": "hbm" if bound_hbm else "mfma", "kernel": "k_kda_prefill<128,128>",
                     "achieved": round(gbs if bound_hbm else tfl, 2),
                     "peak": HBM_PEAK_GBS if bound_hbm else MFMA_FP32_PEAK_TFLOPS,
                     "unit": "GB/s" if bound_hbm else "TFLOP/s",
                     "frac": round(hbm_frac if bound_hbm else mfma_frac, 4),
                     "other": {"hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4)},
                     **_traffic_fields("kda_prefill"), "alg_bytes_per_launch": round(bytes_call),
                     "flops_per_launch": round(flops_call),
                     "avg_launch_us": round(1e6 * pre_s / K, 2), "launches": K},
        "input_gen_s": round(gen_s, 1),
    }, sh


def run_gdn_prefill(args, torch, rb, wl):
    """Gated DeltaNet prefill: a T-token prompt per sequence into the checkpoint (batch 256, 32
    heads, 128 x 128), against the conventional sequential scan (state read once, the T updates
    applied in order in registers, state written once)."""
    T = args.prompt
    sh = wl.GDNShape(batch=args.batch or 256, nheads=32, d_k=128, d_v=128, window=16)
    DV, DK, W, H, B = sh.d_v, sh.d_k, sh.window, sh.nheads, sh.batch
    K, Wm, S = args.steps, args.warmup, 32
    t0 = time.time()
    s0 = torch.from_numpy(wl.gdn_state0(sh, 0)).cuda()
    pool = [{k: torch.from_numpy(v[0]).cuda() for k, v in wl.gdn_token_inputs(sh, 0, s).items()}
            for s in range(S)]
    prompt = {k: torch.stack([pool[t % S][k] for t in range(T)]) for k in pool[0]}
    del pool
    gen_s = time.time() - t0
    ctx = rb.Context("gdn", B, H, DV, DK, W)
    o = torch.empty(T, B, H, DV, device="cuda")
    ctx.init_checkpoint(s0)
    for _ in range(Wm):
        ctx.prefill(o, **prompt)
    torch.cuda.synchronize()
    ev = _events(torch, 2 * K)
    for k in range(K):
        ev[2 * k].record()
        ctx.prefill(o, **prompt)
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    ms = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(K)]
    pre_s = sum(ms) / 1e3
    cfg = rb.make_config(rb.RSSM_GDN, B, H, H, DV, DK, W)
    st = s0.clone()
    for _ in range(Wm):
        rb.step_baseline(cfg, st, o, **prompt)
    torch.cuda.synchronize()
    ev2 = _events(torch, 2)
    ev2[0].record()
    for _ in range(K):
        rb.step_baseline(cfg, st, o, **prompt)
    ev2[1].record()
    torch.cuda.synchronize()
    conv_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    bytes_call = gdn_prefill_bytes(DV, DK, T) * B * H
    flops_call = gdn_prefill_flops(DV, DK, T) * B * H
    gbs = bytes_call * K / pre_s / 1e9
    tfl = flops_call * K / pre_s / 1e12
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tfl / MFMA_FP32_PEAK_TFLOPS
    bound_hbm = hbm_frac >= mfma_frac
    return {
        "metric": "SSM prefill tokens/s (prompt into the checkpoint) vs the conventional sequential scan",
        "value": round(B * T * K / pre_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": round(1e3 * pre_s / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded; prompt token t is pool slot t mod 32 of the decode inputs)",
        "config": {"workload": f"gdn_prefill_b{B}_h{H}_dk{DK}_dv{DV}_t{T}",
                   "batch": B, "heads": H, "d_k": DK, "d_v": DV, "prompt": T},
        "alg_gbs": round(gbs, 1), "mfma_tflops": round(tfl, 2),
        "conventional_ms": round(1e3 * conv_s / K, 4),
        "speedup_vs_conventional": round(conv_s / pre_s, 3),
        "roofline": {"bound": "hbm" if bound_hbm else "mfma", "kernel": "k_gdn_prefill<128,128>",
                     "achieved": round(gbs if bound_hbm else tfl, 2),
                     "peak": HBM_PEAK_GBS if bound_hbm else MFMA_FP32_PEAK_TFLOPS,
                     "unit": "GB/s" if bound_hbm else "TFLOP/s",
                     "frac": round(hbm_frac if bound_hbm else mfma_frac, 4),
                     "other": {"hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4)},
                     **_traffic_fields("gdn_prefill"), "alg_bytes_per_launch": round(bytes_call),
                     "flops_per_launch": round(flops_call),
                     "avg_launch_us": round(1e6 * pre_s / K, 2), "launches": K},
        "input_gen_s": round(gen_s, 1),
    }, sh


def run_m2_fork(args, torch, rb, wl):
    """Per-sequence state copies at the Mamba-2 serving shape (batch 256, 128 heads, 64 x 128,
    W = 16, C kept): fork half of the sequences onto the other half, export them to a packed
    buffer and import them back. Bytes: each copied sequence's state read once and written once."""
    sh = wl.M2Shape(batch=args.batch or 256, nheads=128, ngroups=args.groups or 128, head_dim=64,
                    d_state=128, window=16)
    P, N, W, H, B = sh.head_dim, sh.d_state, sh.window, sh.nheads, sh.batch
    K, Wm = args.steps, args.warmup
    prm = wl.m2_params(sh, 0)
    ctx = rb.Context("mamba2", B, H, P, N, W, ngroups=sh.ngroups)
    ctx.set_params(torch.from_numpy(prm["A"]).cuda(), torch.from_numpy(prm["D"]).cuda())
    ctx.init_checkpoint(torch.from_numpy(wl.m2_state0(sh, 0)).cuda())
    half = B // 2
    src = torch.arange(half, dtype=torch.int32, device="cuda")
    dst = src + half
    nb = ctx.seq_state_bytes()
    buf = torch.empty(half * nb, dtype=torch.uint8, device="cuda")
    seg = nb - 16                                  # state bytes of one sequence (incl. padding)

    def timed(fn):
        for _ in range(Wm):
            fn()
        torch.cuda.synchronize()
        ev = _events(torch, 2)
        ev[0].record()
        for _ in range(K):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / 1e3 / K

    t_fork = timed(lambda: ctx.fork(src, dst))
    t_exp = timed(lambda: ctx.export(src, buf))
    t_imp = timed(lambda: ctx.import_(dst, buf))
    moved = 2 * half * seg
    gbs = moved / t_fork / 1e9
    return {
        "metric": "per-sequence state copy GB/s (fork / export / import), % of HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(1e3 * t_fork, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic (seeded checkpoint)",
        "config": {"workload": f"mamba2_fork_b{B}_h{H}_p{P}_n{N}_w{W}", "batch": B, "heads": H,
                   "head_dim": P, "d_state": N, "window": W, "sequences_copied": half,
                   "state_bytes_per_sequence": seg},
        "export_gbs": round(moved / t_exp / 1e9, 1), "import_gbs": round(moved / t_imp / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "k_seq_copy (fork)", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     **_traffic_fields("fork"), "alg_bytes_per_launch": moved,
                     "avg_launch_us": round(1e6 * t_fork, 2), "launches": K},
    }


def run_gdn(args, torch, rb, wl, layer="gdn"):
    """Delta-rule decode (Gated DeltaNet, or Kimi Delta Attention with layer="kda"): batch 256,
    32 heads, d_k = d_v = 128, W = 16."""
    L = DELTA[layer]
    sh = wl.GDNShape(batch=args.batch or 256, nheads=32, d_k=128, d_v=128, window=16)
    DV, DK, W, H, B = sh.d_v, sh.d_k, sh.window, sh.nheads, sh.batch
    ga = DK if layer == "kda" else 1
    K, Wm, S = args.steps, args.warmup, 32
    t0 = time.time()
    s0 = torch.from_numpy(getattr(wl, L["state0"])(sh, 0)).cuda()
    pool = []
    for s in range(S):
        ins = getattr(wl, L["inputs"])(sh, 0, s)
        pool.append({k: torch.from_numpy(v[0]).cuda() for k, v in ins.items()})
    gen_s = time.time() - t0
    ctx = rb.Context(layer, B, H, DV, DK, W)
    o = torch.empty(B, H, DV, device="cuda")
    # the timed steps start at ring fill `pre`: K steps hold ceil(K / W) folds
    pre = 0 if args.graph else (W - K % W) % W

    def restart():
        ctx.init_checkpoint(s0)
        for t in range(pre):
            ctx.decode_step(o, **pool[(S - 1 - t) % S])

    restart()
    for t in range(Wm):
        ctx.decode_step(o, **pool[t % S])
    restart()
    torch.cuda.synchronize()
    reps = None
    if not args.graph:
        ev = _events(torch, 2)
        ev[0].record()
        for t in range(K):
            ctx.decode_step(o, **pool[t % S])
        ev[1].record()
        torch.cuda.synchronize()
        total_ms = ev[0].elapsed_time(ev[1])
        reps = _repeat_ms(torch, total_ms, args.reps, restart,
                          lambda t: ctx.decode_step(o, **pool[t % S]), K)
    restart()
    torch.cuda.synchronize()
    evl = _events(torch, 2 * K)
    for t in range(K):
        evl[2 * t].record()
        ctx.decode_step(o, **pool[t % S])
        evl[2 * t + 1].record()
    torch.cuda.synchronize()
    launch_ms = [evl[2 * t].elapsed_time(evl[2 * t + 1]) for t in range(K)]
    if args.graph:
        ctx.init_checkpoint(s0)
        total_ms = _graph_time(torch, S, lambda t: ctx.decode_step(o, **pool[t]), 1, K // S)
        h, l, n, e = ctx.bookkeeping()
        assert e == 0 and l[0] == 0, "unexpected bookkeeping after the graph replays"
    alg = sum(gdn_bytes(DV, DK, W, (pre + t) % W, ga) for t in range(K)) * B * H
    cfg = rb.make_config(getattr(rb, L["kind"]), B, H, H, DV, DK, W)
    st = s0.clone()
    o1 = torch.empty(1, B, H, DV, device="cuda")
    pool1 = [{k: v.unsqueeze(0) for k, v in pool[t].items()} for t in range(S)]
    for t in range(Wm):
        rb.step_baseline(cfg, st, o1, **pool1[t % S])
    st.copy_(s0)
    torch.cuda.synchronize()
    if args.graph:
        rmw_s = _graph_time(torch, S, lambda t: rb.step_baseline(cfg, st, o1, **pool1[t]), 1, K // S) / 1e3
    else:
        ev2 = _events(torch, 2)
        ev2[0].record()
        for t in range(K):
            rb.step_baseline(cfg, st, o1, **pool1[t % S])
        ev2[1].record()
        torch.cuda.synchronize()
        rmw_s = ev2[0].elapsed_time(ev2[1]) / 1e3
    rmw_bytes = (2 * DV * DK * 4 + (2 * DK + DV + 1 + ga) * 4 + DV * 4) * B * H * K
    rep = [t for t in range(K) if (pre + t) % W != W - 1]
    fol = [t for t in range(K) if (pre + t) % W == W - 1]
    rep_b = sum(gdn_bytes(DV, DK, W, (pre + t) % W, ga) for t in rep) * B * H
    fol_b = sum(gdn_bytes(DV, DK, W, (pre + t) % W, ga) for t in fol) * B * H
    rep_s = sum(launch_ms[t] for t in rep) / 1e3
    fol_s = sum(launch_ms[t] for t in fol) / 1e3
    replay_s = total_ms / 1e3
    return {
        "metric": f"{L['name']} decode state GB/s (% of HBM peak) + tokens/s vs conventional, "
                  "batch 256 W=16",
        "value": round(alg / replay_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": Wm, "ms_per_step": round(total_ms / K, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": L["data"],
        "config": {"workload": f"{layer}_decode_b{B}_h{H}_dk{DK}_dv{DV}_w{W}" + ("_graph" if args.graph else ""),
                   "batch": B, "heads": H, "d_k": DK, "d_v": DV, "window": W, "input_pool_slots": S,
                   "ring_fill": f"lock-step: every sequence starts at {pre} entries "
                                f"({sum(1 for t in range(K) if (pre + t) % W == W - 1)} folding steps in {K})",
                   "launch": "hip graph of 2 W steps, replayed" if args.graph else "eager"},
        "pct_hbm_peak": round(100 * alg / replay_s / 1e9 / HBM_PEAK_GBS, 2),
        "ms_per_step_reps": reps,
        "tokens_per_s": round(B * K / replay_s, 1),
        "rmw_ms_per_step": round(rmw_s * 1e3 / K, 5),
        "rmw_gbs": round(rmw_bytes / rmw_s / 1e9, 1),
        "speedup_vs_rmw": round(rmw_s / replay_s, 3),
        "roofline": {"bound": "hbm", "kernel": f"k_{layer}_decode<128,128,kUniform> (steps that replay)",
                     "achieved": round(rep_b / rep_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(rep_b / rep_s / 1e9 / HBM_PEAK_GBS, 4),
                     **_traffic_fields(f"{layer}_replay"),
                     "alg_bytes_per_launch": round(rep_b / len(rep)),
                     "avg_launch_us": round(1e6 * rep_s / len(rep), 2), "launches": len(rep)},
        "fold_steps": {"kernel": f"k_{layer}_decode<128,128,kMayFold> (the step that fills the ring)",
                       "achieved_gbs": round(fol_b / fol_s / 1e9, 1) if fol else None,
                       **_traffic_fields(f"{layer}_fold"),
                       "alg_bytes_per_launch": round(fol_b / len(fol)) if fol else None,
                       "avg_launch_us": round(1e6 * fol_s / len(fol), 2) if fol else None,
                       "launches": len(fol)},
        "input_gen_s": round(gen_s, 1),
    }, sh


def cpu_baseline_gdn(sh, wl, budget_s=8.0, layer="gdn"):
    import oracle
    L = DELTA[layer]
    step = getattr(oracle, L["step"])
    cores = oracle.set_threads(0)
    state = getattr(wl, L["state0"])(sh, 0).astype(np.float64)
    toks = [{k: np.ascontiguousarray(v[0]) for k, v in getattr(wl, L["inputs"])(sh, 0, s).items()}
            for s in range(4)]
    for _ in range(2):
        t0 = time.perf_counter()
        step(*(toks[0][k] for k in ("q", "k", "v", "beta", "alpha")), state)
        one = time.perf_counter() - t0
    steps = max(2, min(512, int(budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    for t in range(steps):
        step(*(toks[t % 4][k] for k in ("q", "k", "v", "beta", "alpha")), state)
    el = time.perf_counter() - t0
    tok_s = sh.batch * steps / el
    one_core = _single_core(lambda k, st: step(*(k[n] for n in ("q", "k", "v", "beta", "alpha")), st),
                            toks, state, sh.batch, cores)
    return {"value": round(2 * sh.d_v * sh.d_k * 8 * sh.nheads * tok_s / 1e9, 3),
            "unit": "GB/s (fp64 state read+write)", "cores": cores, "kind": "oracle",
            "tokens_per_s": round(tok_s, 1), "cpu_model": _cpu_model(),
            "single_core_tokens_per_s": one_core,
            "sample": f"first {steps} decode steps of all {sh.batch} sequences, conventional fp64 "
                      f"recurrence, {el:.1f} s"}


def cpu_baseline_m2_spec(sh, prm, wl, budget_s=8.0):
    import oracle
    cores = oracle.set_threads(0)
    nseq = 64
    K = sh.max_draft
    small = wl.M2Shape(nseq, sh.nheads, sh.ngroups, sh.head_dim, sh.d_state, sh.window, K)
    state = wl.m2_state0(sh, 0)[:nseq].astype(np.float64)
    drafts = [{k: np.ascontiguousarray(v[:, :nseq]) for k, v in wl.m2_token_inputs(sh, 0, s, ntok=K).items()}
              for s in range(2)]
    acc = wl.spec_accepted(sh.batch, 512, K, seed=0)[:, :nseq]
    t0 = time.perf_counter()
    oracle.m2_spec_round(prm["A"], prm["D"], drafts[0], state, acc[0])
    one = time.perf_counter() - t0
    rounds = max(2, min(256, int(budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    for r in range(rounds):
        oracle.m2_spec_round(prm["A"], prm["D"], drafts[r % 2], state, acc[r])
    el = time.perf_counter() - t0
    del small
    return {"value": round(int(acc[:rounds].sum()) / el, 1), "unit": "accepted tokens/s",
            "cores": cores, "kind": "oracle",
            "sample": f"first {rounds} rounds of sequences 0..{nseq - 1} (all heads), conventional fp64 "
                      f"recurrence with a state copy per draft, {el:.1f} s"}


def cpu_baseline_m2(sh, prm, wl, host_pool=None, budget_s=12.0):
    """Time the CPU oracle (conventional fp64 recurrence) on the first steps of the same seeded
    schedule (step t takes token slot t mod 32, as the GPU legs), sized to about `budget_s` of CPU
    time."""
    import oracle
    cores = oracle.set_threads(0)
    nseq = sh.batch
    state = wl.m2_state0(sh, 0).astype(np.float64)
    if host_pool is None:
        host_pool = [{k: v[0] for k, v in wl.m2_token_inputs(sh, 0, s).items()} for s in range(32)]
    toks = [{k: np.ascontiguousarray(v) for k, v in t.items()} for t in host_pool]
    S = len(toks)
    for _ in range(2):   # first calls pay for thread start-up and page faults
        t0 = time.perf_counter()
        oracle.m2_step(prm["A"], prm["D"], toks[0]["x"], toks[0]["B"], toks[0]["C"], toks[0]["dt"], state)
        one = time.perf_counter() - t0
    state = wl.m2_state0(sh, 0).astype(np.float64)
    steps = max(2, min(512, int(budget_s / max(one, 1e-6))))
    t0 = time.perf_counter()
    for t in range(steps):
        k = toks[t % S]
        oracle.m2_step(prm["A"], prm["D"], k["x"], k["B"], k["C"], k["dt"], state)
    el = time.perf_counter() - t0
    tok_s = nseq * steps / el
    # the oracle reads and rewrites the fp64 state once per token
    gbs = 2 * sh.head_dim * sh.d_state * 8 * sh.nheads * tok_s / 1e9
    one_core = _single_core(lambda k, st: oracle.m2_step(prm["A"], prm["D"], k["x"], k["B"], k["C"],
                                                         k["dt"], st),
                            toks, state, nseq, cores)
    return {"value": round(gbs, 3), "unit": "GB/s (fp64 state read+write)", "cores": cores,
            "kind": "oracle", "tokens_per_s": round(tok_s, 1), "cpu_model": _cpu_model(),
            "single_core_tokens_per_s": one_core,
            "sample": f"decode steps 0..{steps - 1} of sequences 0..{nseq - 1} (all {sh.nheads} heads), "
                      f"step t on token slot t mod {S} as on the GPU, from the same initial state; "
                      f"conventional fp64 recurrence, {el:.1f} s"}


def _single_core(step, toks, state, nseq, cores, budget_s=2.0):
    """The same oracle step on one thread (about `budget_s` of work), tokens/s; the thread count is
    restored afterwards."""
    import oracle
    oracle.set_threads(1)
    try:
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            step(toks[n % len(toks)], state)
            n += 1
        el = time.perf_counter() - t0
    finally:
        oracle.set_threads(cores)
    return round(nseq * n / el, 1)


def calibrate_copy(torch, nbytes=1 << 30, reps=3):
    """A plain device copy of known size, so rocprofv3 counter runs can scale FETCH_SIZE /
    WRITE_SIZE to bytes."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (decode tokens; verify rounds for m2_spec); default 512 / 256")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="m2_serve",
                    choices=["m2_serve", "m2_serve_bf16", "m2_spec", "gdn_serve", "gdn_spec",
                             "kda_serve", "kda_spec", "m2_prefill", "gdn_prefill", "kda_prefill",
                             "m2_fork"])
    ap.add_argument("--prompt", type=int, default=512,
                    help="prompt tokens (m2_prefill, gdn_prefill, kda_prefill)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch (sweeps)")
    ap.add_argument("--groups", type=int, default=0,
                    help="Mamba-2 B/C groups (default: one per head)")
    ap.add_argument("--stagger", action="store_true",
                    help="m2_serve legs: every sequence at its own ring fill (b mod W), so every "
                         "launch mixes folding and replaying tiles")
    ap.add_argument("--graph", action="store_true",
                    help="decode legs: time replays of a captured HIP graph of 2 W steps (both paths)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rmw", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--reps", type=int, default=5,
                    help="serving legs: runs of the timed region (the first gives value)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path has no cross-GPU step; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    from checkpoint_replay_buffer_amd import binding as rb
    rb.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
    if args.graph and args.steps:
        args.steps = (args.steps + 31) // 32 * 32     # whole captured windows of 32 steps
    if args.workload == "m2_spec":
        line, (sh, prm) = run_m2_spec(args, torch, rb, wl)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_m2_spec(sh, prm, wl)
    elif args.workload in ("gdn_spec", "kda_spec"):
        layer = args.workload[:3]
        line, sh = run_gdn_spec(args, torch, rb, wl, layer)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_gdn_spec(sh, wl, layer=layer)
    elif args.workload == "m2_prefill":
        args.steps = args.steps or 8
        args.warmup = min(args.warmup, 2)
        line, (sh, prm) = run_m2_prefill(args, torch, rb, wl)
        if not args.no_cpu_baseline:
            cb = cpu_baseline_m2(sh, prm, wl)
            cb["gbs_fp64_state"] = cb["value"]
            cb["value"], cb["unit"] = cb["tokens_per_s"], "tokens/s"
            line["cpu_baseline"] = cb
    elif args.workload == "gdn_prefill":
        args.steps = args.steps or 8
        args.warmup = min(args.warmup, 2)
        line, sh = run_gdn_prefill(args, torch, rb, wl)
        if not args.no_cpu_baseline:
            cb = cpu_baseline_gdn(sh, wl)
            cb["gbs_fp64_state"] = cb["value"]
            cb["value"], cb["unit"] = cb["tokens_per_s"], "tokens/s"
            line["cpu_baseline"] = cb
    elif args.workload == "kda_prefill":
        args.steps = args.steps or 4
        args.warmup = min(args.warmup, 1)
        line, sh = run_kda_prefill(args, torch, rb, wl)
        if not args.no_cpu_baseline:
            cb = cpu_baseline_gdn(sh, wl, layer="kda")
            cb["gbs_fp64_state"] = cb["value"]
            cb["value"], cb["unit"] = cb["tokens_per_s"], "tokens/s"
            line["cpu_baseline"] = cb
    elif args.workload == "m2_fork":
        args.steps = args.steps or 20
        args.warmup = min(args.warmup, 3)
        line = run_m2_fork(args, torch, rb, wl)
    elif args.workload in ("gdn_serve", "kda_serve"):
        layer = args.workload[:3]
        args.steps = args.steps or 512
        line, sh = run_gdn(args, torch, rb, wl, layer)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_gdn(sh, wl, layer=layer)
    else:
        args.steps = args.steps or 512
        line, (sh, prm, host_pool) = run_m2(args, torch, rb, wl)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_m2(sh, prm, wl, host_pool)
    if args.workload in ("m2_serve", "m2_serve_bf16", "gdn_serve", "kda_serve", "m2_spec", "gdn_spec",
                         "kda_spec", "m2_fork"):
        cg = measure_copy_gbs(torch)
        line["copy_gbs"] = round(cg, 1)
        line["pct_of_copy"] = round(100 * line["value"] / cg, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
