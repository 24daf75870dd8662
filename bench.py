"""Benchmark: SMC-SD verify + resample + KV pointer-exchange steps per second on one MI355X.

Workload (default): B=32 prompts x N=16 particles, K=4 draft tokens, V=128256, bf16 logits
with the Zipf generator (one seeded vocabulary permutation, noise 0.3; draft = target +
Normal(0, 0.8)), temperature 0.8, tau = 0.5, 2048-token shared prefix in 16-token blocks.
A step is one pass of the whole hot path over one batch: the verify (LSE pass, gathers,
bonus token, weight update), the resample (ESS, systematic resampling) and the KV exchange
(refcounted block-table exchange + reservation), timed as one smcsd_step call per round
(--two-calls: smcsd_verify + smcsd_resample_kv_reassign; --separate-kv: three calls).  Inputs are resident in HBM: four distinct
logit sets (4.7 GB, far above the 256 MB last-level cache) are generated untimed and step t
uses set t mod 4.

Prints one JSON line.  Before the W warm-up steps the bench runs whole steps, untimed, for
--settle-ms (after any idle period this GPU runs the path ~10 % slower for ~20 ms while its
clocks settle); the W warm-up steps then start a fresh episode that the timed steps continue.
`roofline` covers the dominant work, the smcsd_verify call: its algorithmic bytes
(B*N*(2K+1)*V*elt logit bytes) over its average duration from back-to-back calls between one
pair of HIP events on its stream, right after the timed region.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload and scales it to steps/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EVENT_EVERY = 16

# HBM bytes per smcsd_verify call (k_lse_partials + k_smc_finalize) on c3_batched, from two
# rocprofv3 passes (FETCH_SIZE, WRITE_SIZE) scaled by the same counters on a 1 GiB device
# copy; profiles/smcsd_verify_c3_batched_hbm_bytes.md has the commands and figures.  Valid
# only for the kernel sources they were taken on: any change to them reports null.
READ_CEILING_MIN_BYTES = 512 << 20

VERIFY_TRAFFIC = {
    "workload": "c3_batched",
    "bytes": 1186553475,
    "sources": {
        "smc_verification_resampling_amd/csrc/verify.hip":
            "b8001d90a3b8f29615b9f3940ba9837605be9cef89d69535d3c1f18d8835a71a",
        "smc_verification_resampling_amd/csrc/device.hpp":
            "2522278716f37d21a7304625ff4722f81d617ddcbba29605d41050dbafd80786",
        "smc_verification_resampling_amd/csrc/internal.hpp":
            "528605770c5bffd5d202d05a1705d168973a6b2cc20655e289dd8275e2eec320",
    },
}


def verify_traffic(workload):
    """Counter-measured HBM bytes per verify call, or None if the workload differs or the
    kernel sources changed since the counters were taken."""
    import hashlib

    if workload != VERIFY_TRAFFIC["workload"]:
        return None
    for rel, digest in VERIFY_TRAFFIC["sources"].items():
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return VERIFY_TRAFFIC["bytes"]


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_batched",
                    help="c1_tiny | c2_single_prompt | c3_batched | c4_wide_particle | c5_power")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps run for this long before the warm-up steps: after any "
                         "idle period the MI355X runs this path ~10%% slower for ~20 ms")
    ap.add_argument("--draft-logq", action="store_true",
                    help="draft tokens and their log q from smcsd_draft_sample (untimed, part of "
                         "the Extend step); the timed verify takes them and skips the draft rows")
    ap.add_argument("--race-bonus", action="store_true",
                    help="SMCSD_MODE_SMC_RACE: the bonus token by an exponential race inside the "
                         "LSE pass instead of the inverse CDF with its one-slab re-read")
    ap.add_argument("--two-calls", action="store_true",
                    help="time smcsd_verify then smcsd_resample_kv_reassign instead of smcsd_step "
                         "(the whole round in one call; same results)")
    ap.add_argument("--separate-kv", action="store_true",
                    help="time smcsd_verify, smcsd_resample and smcsd_kv_reassign as three calls "
                         "(same results)")
    ap.add_argument("--graph", action="store_true",
                    help="record each run of timed steps in a HIP graph (untimed) and time its "
                         "replay: the same launches with the same arguments, without the host's "
                         "per-launch cost (for the launch-bound small workloads)")
    ap.add_argument("--probe-mib", type=int, default=1024,
                    help="size of the reference copy kernel (0 = skip)")
    return ap.parse_args()


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verify / resample / KV path shards by prompt "
              "with no exchange, so one GPU's figure is the one measured (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import smc_verification_resampling_amd as sm
    from workloads import configs, synth

    cfg = configs.get(args.workload)
    dev = "cuda"
    torch.cuda.init()
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    print("[bench] %s: generating %d logit sets of %.4g GB" % (
        cfg.name, cfg.n_sets, cfg.logit_bytes_per_step / 1e9), file=sys.stderr, flush=True)
    base = synth.zipf_base(cfg, dev) if cfg.target_kind == "zipf" else None
    sets = []
    for s in range(cfg.n_sets):
        t, d = synth.make_logit_set(cfg, s, dev, base)
        sets.append((t, d, synth.sample_draft_tokens(cfg, d, s), None))
    draft_info = None
    mode = sm.MODE_SMC_RACE if args.race_bonus else sm.MODE_SMC
    variant = ("+draft_logq" if args.draft_logq else "") + ("+race_bonus" if args.race_bonus else "")
    if args.draft_logq:
        sets, draft_info = draft_side(cfg, sets)

    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    lw = torch.zeros(S, **f32)
    kv = synth.initial_kv(cfg)
    # the episode's start state stays resident: a restart is device-to-device copies, so the
    # GPU never waits on the host between the warm-up and the timed steps
    kv0 = {k: torch.from_numpy(kv[k]).to(dev) for k in ("tables", "refcounts", "free_list",
                                                        "free_top")}
    tables, rc, fl, top = (kv0[k].clone() for k in ("tables", "refcounts", "free_list", "free_top"))
    ident = torch.arange(N, **i32).repeat(B, 1)
    no_res = torch.zeros(B, **i32)
    L0 = int(kv["seq_len"])
    ws_v = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    ws_kv = sm.alloc_workspace(sm.OP_KV, B, N, P=cfg.pool)
    tokens = torch.zeros((S, K + 1), **i32)
    num = torch.zeros(S, **i32)
    logp = torch.zeros((S, K + 1), **f32)
    logq = torch.zeros((S, max(K, 1)), **f32)
    status = torch.zeros(1, **i32)
    anc = torch.zeros((B, N), **i32)
    ess = torch.zeros(B, **f32)
    resampled = torch.zeros(B, **i32)
    cow = torch.zeros((S, 3), **i32)
    ncow = torch.zeros(1, **i32)
    seed = cfg.rng_seed
    state = {"L": L0, "round": 0, "t": 0}

    def kv_call(a, r):
        sm.kv_reassign(a, r, B, N, tables, cfg.block_size, state["L"], K + 1, rc, fl, top, cow, ncow,
                       status, ws_kv)

    def reset():
        """Restart the episode (enqueued on the stream; no host synchronisation)."""
        lw.zero_()
        tables.copy_(kv0["tables"])
        rc.copy_(kv0["refcounts"])
        fl.copy_(kv0["free_list"])
        top.copy_(kv0["free_top"])
        state["L"] = L0
        state["round"] = 0
        kv_call(ident, no_res)

    # the block pool holds M_cap slots per sequence: an episode is at most cfg.iters rounds
    max_rounds = cfg.iters

    one_call = not (args.two_calls or args.separate_kv)

    def step(ev=None):
        t = state["t"]
        tgt, drf, toks, lq_in = sets[t % cfg.n_sets]
        if one_call:
            state["L"] += K + 1
            sm.step(tgt, None if lq_in is not None else drf, toks, B, N, K, V, cfg.temperature,
                    cfg.alpha, mode, cfg.tau, seed, t, lw, tokens, anc, ess, resampled, tables,
                    cfg.block_size, state["L"], K + 1, rc, fl, top, cow, ncow, status, ws_v, ws_kv,
                    out_num_tokens=num, out_logp=logp, out_logq=logq, logq_in=lq_in)
            state["t"] += 1
            state["round"] += 1
            return
        if ev is not None:
            ev[0].record()
        sm.verify(tgt, None if lq_in is not None else drf, toks, B, N, K, V, cfg.temperature,
                  cfg.alpha, mode, seed, t, tokens, status, ws_v, log_weights=lw,
                  out_num_tokens=num, out_logp=logp, out_logq=logq, logq_in=lq_in)
        if ev is not None:
            ev[1].record()
        state["L"] += K + 1
        if args.separate_kv:
            sm.resample(lw.view(B, N), B, N, cfg.tau, seed, t, anc, ess, resampled, status)
            kv_call(anc, resampled)
        else:
            sm.resample_kv_reassign(lw.view(B, N), B, N, cfg.tau, seed, t, anc, ess, resampled,
                                    tables, cfg.block_size, state["L"], K + 1, rc, fl, top, cow,
                                    ncow, status, ws_kv)
        state["t"] += 1
        state["round"] += 1

    def steps_in_episode(n):
        """Steps that fit before the episode's end, restarting it first if it is full."""
        if state["round"] >= max_rounds:
            reset()
        return min(n, max_rounds - state["round"])

    # settle: after an idle period this GPU's clocks take ~20 ms of load to settle (the verify
    # call runs ~10 % slower meanwhile); run whole steps, untimed, for settle_ms first
    reset()
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_ms / 1e3:
        n = steps_in_episode(50)
        for _ in range(n):
            step()
        settle_steps += n
        torch.cuda.synchronize()
    # warm-up: the W steps just before the timed region, from a fresh episode that the timed
    # steps then continue
    reset()
    done_w = 0
    while done_w < args.warmup:
        n = steps_in_episode(args.warmup - done_w)
        for _ in range(n):
            step()
        done_w += n
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps; an episode restart (device copies) between runs of
    # steps is outside the clock.  HIP events bracket the verify call of one step in
    # EVENT_EVERY (not a run's first step): each recorded event costs a few microseconds
    events = []
    chunks = []
    t_total = 0.0
    done = 0
    while done < args.steps:
        n = steps_in_episode(args.steps - done)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               if (not args.graph and not one_call and i > 0 and (done + i) % EVENT_EVERY == 0)
               else None for i in range(n)]
        graph = None
        if args.graph:
            # record the run's steps (nothing executes during capture), then replay them once
            saved = dict(state)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(n):
                    step()
            state.update(saved)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if graph is not None:
            graph.replay()
        else:
            for i in range(n):
                step(evs[i])
        torch.cuda.synchronize()
        t_total += time.perf_counter() - t0
        if graph is not None:
            for i in range(n):  # the host-side counters the replay advanced
                state["t"] += 1
                state["round"] += 1
                state["L"] += K + 1
            del graph
        events += [e for e in evs if e is not None]
        done += n
        chunks.append(n)
    st = int(status.cpu()[0])
    # KV occupancy at the end of the timed region: blocks off the free stack (the next
    # round's reservation included) against every sequence holding its own copy
    live = cfg.pool - int(top.cpu()[0])
    unshared = S * -(-(state["L"] + K + 1) // cfg.block_size)
    kv_occ = {"rounds_in_episode": state["round"], "context_tokens": state["L"],
              "live_blocks": live, "unshared_blocks": unshared,
              "saving": round(1.0 - live / unshared, 4)}
    in_region_us = [e[0].elapsed_time(e[1]) * 1e3 for e in events]
    ms_per_step = t_total / args.steps * 1e3
    steps_per_s = args.steps / t_total
    bytes_per_verify = cfg.logit_bytes_per_step
    if args.draft_logq:  # the K draft rows are not read
        bytes_per_verify = bytes_per_verify * (K + 1) // (2 * K + 1)
    step_gbs = bytes_per_verify * steps_per_s / 1e9

    # roofline: the verify call's average duration over back-to-back calls between one event
    # pair, right after the timed region (the GPU still under load), independent of --steps
    verify_reps = max(50, min(200, args.steps))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tgt0, drf0, toks0, lq0 = sets[0]
    ev[0].record()
    for i in range(verify_reps):
        tgt, drf, toks, lq_in = sets[i % cfg.n_sets]
        sm.verify(tgt, None if lq_in is not None else drf, toks, B, N, K, V, cfg.temperature,
                  cfg.alpha, mode, seed, state["t"] + i, tokens, status, ws_v, log_weights=lw,
                  out_num_tokens=num, out_logp=logp, out_logq=logq, logq_in=lq_in)
    ev[1].record()
    torch.cuda.synchronize()
    verify_avg_s = ev[0].elapsed_time(ev[1]) / 1e3 / verify_reps
    achieved_gbs = bytes_per_verify / verify_avg_s / 1e9

    # the read ceiling only where the verify streams well past the 256 MB last-level cache
    # (the tiny shapes are launch-bound: a read of their few bytes measures launches)
    ceiling = read_ceiling(bytes_per_verify) if bytes_per_verify >= READ_CEILING_MIN_BYTES else None
    sps = sps_timing(cfg, sets, args.steps) if cfg.sps else None
    ref = reference_kernels(args.probe_mib) if args.probe_mib > 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, sets, args.cpu_seconds, "race" if args.race_bonus else "cdf")

    out = {
        "metric": "SMC verify+resample steps/s; HBM GB/s % of peak (V=128256,N=16,K=4,B=32)",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type of the path (fp32 accumulation); the logits' storage type is
        # config.logits_dtype
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "%s%s: B=%d prompts x N=%d particles, K=%d, V=%d, %s logits (%s), T=%g, "
                        "alpha=%g, tau=%g, ctx %d in %d-token blocks%s" % (
                            cfg.name, variant, B, N, K, V,
                            cfg.dtype, cfg.target_kind, cfg.temperature, cfg.alpha, cfg.tau,
                            cfg.ctx0, cfg.block_size, ", shared prefix" if cfg.shared_prefix else ""),
            "logits_dtype": cfg.dtype,
            "step": ("smcsd_step (verify + resample + KV exchange in one call)" if one_call else
                     "smcsd_verify + %s" % ("smcsd_resample + smcsd_kv_reassign" if args.separate_kv
                                            else "smcsd_resample_kv_reassign"))
                    + (" (logq_in: target rows only)" if args.draft_logq else "")
                    + (" (race-mode bonus)" if args.race_bonus else "")
                    + ("; timed as HIP graph replays" if args.graph else ""),
            "settle": {"ms": args.settle_ms, "steps": settle_steps},
            "draft_sample": draft_info,
            "logit_sets": cfg.n_sets,
            "algorithmic_bytes_per_step": bytes_per_verify,
            "step_hbm_gbs": round(step_gbs, 1),
            "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "kv_occupancy": kv_occ,
            "sps_verify": sps,
            "combined_ms_per_step": (round(ms_per_step + sps["us_per_call"] / 1e3, 5)
                                     if sps else None),
            "status": st,
            "reference_kernels": ref,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "smcsd_verify (LSE pass + finalize)",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": verify_traffic(cfg.name + variant),
            "avg_launch_us": round(verify_avg_s * 1e6, 2),
            "launches_timed": verify_reps,
            "timing": "back-to-back verify calls between one event pair after the timed region",
            "in_region_median_us": round(float(np.median(in_region_us)), 2) if in_region_us else None,
            "in_region_launches": len(in_region_us),
            # the achievable read rate on this GPU (smcsd_stream_read over as many bytes),
            # and the verify call's rate as a fraction of it
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": (round(ceiling["avg_us"] * 1e-6 * bytes_per_verify
                                           / (verify_avg_s * ceiling["bytes"]), 4)
                                     if ceiling else None),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def draft_side(cfg, sets):
    """Draft tokens and their log q for every logit set from smcsd_draft_sample, one draft
    position per call (as the Extend step would call it), untimed in the step; the cost
    of one position call over the whole batch is timed here with HIP events."""
    import torch

    import smc_verification_resampling_amd as sm

    S, K, V = cfg.S, cfg.K, cfg.V
    ws = sm.alloc_workspace(sm.OP_DRAFT, S, 1, 0, V)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = []
    for s, (tgt, drf, _, _) in enumerate(sets):
        toks = torch.zeros((S, K), dtype=torch.int32, device="cuda")
        lq = torch.zeros((S, K), dtype=torch.float32, device="cuda")
        flat = drf.reshape(-1)
        for k in range(K):
            tk = torch.zeros(S, dtype=torch.int32, device="cuda")
            lk = torch.zeros(S, dtype=torch.float32, device="cuda")
            sm.draft_sample(flat[k * V:], S, V, cfg.temperature, cfg.rng_seed, s, k, tk, st, ws,
                            out_logq=lk, row_stride=K * V)
            toks[:, k] = tk
            lq[:, k] = lk
        out.append((tgt, drf, toks, lq))
    tk = torch.zeros(S, dtype=torch.int32, device="cuda")
    lk = torch.zeros(S, dtype=torch.float32, device="cuda")
    flat = sets[0][1].reshape(-1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    reps = 50
    torch.cuda.synchronize()
    ev[0].record()
    for r in range(reps):
        sm.draft_sample(flat[(r % K) * V:], S, V, cfg.temperature, cfg.rng_seed, 99, r % K, tk, st,
                        ws, out_logq=lk, row_stride=K * V)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    elt = 2 if cfg.dtype == "bf16" else 4
    return out, {"us_per_position_call": round(us, 2), "rows_per_call": S,
                 "GBps": round(S * V * elt / (us * 1e-6) / 1e9, 1), "status": int(st.cpu()[0])}


def sps_timing(cfg, sets, steps):
    """The SpS modified-rejection verify on particle 0 of every prompt, on the same logits,
    timed on its own (HIP events around a run of calls) after the SMC steps."""
    import torch

    import smc_verification_resampling_amd as sm

    B, N, K, V = cfg.B, cfg.N, cfg.K, cfg.V
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = sm.alloc_workspace(sm.OP_VERIFY_SPS, B, 1, K, V)
    tok = torch.zeros((B, K + 1), **i32)
    num = torch.zeros(B, **i32)
    status = torch.zeros(1, **i32)
    emitted = torch.zeros(B, dtype=torch.int64, device="cuda")

    def call(t):
        tgt, drf, toks, _ = sets[t % cfg.n_sets]
        sm.verify(tgt, drf, toks, B, 1, K, V, cfg.temperature, 1.0, sm.MODE_SPS, cfg.rng_seed,
                  t, tok, status, ws, out_num_tokens=num, seq_step=N)

    for t in range(5):
        call(t)
    n = max(1, min(steps, 200))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for t in range(n):
        call(t)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / n
    for t in range(n):  # untimed: the number of tokens each call emits
        call(t)
        emitted += num
    torch.cuda.synchronize()
    return {"calls": n, "sequences": B, "us_per_call": round(us, 2),
            "mean_emitted_tokens": round(float(emitted.sum()) / (n * B), 4),
            "status": int(status.cpu()[0])}


def read_ceiling(nbytes, reps=50):
    """The achievable HBM read rate of this GPU: smcsd_stream_read (the LSE pass's 16-byte
    nontemporal loads, nothing else) over a buffer of random bits of the verify call's byte
    count, several times the 256 MB last-level cache, `reps` back-to-back calls between
    one event pair."""
    import torch

    import smc_verification_resampling_amd as sm

    n = (int(nbytes) + 15) // 16 * 16
    buf = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    buf.random_()                                   # random bits, as incompressible as logits
    out = torch.empty(-(-n // sm.STREAM_READ_TILE_BYTES), dtype=torch.int32, device="cuda")
    for _ in range(3):
        sm.stream_read(buf, out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        sm.stream_read(buf, out)
    ev[1].record()
    torch.cuda.synchronize()
    s = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    del buf
    return {"bytes": n, "reps": reps, "avg_us": round(s * 1e6, 2),
            "GBps": round(n / s / 1e9, 1), "kernel": "smcsd_stream_read"}


def reference_kernels(mib):
    """A plain kernel of known size on the same GPU: a device copy (reads and writes `mib`
    MiB), the calibration kernel for the HBM byte counters."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    reps = 5
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    copy_s = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    return {"bytes": n, "copy_GBps": round(2 * n / copy_s / 1e9, 1)}


def cpu_baseline(cfg, sets, budget_s, bonus="cdf"):
    """The oracle as it stands, on a bounded sample: verify on a subset of sequences (scaled
    to the full batch), resample and KV exchange on the whole batch."""
    import numpy as np
    import torch

    import oracle
    from workloads import synth

    B, N, K, S = cfg.B, cfg.N, cfg.K, cfg.S
    nsamp = min(S, 32)
    tgt, drf, toks, _ = sets[0]
    sel = torch.arange(nsamp, device=tgt.device)

    def host(x):
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).cpu().numpy().view(np.uint16)
        return x.cpu().numpy()

    th, dh, xh = host(tgt[sel]), host(drf[sel]), toks[sel].cpu().numpy()

    def sample(seconds):
        lw = np.zeros(nsamp, np.float32)
        kv = synth.initial_kv(cfg)
        T, rc, fl, top = kv["tables"], kv["refcounts"], kv["free_list"], int(kv["free_top"][0])
        L = int(kv["seq_len"])
        ident = np.tile(np.arange(N, dtype=np.int32), (B, 1))
        o = oracle.kv_reassign(ident, np.zeros(B, np.int32), T, cfg.block_size, L, K + 1, rc, fl,
                               top)
        rng = np.random.default_rng(0)
        t_verify = t_rest = 0.0
        reps = 0
        t_start = time.perf_counter()
        while reps < 2 or time.perf_counter() - t_start < seconds:
            a = time.perf_counter()
            v = oracle.verify_smc(th, dh, xh, float(np.float32(cfg.temperature)), cfg.alpha,
                                  cfg.rng_seed, reps, lw, bonus=bonus)
            b = time.perf_counter()
            lwfull = rng.normal(0, 2, (B, N)).astype(np.float32)
            r = oracle.resample(lwfull, float(np.float32(cfg.tau)), cfg.rng_seed, reps)
            L += K + 1
            o = oracle.kv_reassign(r["ancestors"], r["resampled"], o["tables"], cfg.block_size,
                                   L, K + 1, o["refcounts"], o["free_list"], o["free_top"])
            c = time.perf_counter()
            t_verify += b - a
            t_rest += c - b
            reps += 1
            if L + 2 * (K + 1) > cfg.M_cap * cfg.block_size:
                break
            del v
        return reps, t_verify / reps * (S / nsamp) + t_rest / reps

    cores = oracle.max_threads()
    reps, per_step = sample(budget_s)
    oracle.set_threads(1)
    reps1, per_step1 = sample(budget_s / 4)
    oracle.set_threads(cores)
    return {
        "value": round(1.0 / per_step, 4),
        "unit": "steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d reps: verify (%s bonus) on %d of %d sequences (scaled x%d), resample + KV "
                  "exchange on all %d prompts; fp64 C, OpenMP over rows" % (
                      reps, bonus, nsamp, S, S // nsamp, B),
        "single_thread_value": round(1.0 / per_step1, 4),
        "single_thread_reps": reps1,
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
