"""Temperature sweep: SpS tokens per round against SMC-SD's fixed K+1, on the same logits.

The SMC explainers (section 2 and the experiments) contrast the two verifiers: SpS stops
at the first rejected draft token, so its tokens per round vary with how closely the
draft tracks the target (which the sampling temperature changes), while an SMC-SD round
always emits K+1 tokens per particle and pays instead in weight degeneracy (ESS) and
resampling.  This sweep measures both on seeded synthetic logits with the shapes of a
workload, with every step run by the library's kernels:

  * SpS: mean tokens emitted per round by the modified-rejection verify on particle 0 of
    every prompt;
  * SMC-SD: mean ESS / N before the resampling decision and the fraction of prompts that
    resample, over consecutive rounds (weights carried between rounds, reset on a
    resample).

Run:  python -m smc_verification_resampling_amd.sweep [--workload c3_batched]
          [--temperatures 0.5,0.8,1.0,1.5,2.0] [--rounds 50]
Prints one JSON line per temperature.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys


def sweep(cfg0, temperatures, rounds, observer=None):
    """The sweep over `temperatures` on cfg0's workload (its n_sets logit sets, generated
    once): one dict of figures per temperature.  observer(info), if given, is called after
    every round with that round's inputs and outputs (device tensors, the stream
    synchronised): the log-weights before the verify, after it and after the resample,
    the ESS, decisions and ancestors, and the SpS tokens and counts."""
    import torch

    import smc_verification_resampling_amd as sm
    from workloads import synth

    B, N, K, V, S = cfg0.B, cfg0.N, cfg0.K, cfg0.V, cfg0.S
    dev = "cuda"
    base = synth.zipf_base(cfg0, dev) if cfg0.target_kind == "zipf" else None
    logits = [synth.make_logit_set(cfg0, s, dev, base) for s in range(cfg0.n_sets)]
    i32 = dict(dtype=torch.int32, device=dev)
    ws_smc = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    ws_sps = sm.alloc_workspace(sm.OP_VERIFY_SPS, B, 1, K, V)
    results = []
    for temp in temperatures:
        cfg = dataclasses.replace(cfg0, temperature=temp)
        drafts = [synth.sample_draft_tokens(cfg, d, s) for s, (_, d) in enumerate(logits)]
        lw = torch.zeros(S, dtype=torch.float32, device=dev)
        tok = torch.zeros((S, K + 1), **i32)
        stok = torch.zeros((B, K + 1), **i32)
        num = torch.zeros(B, **i32)
        st = torch.zeros(1, **i32)
        anc = torch.zeros((B, N), **i32)
        ess = torch.zeros(B, dtype=torch.float32, device=dev)
        res = torch.zeros(B, **i32)
        ess_sum = torch.zeros((), dtype=torch.float64, device=dev)
        res_sum = torch.zeros((), dtype=torch.float64, device=dev)
        sps_sum = torch.zeros((), dtype=torch.float64, device=dev)
        for t in range(rounds):
            tgt, drf = logits[t % cfg.n_sets]
            x = drafts[t % cfg.n_sets]
            lw_in = lw.clone() if observer else None
            sm.verify(tgt, drf, x, B, N, K, V, temp, cfg.alpha, sm.MODE_SMC, cfg.rng_seed, t, tok, st,
                      ws_smc, log_weights=lw)
            lw_post = lw.clone() if observer else None
            sm.resample(lw.view(B, N), B, N, cfg.tau, cfg.rng_seed, t, anc, ess, res, st)
            sm.verify(tgt, drf, x, B, 1, K, V, temp, 1.0, sm.MODE_SPS, cfg.rng_seed, t, stok, st,
                      ws_sps, out_num_tokens=num, seq_step=N)
            ess_sum += ess.double().sum()
            res_sum += res.double().sum()
            sps_sum += num.double().sum()
            if observer:
                torch.cuda.synchronize()
                observer(dict(cfg=cfg, t=t, target=tgt, draft=drf, draft_tokens=x, lw_in=lw_in,
                              lw_post=lw_post, lw_out=lw.clone(), tokens=tok.clone(), ess=ess.clone(),
                              resampled=res.clone(), ancestors=anc.clone(), sps_tokens=stok.clone(),
                              sps_num=num.clone()))
        torch.cuda.synchronize()
        n = rounds * B
        results.append({
            "workload": cfg.name, "temperature": temp, "rounds": rounds, "prompts": B,
            "particles": N, "K": K,
            "sps_tokens_per_round": round(float(sps_sum) / n, 4),
            "smc_tokens_per_round": K + 1,
            "smc_mean_ess_fraction": round(float(ess_sum) / (n * N), 4),
            "smc_resample_rate": round(float(res_sum) / n, 4),
            "status": int(st.cpu()[0]),
        })
    return results


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c3_batched")
    ap.add_argument("--temperatures", default="0.5,0.8,1.0,1.5,2.0")
    ap.add_argument("--rounds", type=int, default=50)
    ap.add_argument("--sets", type=int, default=2)
    args = ap.parse_args(argv)

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import configs

    base_cfg = configs.get(args.workload)
    cfg0 = dataclasses.replace(base_cfg, n_sets=min(base_cfg.n_sets, args.sets))
    for d in sweep(cfg0, [float(t) for t in args.temperatures.split(",")], args.rounds):
        print(json.dumps(d), flush=True)


if __name__ == "__main__":
    main()
