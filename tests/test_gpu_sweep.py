"""The temperature sweep (SpS tokens per round against SMC-SD's fixed K+1, mean ESS / N,
resample rate; SMC explainers, section 4: robustness to the sampling temperature) checked
against the oracle round by round, in lock-step: every round's GPU inputs (the log-weights
at the round's start) are replayed through the oracle, and

  * every sequence's bonus token and log-weight after the verify (1e-4), every prompt's ESS
    (1e-6 relative), resampling decision and ancestors, and every SpS sequence's emitted
    tokens and count must match, except at decisions whose oracle margin is below 1e-6
    (flagged and counted);
  * the sweep's reported figures must equal the same figures formed from the oracle's
    outputs (the SpS count and resample rate exactly when no flagged decision went the
    other way; the mean ESS / N to 1e-6 relative).

A downsized workload (B = 3 prompts of N = 16 at V = 20011, Zipf logits, K = 4) at three
temperatures keeps the oracle's work to seconds while rows still span several tiles.
"""
import numpy as np
import pytest
import torch

import oracle
from smc_verification_resampling_amd import sweep
from tests import gpu_harness as H
from workloads import configs as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def test_temperature_sweep_matches_the_oracle():
    cfg0 = C.C3.scaled(name="c3_sweep_small", B=3, V=20011, n_sets=2)
    temps, rounds = [0.6, 1.0, 1.8], 8
    B, N, K = cfg0.B, cfg0.N, cfg0.K
    st = H.Stats()
    agg = {}

    def observe(info):
        cfg, t = info["cfg"], info["t"]
        T32, tau32 = float(np.float32(cfg.temperature)), float(np.float32(cfg.tau))
        th, dh = H.host_logits(info["target"]), H.host_logits(info["draft"])
        x = info["draft_tokens"].cpu().numpy()
        o = oracle.verify_smc(th, dh, x, T32, float(np.float32(cfg.alpha)), cfg.rng_seed, t,
                              info["lw_in"].cpu().numpy())
        gtok, glw = info["tokens"].cpu().numpy(), info["lw_post"].cpu().numpy()
        for g in range(B * N):
            same = gtok[g, K] == o["tokens"][g, K]
            st.decision(same, o["margin"][g], "bonus g=%d t=%d T=%g" % (g, t, cfg.temperature))
            if same:
                st.max_dlw = max(st.max_dlw, abs(float(glw[g]) - o["lw"][g]))
        r = oracle.resample(info["lw_post"].cpu().numpy().reshape(B, N), tau32, cfg.rng_seed, t)
        gres, gess = info["resampled"].cpu().numpy(), info["ess"].cpu().numpy()
        ganc = info["ancestors"].cpu().numpy()
        for b in range(B):
            if r["ess"][b] > 0:
                st.max_rel_ess = max(st.max_rel_ess, abs(gess[b] - r["ess"][b]) / r["ess"][b])
            same = gres[b] == r["resampled"][b]
            st.decision(same, r["margin_ess"][b], "resample b=%d t=%d" % (b, t))
            if same and gres[b]:
                for i in range(N):
                    st.decision(ganc[b, i] == r["ancestors"][b, i], r["margin_pos"][b, i],
                                "ancestor b=%d i=%d t=%d" % (b, i, t))
        src = np.arange(B) * N
        s = oracle.verify_sps(th[src], dh[src], x[src], T32, cfg.rng_seed, t,
                              rng_index=np.arange(B))
        gst, gnum = info["sps_tokens"].cpu().numpy(), info["sps_num"].cpu().numpy()
        for b in range(B):
            same = gnum[b] == s["num_tokens"][b] and np.array_equal(gst[b], s["tokens"][b])
            st.decision(same, min(s["margin_accept"][b], s["margin_final"][b]), "sps b=%d t=%d" % (b, t))
        a = agg.setdefault(cfg.temperature, {"ess": 0.0, "res": 0, "sps": 0, "flag_miss": 0})
        a["ess"] += float(r["ess"].sum())
        a["res"] += int(r["resampled"].sum())
        a["sps"] += int(s["num_tokens"].sum())
        a["flag_miss"] = st.flagged_mismatch

    figs = sweep.sweep(cfg0, temps, rounds, observer=observe)
    msg = st.assert_ok()
    print("[sweep vs oracle]", msg, flush=True)
    assert st.decisions > rounds * len(temps) * (B * N + B)
    n = rounds * B
    for d in figs:
        a = agg[d["temperature"]]
        assert d["status"] == 0
        assert d["smc_tokens_per_round"] == K + 1
        assert abs(d["smc_mean_ess_fraction"] - round(a["ess"] / (n * N), 4)) <= 1e-4
        if st.flagged_mismatch == 0:
            assert d["sps_tokens_per_round"] == round(a["sps"] / n, 4)
            assert d["smc_resample_rate"] == round(a["res"] / n, 4)
    # the sweep moves with the temperature: SpS keeps more drafts as the distributions flatten
    sps = [d["sps_tokens_per_round"] for d in figs]
    assert sps[0] < sps[-1]
