"""Distribution-level checks of the GPU path on a tiny vocabulary (V = 8, K = 2).

The same construction as the oracle's law pins (prefix-dependent seeded logit tables,
8^3 one-round continuations), run through the library instead of the oracle:

* SMC-SD: one round over many independent prompts with N particles, resampling forced
  (tau > 1), a uniformly chosen output particle -> the sampling-importance-resampling law
  P_N, computed exactly by enumeration (SMC explainers, section 2: importance-weighted
  resampling).  alpha = 1 and the power target alpha = 4; the bonus drawn by inverse CDF
  and by the exponential race.
* SpS: rounds of the modified-rejection verify until three tokens are emitted -> the
  target law (the speculative-sampling notes: the output follows the target exactly).
* Many particles: the same SIR round at N = 8, 16, 64 against P_N by Rao-Blackwellised
  Monte Carlo, and the decay of the sampler's distance to the target with N (SMC
  explainers, section 3: L1 error O(1/sqrt N), bias O(1/N)): the empirical L1 distance of
  the GPU's samples and an unbiased estimate of their squared L2 distance, fitted on a
  log-log scale beside the analytic slopes of ||P_N - pi||.

Each GPU call draws its randomness from (seed, step, sequence index); the chi-square
tests use p > 1e-4 on merged cells, like the oracle's pins.
"""
import numpy as np
import pytest
import torch

import smc_verification_resampling_amd as sm
from tests import test_oracle_laws as L

pytestmark = pytest.mark.gpu

V, K = L.V, L.K


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("mode", [sm.MODE_SMC, sm.MODE_SMC_RACE], ids=["cdf_bonus", "race_bonus"])
@pytest.mark.parametrize("N,alpha", [(4, 1.0), (3, 4.0)])
def test_gpu_smc_round_follows_sir_law(N, alpha, mode):
    tgt, drf = L._tables(31337)
    P, PI = L._sir_law(tgt, drf, N, alpha)
    runs, seed = 60000, 11
    rng = np.random.default_rng(seed)
    S = runs * N
    x1 = L._sample_rows(rng, np.repeat(L._softmax(drf[0][[0]]), S, 0))
    x2 = L._sample_rows(rng, L._softmax(drf[1][x1]))
    t_rows = np.stack([np.repeat(tgt[0][[0]], S, 0), tgt[1][x1], tgt[2][x1 * V + x2]], axis=1)
    d_rows = np.stack([np.repeat(drf[0][[0]], S, 0), drf[1][x1]], axis=1)
    toks = np.stack([x1, x2], axis=1).astype(np.int32)
    t_d = torch.from_numpy(np.ascontiguousarray(t_rows, np.float32)).cuda()
    d_d = torch.from_numpy(np.ascontiguousarray(d_rows, np.float32)).cuda()
    x_d = torch.from_numpy(toks).cuda()
    lw = torch.zeros(S, dtype=torch.float32, device="cuda")
    out, st = _i32(S, K + 1), _i32(1)
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, runs, N, K, V)
    sm.verify(t_d, d_d, x_d, runs, N, K, V, 1.0, alpha, mode, seed, 0, out, st, ws,
              log_weights=lw)
    anc, ess, res = _i32(runs, N), torch.zeros(runs, device="cuda"), _i32(runs)
    sm.resample(lw.view(runs, N), runs, N, 2.0, seed, 0, anc, ess, res, st)   # tau > 1: always
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == 0
    assert bool((res == 1).all())
    y = out.cpu().numpy()
    assert np.array_equal(y[:, :K], toks) and (y[:, K] >= 0).all() and (y[:, K] < V).all()
    pick = rng.integers(0, N, runs)
    g = np.arange(runs) * N + anc.cpu().numpy()[np.arange(runs), pick]
    ys = y[g, 0] * 64 + y[g, 1] * 8 + y[g, 2]
    counts = np.bincount(ys, minlength=V ** 3).astype(np.float64)
    assert L._chi2_pvalue(counts, P) > 1e-4
    assert np.abs(P - PI).sum() > 0.02     # the test can tell P_N from the target


def test_gpu_sps_law_equals_target():
    tgt, drf = L._tables(2024)
    pi = L._target_law(tgt)
    rng = np.random.default_rng(98)
    runs = 60000
    emitted = [[] for _ in range(runs)]
    code = np.zeros(runs, np.int64)
    length = np.zeros(runs, np.int64)
    st = _i32(1)
    rnd = 0
    active = np.arange(runs)
    while len(active):
        len_at_start = length[active].copy()
        for d in (0, 1, 2):
            grp = active[len_at_start == d]
            if not len(grp):
                continue
            c0 = code[grp]
            x1 = L._sample_rows(rng, L._softmax(drf[d][c0]))
            c1 = c0 * V + x1
            x2 = L._sample_rows(rng, L._softmax(drf[d + 1][c1]))
            c2 = c1 * V + x2
            t_rows = np.stack([tgt[d][c0], tgt[d + 1][c1], tgt[d + 2][c2]], axis=1)
            d_rows = np.stack([drf[d][c0], drf[d + 1][c1]], axis=1)
            toks = np.stack([x1, x2], axis=1).astype(np.int32)
            n = len(grp)
            out, num = _i32(n, K + 1), _i32(n)
            ws = sm.alloc_workspace(sm.OP_VERIFY_SPS, n, 1, K, V)
            # distinct (step, index) per round and depth group: independent draws
            sm.verify(torch.from_numpy(np.ascontiguousarray(t_rows, np.float32)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(d_rows, np.float32)).cuda(),
                      torch.from_numpy(toks).cuda(), n, 1, K, V, 1.0, 1.0, sm.MODE_SPS, 77,
                      rnd * 3 + d, out, st, ws, out_num_tokens=num)
            o, nt = out.cpu().numpy(), num.cpu().numpy()
            for j, r in enumerate(grp):
                k = int(nt[j])
                new = o[j, :k].tolist()
                assert 1 <= k <= K + 1 and all(0 <= v < V for v in new)
                emitted[r].extend(new)
                for v in new:
                    if length[r] < 3:
                        code[r] = code[r] * V + v
                        length[r] += 1
        rnd += 1
        active = np.array([r for r in active if length[r] < 3], dtype=np.int64)
    assert int(st.cpu()[0]) == 0
    ys = np.array([e[0] * 64 + e[1] * 8 + e[2] for e in emitted])
    counts = np.bincount(ys, minlength=V ** 3).astype(np.float64)
    assert L._chi2_pvalue(counts, pi) > 1e-4


def test_temperature_sweep_runs_and_reports_ranges(capsys):
    """The temperature sweep (SpS tokens per round vs SMC-SD's K+1, ESS, resample rate) on
    the tiny workload: every reported figure inside its range."""
    import json

    from smc_verification_resampling_amd import sweep

    sweep.main(["--workload", "c1_tiny", "--temperatures", "0.7,1.3", "--rounds", "6",
                "--sets", "2"])
    lines = [json.loads(x) for x in capsys.readouterr().out.strip().splitlines()]
    assert [d["temperature"] for d in lines] == [0.7, 1.3]
    for d in lines:
        assert d["status"] == 0
        assert 1.0 <= d["sps_tokens_per_round"] <= d["K"] + 1
        assert d["smc_tokens_per_round"] == d["K"] + 1
        assert 0.0 < d["smc_mean_ess_fraction"] <= 1.0
        assert 0.0 <= d["smc_resample_rate"] <= 1.0


def _gpu_sir_counts(tgt, drf, N, runs, seed, alpha=1.0, mode=sm.MODE_SMC):
    """Counts of the 512 continuations from one SMC-SD round on the GPU: drafts drawn with
    torch on the device (no host copies of the rows), verify, forced resampling, and one
    uniformly chosen output particle per prompt."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    S = runs * N
    t = {d: torch.from_numpy(tgt[d]).cuda() for d in range(3)}
    q0 = torch.softmax(torch.from_numpy(drf[0][0]).double().cuda(), -1)
    q1 = torch.softmax(torch.from_numpy(drf[1]).double().cuda(), -1)
    x1 = torch.multinomial(q0.float(), S, replacement=True, generator=g)
    u = torch.rand(S, 1, generator=g, device="cuda", dtype=torch.float64)
    x2 = (torch.cumsum(q1, -1)[x1] < u).sum(1).clamp(max=V - 1)
    t_rows = torch.stack([t[0][0].expand(S, V), t[1][x1], t[2][x1 * V + x2]], 1).contiguous()
    d0 = torch.from_numpy(drf[0][0]).cuda()
    d1 = torch.from_numpy(drf[1]).cuda()
    d_rows = torch.stack([d0.expand(S, V), d1[x1]], 1).contiguous()
    toks = torch.stack([x1, x2], 1).to(torch.int32).contiguous()
    del u
    lw = torch.zeros(S, dtype=torch.float32, device="cuda")
    out, st = _i32(S, K + 1), _i32(1)
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, runs, N, K, V)
    sm.verify(t_rows, d_rows, toks, runs, N, K, V, 1.0, alpha, mode, seed, 0, out, st, ws,
              log_weights=lw)
    del t_rows, d_rows, ws
    anc, ess, res = _i32(runs, N), torch.zeros(runs, device="cuda"), _i32(runs)
    sm.resample(lw.view(runs, N), runs, N, 2.0, seed, 0, anc, ess, res, st)   # tau > 1: always
    pick = torch.randint(0, N, (runs,), generator=g, device="cuda")
    r = torch.arange(runs, device="cuda")
    y = out[r * N + anc[r, pick].long()].long()
    assert int(st.cpu()[0]) == 0 and bool((res == 1).all())
    assert bool((y[:, :K] == toks[r * N + anc[r, pick].long()].long()).all())
    ys = y[:, 0] * 64 + y[:, 1] * 8 + y[:, 2]
    return torch.bincount(ys, minlength=V ** 3).double().cpu().numpy()


@pytest.mark.parametrize("N", [8, 16, 64])
def test_gpu_smc_round_follows_sir_law_many_particles(N):
    tgt, drf = L._tables(31337)
    P, PI = L._sir_law_mc(tgt, drf, N, 400000, seed=1000 + N)
    P = P / P.sum()
    counts = _gpu_sir_counts(tgt, drf, N, 100000, seed=300 + N)
    assert L._chi2_pvalue(counts, P) > 1e-4
    if N == 8:
        assert L._chi2_pvalue(counts, PI) < 1e-12   # and it can tell P_8 from the target


def test_gpu_error_decays_with_particles():
    """||emp_N - pi||_1 of the GPU's samples and an unbiased estimate of ||P_N - pi||_2^2
    from them (sum c(c-1)/(n(n-1)) - 2 sum pi c / n + sum pi^2), N = 1 .. 64, 10^6 prompts
    each; log-log slopes printed beside the analytic ones.  The L1 fit stops at N = 8,
    where the bias still exceeds the sampling noise of 10^6 draws (~0.015); the L2 fit
    stops at N = 32 for the same reason."""
    tgt, drf = L._tables(31337)
    pi = L._target_law(tgt)
    Ns = [1, 2, 4, 8, 16, 32, 64]
    n = 1000000
    l1_emp, l2_emp, l1_ana, l2_ana = [], [], [], []
    for N in Ns:
        if N <= 4:
            P, PI = L._sir_law(tgt, drf, N, 1.0)
        else:
            P, PI = L._sir_law_mc(tgt, drf, N, 200000, seed=N)
        assert np.allclose(PI, pi)
        c = _gpu_sir_counts(tgt, drf, N, n, seed=500 + N)
        assert c.sum() == n
        l1_emp.append(np.abs(c / n - pi).sum())
        l2_emp.append(np.sum(c * (c - 1)) / (n * (n - 1)) - 2 * np.sum(pi * c) / n + np.sum(pi ** 2))
        l1_ana.append(np.abs(P - PI).sum())
        l2_ana.append(np.sum((P - PI) ** 2))
    logN = np.log(Ns)
    s_l1_emp = np.polyfit(logN[:4], np.log(l1_emp[:4]), 1)[0]
    s_l1_ana = np.polyfit(logN, np.log(l1_ana), 1)[0]
    s_l2_emp = np.polyfit(logN[:6], 0.5 * np.log(np.maximum(l2_emp[:6], 1e-30)), 1)[0]
    s_l2_ana = np.polyfit(logN, 0.5 * np.log(l2_ana), 1)[0]
    print("\n[error decay] N = %s" % Ns)
    print("[error decay] L1 GPU samples  %s  slope(N<=8) %.3f" % (
        " ".join("%.4f" % x for x in l1_emp), s_l1_emp))
    print("[error decay] L1 analytic     %s  slope %.3f" % (
        " ".join("%.4f" % x for x in l1_ana), s_l1_ana))
    print("[error decay] L2 GPU (unbiased) %s  slope(N<=32) %.3f" % (
        " ".join("%.2e" % np.sqrt(max(x, 0.0)) for x in l2_emp), s_l2_emp))
    print("[error decay] L2 analytic       %s  slope %.3f" % (
        " ".join("%.2e" % np.sqrt(x) for x in l2_ana), s_l2_ana), flush=True)
    assert s_l1_emp <= -0.4 and s_l1_ana <= -0.4
    assert s_l2_emp <= -0.4 and s_l2_ana <= -0.4
    # each unbiased L2 estimate agrees with the analytic value within its sampling error
    for e, a in zip(l2_emp[:6], l2_ana[:6]):
        assert abs(e - a) <= 0.25 * a + 6.0 / n, (e, a)
