"""Pins of the oracle's exponential-race bonus sampler (CPU).

The race ("Speculative Sampling via Exponential Races" summary page, key design): every
token v gets an exponential clock E_v ~ Exp(1) run at rate p_v, and the first to finish,
argmin_v E_v / p_v, is a draw from p.  The oracle evaluates it as argmax_v (z_v - ln E_v)
on the tempered logits z = l / T, with E_v = -ln u_v and u_v from Philox stream
(index, t, tag 6 | (v div 4) << 8), word v mod 4.

Pins: the clocks follow Exp(1) (Kolmogorov-Smirnov) and are uncorrelated within and
across Philox blocks; the probability-domain definition argmin E_v / p_v with p from
scipy's softmax; chi-square law checks against softmax(z / T), masked tokens included;
one-hot, empty and tied rows; the SMC verify's bonus under the race rule, with the
log-weight of the power target checked against scipy's log_softmax.
"""
import numpy as np
import pytest
from scipy import special, stats

from tests import test_oracle_laws as laws


def test_race_clocks_are_exponential_and_uncorrelated(orc):
    seed, t = 1234, 77
    E = np.array([[orc.race_clock(seed, i, t, v) for v in range(16)] for i in range(2500)])
    assert np.all(E > 0.0)
    ks = stats.kstest(E.reshape(-1), "expon")
    assert ks.pvalue > 1e-4
    # neighbours inside one Philox block (v, v+1) and across blocks (v, v+4): no correlation
    for a, b in [(0, 1), (1, 2), (2, 3), (3, 4), (0, 4), (5, 9)]:
        r = np.corrcoef(E[:, a], E[:, b])[0, 1]
        assert abs(r) < 0.06, (a, b, r)
    # the step and the stream index change every clock
    assert orc.race_clock(seed, 3, t, 5) != orc.race_clock(seed, 3, t + 1, 5)
    assert orc.race_clock(seed, 3, t, 5) != orc.race_clock(seed, 4, t, 5)
    assert orc.race_clock(seed, 3, t, 5) != orc.race_clock(seed + 1, 3, t, 5)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_race_is_argmin_of_clock_over_probability(orc, T):
    """The race's definition in the probability domain (arrival time E_v / p_v, p from
    scipy's softmax of the tempered logits) picks the oracle's token."""
    rng = np.random.default_rng(3)
    n, V, seed, t = 40, 257, 5, 9
    rows = rng.normal(0, 2, (n, V)).astype(np.float32)
    rows[:, ::13] = -np.inf
    idx = rng.integers(0, 2**31, n).astype(np.int64)
    out = orc.race_sample(rows, T, seed, t, rng_index=idx)
    p = special.softmax(rows.astype(np.float64) / T, axis=1)
    for r in range(n):
        E = np.array([orc.race_clock(seed, int(idx[r]), t, v) for v in range(V)])
        with np.errstate(divide="ignore"):
            arrival = np.where(p[r] > 0, E / p[r], np.inf)
        want = int(np.argmin(arrival))
        assert out["tokens"][r] == want
        assert rows[r, want] > -np.inf
        assert out["margin"][r] > 0.0


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_race_law_chi_square(orc, T):
    row = np.array([[0.3, -1.2, 2.0, -np.inf, 0.3, 1.1, -0.5, 1.7, -3.0, 0.9, -np.inf, 0.0]],
                   np.float32)
    V = row.shape[1]
    n = 150000
    out = orc.race_sample(np.repeat(row, n, 0), T, 11, 2, rng_index=np.arange(n, dtype=np.int64))
    counts = np.bincount(out["tokens"], minlength=V).astype(np.float64)
    p = special.softmax(row[0].astype(np.float64) / T)
    assert counts[3] == 0 and counts[10] == 0        # masked tokens never win
    live = p > 0
    assert laws._chi2_pvalue(counts[live], p[live]) > 1e-4
    # the two equal logits (ids 0 and 4) win equally often
    assert stats.binomtest(int(counts[0]), int(counts[0] + counts[4]), 0.5).pvalue > 1e-4


def test_race_special_rows(orc):
    V = 40
    rows = np.full((3, V), -np.inf, np.float32)
    rows[0, 17] = 5.0                                 # one finite logit
    rows[1, :] = 0.0                                  # uniform: any id, margin finite
    out = orc.race_sample(rows, 1.0, 1, 0)
    assert out["tokens"][0] == 17 and out["margin"][0] == np.inf
    assert 0 <= out["tokens"][1] < V and 0.0 < out["margin"][1] < np.inf
    assert out["tokens"][2] == -1                     # nothing finite: no token
    # a uniform row's winner is the token with the smallest clock
    E = np.array([orc.race_clock(1, 1, 0, v) for v in range(V)])
    assert out["tokens"][1] == int(np.argmin(E))


@pytest.mark.parametrize("alpha", [1.0, 4.0])
def test_verify_race_bonus_is_the_race_and_reweights(orc, alpha):
    rng = np.random.default_rng(12)
    nseq, K, V, T = 16, 3, 211, 0.8
    tgt = rng.normal(0, 2, (nseq, K + 1, V)).astype(np.float32)
    drf = (tgt[:, :K] + rng.normal(0, 1, (nseq, K, V))).astype(np.float32)
    toks = rng.integers(0, V, (nseq, K)).astype(np.int32)
    lw0 = rng.normal(0, 1, nseq)
    idx = np.arange(100, 100 + nseq, dtype=np.int64)
    o = orc.verify_smc(tgt, drf, toks, T, alpha, 41, 6, lw0, rng_index=idx, bonus="race")
    c = orc.verify_smc(tgt, drf, toks, T, alpha, 41, 6, lw0, rng_index=idx, bonus="cdf")
    assert o["status"] == 0
    r = orc.race_sample(tgt[:, K], T, 41, 6, rng_index=idx)
    assert np.array_equal(o["tokens"][:, K], r["tokens"])
    assert np.array_equal(o["tokens"][:, :K], toks)
    assert not np.array_equal(o["tokens"][:, K], c["tokens"][:, K])   # a different draw
    lp = special.log_softmax(tgt.astype(np.float64) / T, axis=2)
    lq = special.log_softmax(drf.astype(np.float64) / T, axis=2)
    s = np.arange(nseq)[:, None]
    k = np.arange(K)[None, :]
    bonus = o["tokens"][:, K]
    want = lw0 + (alpha * lp[s, k, toks] - lq[s, k, toks]).sum(1) + \
        (alpha - 1.0) * lp[np.arange(nseq), K, bonus]
    assert np.max(np.abs(o["lw"] - want)) < 1e-12
    assert np.max(np.abs(o["logp"][:, K] - lp[np.arange(nseq), K, bonus])) < 1e-12
