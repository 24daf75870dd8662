"""Pins of the oracle's verify step (score, gather, bonus, reweight) - CPU only.

Each check compares the oracle with something other than itself:
  * scipy.special.logsumexp / log_softmax on the same rows (library routines),
  * closed forms (constant rows, masked rows, one-hot rows),
  * numpy.searchsorted on the cumulative distribution (textbook inverse CDF),
  * a chi-square test of the bonus tokens against the target probabilities,
  * the importance-sampling identity E_q[w] = prod_k sum_v p_k(v)^alpha, evaluated by
    enumerating every draft tuple on a tiny vocabulary.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy import special, stats

from tests.helpers import rocrand_probe


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- LSE
@pytest.mark.parametrize("T", [1.0, 0.8, 1.7])
@pytest.mark.parametrize("V", [1, 7, 8, 1000, 32000])
def test_row_lse_matches_scipy_fp32(orc, T, V):
    x = np.random.default_rng(V).normal(0, 3, V).astype(np.float32)
    got, st = orc.row_lse(x, T)
    assert st == 0
    ref = special.logsumexp(x.astype(np.float64) / T)
    assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("T", [1.0, 0.8])
def test_row_lse_matches_scipy_bf16(orc, T):
    x = np.random.default_rng(3).normal(0, 2, 128256).astype(np.float32)
    bits = bf16_bits(x)
    got, st = orc.row_lse(bits, T)
    ref = special.logsumexp(bf16_values(bits) / T)
    assert st == 0 and abs(got - ref) <= 1e-12 * abs(ref)


def test_row_lse_closed_forms(orc):
    # constant row c: LSE = c/T + ln V
    for c, T, V in [(0.0, 1.0, 8), (2.5, 0.8, 1000), (-7.0, 1.3, 128256)]:
        got, _ = orc.row_lse(np.full(V, c, np.float32), T)
        assert abs(got - (float(np.float32(c)) / T + np.log(V))) < 1e-12 * max(1, abs(got))
    # masked tokens carry probability 0: one finite logit among -inf gives that logit / T
    row = np.full(50, -np.inf, np.float32)
    row[17] = 3.0
    got, st = orc.row_lse(row, 0.5)
    assert st == 0 and got == 6.0


def test_row_lse_status_bits(orc):
    row = np.full(10, -np.inf, np.float32)
    _, st = orc.row_lse(row, 1.0)
    assert st == orc.ST_EMPTY_ROW
    row = np.zeros(10, np.float32)
    row[4] = np.nan
    _, st = orc.row_lse(row, 1.0)
    assert st == orc.ST_NAN_INPUT
    row[4] = np.inf
    _, st = orc.row_lse(row, 1.0)
    assert st == orc.ST_NAN_INPUT


def test_bf16_decoding_against_torch(orc):
    # single-element rows: LSE equals the decoded value / T
    vals = np.array([1.0, -2.0, 0.15625, 3.140625, -1e-3, 65280.0], np.float32)
    bits = bf16_bits(vals)
    dec = bf16_values(bits)
    for b, d in zip(bits, dec):
        got, _ = orc.row_lse(np.array([b], np.uint16), 1.0)
        assert got == d


# ----------------------------------------------------------------------------- verify
def _random_case(rng, nseq, K, V, dtype, scale=2.0, noise=1.0):
    t = rng.normal(0, scale, (nseq, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, noise, (nseq, K, V))).astype(np.float32)
    toks = rng.integers(0, V, (nseq, K)).astype(np.int32)
    if dtype == "bf16":
        return bf16_bits(t), bf16_bits(d), toks, bf16_values(bf16_bits(t)), bf16_values(bf16_bits(d))
    return t, d, toks, t.astype(np.float64), d.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("alpha", [1.0, 4.0])
def test_verify_gather_and_weights_vs_log_softmax(orc, dtype, alpha):
    rng = np.random.default_rng(11)
    nseq, K, V, T = 5, 3, 777, 0.8
    t, d, toks, tv, dv = _random_case(rng, nseq, K, V, dtype)
    lw_in = rng.normal(0, 1, nseq).astype(np.float32)
    out = orc.verify_smc(t, d, toks, T, alpha, seed=5, t=9, lw_in=lw_in)
    assert out["status"] == 0
    lsp = special.log_softmax(tv / T, axis=-1)
    lsq = special.log_softmax(dv / T, axis=-1)
    for s in range(nseq):
        for k in range(K):
            assert abs(out["logp"][s, k] - lsp[s, k, toks[s, k]]) < 1e-12
            assert abs(out["logq"][s, k] - lsq[s, k, toks[s, k]]) < 1e-12
            assert out["tokens"][s, k] == toks[s, k]
        b = out["tokens"][s, K]
        assert 0 <= b < V
        assert abs(out["logp"][s, K] - lsp[s, K, b]) < 1e-12
        lse_t = special.logsumexp(tv[s] / T, axis=-1)
        lse_d = special.logsumexp(dv[s] / T, axis=-1)
        assert np.allclose(out["lse"][s], np.concatenate([lse_t, lse_d]), rtol=1e-13, atol=0)
    # K+1 tokens always
    assert out["tokens"].shape == (nseq, K + 1) and np.all(out["tokens"] >= 0)


@pytest.mark.skipif(not rocrand_probe.available(), reason="hipcc / rocRAND headers not present")
def test_bonus_inverse_cdf_vs_searchsorted(orc):
    rng = np.random.default_rng(21)
    nseq, K, V, T = 16, 2, 3001, 1.0
    t, d, toks, tv, _ = _random_case(rng, nseq, K, V, "f32", scale=1.5)
    seed, step = 0xABCDEF12345, 77
    idx = np.arange(100, 100 + nseq, dtype=np.int64)
    out = orc.verify_smc(t, d, toks, T, 1.0, seed, step, np.zeros(nseq, np.float32), rng_index=idx)
    ctr = np.array([[g, step, 0, 1] for g in idx], dtype=np.uint32)
    key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32), (nseq, 1))
    blocks = rocrand_probe.philox_blocks(ctr, key)
    for s in range(nseq):
        u = float(int(blocks[s, 0]) >> 8) / (1 << 24)
        assert out["u"][s] == u
        p = special.softmax(tv[s, K] / T)
        cdf = np.cumsum(p)
        ref = int(np.searchsorted(cdf, u, side="right"))
        if out["margin"][s] > 1e-12:
            assert out["tokens"][s, K] == ref


def test_bonus_one_hot_and_masked(orc):
    V, K = 64, 1
    t = np.full((3, K + 1, V), -np.inf, np.float32)
    d = np.zeros((3, K, V), np.float32)
    t[:, 0, :] = 0.0
    t[0, K, 5] = 1.0
    t[1, K, 63] = -3.0
    t[2, K, [0, 9]] = 0.0          # two tokens, p = 1/2 each; everything else masked
    toks = np.zeros((3, K), np.int32)
    for step in range(40):
        out = orc.verify_smc(t, d, toks, 1.0, 1.0, 3, step, np.zeros(3, np.float32))
        assert out["tokens"][0, K] == 5 and out["tokens"][1, K] == 63
        assert out["tokens"][2, K] in (0, 9)
        assert out["logp"][2, K] == pytest.approx(np.log(0.5), abs=1e-15)


def test_bonus_chi_square_against_target(orc):
    """Bonus tokens over many rounds follow softmax(target row K / T)."""
    rng = np.random.default_rng(5)
    V, K, T = 8, 2, 0.9
    t = rng.normal(0, 1, (1, K + 1, V)).astype(np.float32)
    d = rng.normal(0, 1, (1, K, V)).astype(np.float32)
    toks = np.zeros((1, K), np.int32)
    n = 30000
    tt = np.repeat(t, 200, axis=0)
    dd = np.repeat(d, 200, axis=0)
    tk = np.repeat(toks, 200, axis=0)
    counts = np.zeros(V)
    for step in range(n // 200):
        out = orc.verify_smc(tt, dd, tk, T, 1.0, 42, step, np.zeros(200, np.float32),
                             rng_index=np.arange(200, dtype=np.int64))
        counts += np.bincount(out["tokens"][:, K], minlength=V)
    p = special.softmax(t[0, K].astype(np.float64) / T)
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-4


@pytest.mark.parametrize("alpha", [1.0, 4.0])
def test_weight_identity_by_enumeration(orc, alpha):
    """Importance weights are proper for the unnormalised target prod_k p_k^alpha:
    sum over every draft tuple x of q(x) * exp(incr(x)) = prod_{k<=K} sum_v p_k(v)^alpha.
    Row K has two tokens of probability 1/2 (others masked) so the bonus term
    (alpha-1)*log p_K is deterministic; it contributes sum_b p_K(b)^alpha = 2^(1-alpha)."""
    rng = np.random.default_rng(8)
    V, K, T = 6, 2, 1.0
    t = rng.normal(0, 1, (1, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 0.7, (1, K, V))).astype(np.float32)
    t[0, K, :] = -np.inf
    t[0, K, [1, 4]] = 0.3
    tuples = np.array(list(itertools.product(range(V), repeat=K)), dtype=np.int32)
    n = len(tuples)
    out = orc.verify_smc(np.repeat(t, n, 0), np.repeat(d, n, 0), tuples, T, alpha, 1, 2,
                         np.zeros(n, np.float32))
    q = special.softmax(d[0].astype(np.float64) / T, axis=-1)
    qx = np.prod([q[k, tuples[:, k]] for k in range(K)], axis=0)
    lhs = float(np.sum(qx * np.exp(out["lw"])))
    p = special.softmax(t[0].astype(np.float64) / T, axis=-1)
    rhs = float(np.prod([np.sum(p[k] ** alpha) for k in range(K + 1)]))
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_weight_accumulates_on_input(orc):
    rng = np.random.default_rng(9)
    t, d, toks, _, _ = _random_case(rng, 4, 3, 50, "f32")
    a = orc.verify_smc(t, d, toks, 1.0, 1.0, 1, 1, np.zeros(4, np.float32))
    b = orc.verify_smc(t, d, toks, 1.0, 1.0, 1, 1, np.full(4, 2.5, np.float32))
    assert np.allclose(b["lw"] - a["lw"], 2.5, atol=1e-14)


def test_verify_status_propagates(orc):
    t = np.zeros((2, 2, 16), np.float32)
    d = np.zeros((2, 1, 16), np.float32)
    t[1, 0, 3] = np.nan
    out = orc.verify_smc(t, d, np.zeros((2, 1), np.int32), 1.0, 1.0, 0, 0, np.zeros(2, np.float32))
    assert out["status"] & orc.ST_NAN_INPUT
    t[1, 0, 3] = 0
    d[0, 0, :] = -np.inf
    out = orc.verify_smc(t, d, np.zeros((2, 1), np.int32), 1.0, 1.0, 0, 0, np.zeros(2, np.float32))
    assert out["status"] & orc.ST_EMPTY_ROW
