"""Pins of the oracle's draft-side sampler and of the verify with precomputed log q (CPU).

The draft model proposes each token from its own tempered distribution (SMC explainers,
section 2, "Extend").  The oracle's draft_sample draws it by inverse CDF with the uniform
of stream (g, step, tag 5 | pos << 8) and emits log q of the draw; verify_smc can take
those log q values instead of reading the draft rows.  Pins: the textbook inverse CDF
(np.searchsorted on np.cumsum), scipy's log_softmax, a chi-square law check, masked and
one-hot rows, and the equality of the two verify paths.
"""
import numpy as np
import pytest
from scipy import special, stats

V_SMALL = 37


def _rows(rng, n, V, dtype):
    x = rng.normal(0, 2, (n, V)).astype(np.float32)
    if dtype == "bf16":
        b = (x.view(np.uint32) >> 16).astype(np.uint16)
        return b, (b.astype(np.uint32) << 16).view(np.float32)
    return x, x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.8, 1.0, 1.7])
def test_draft_sample_is_the_textbook_inverse_cdf(orc, dtype, T):
    rng = np.random.default_rng(17)
    n, seed, t, pos = 300, 99, 12345, 3
    rows, vals = _rows(rng, n, V_SMALL, dtype)
    idx = rng.integers(0, 2**31, n).astype(np.int64)
    out = orc.draft_sample(rows, T, seed, t, pos, rng_index=idx)
    assert out["status"] == 0
    p = special.softmax(vals.astype(np.float64) / T, axis=1)
    for r in range(n):
        u = orc.uniform(seed, int(idx[r]), t, 5 | (pos << 8), 0)
        want = int(np.searchsorted(np.cumsum(p[r]), u, side="right"))
        assert out["tokens"][r] == want
        ref = special.log_softmax(vals[r].astype(np.float64) / T)[want]
        assert abs(out["logq"][r] - ref) < 1e-12


def test_draft_sample_law_chi_square(orc):
    rng = np.random.default_rng(5)
    row = rng.normal(0, 1, (1, 12)).astype(np.float32)
    n = 200000
    rows = np.repeat(row, n, 0)
    out = orc.draft_sample(rows, 0.9, 7, 0, 1, rng_index=np.arange(n, dtype=np.int64))
    counts = np.bincount(out["tokens"], minlength=12)
    p = special.softmax(row[0].astype(np.float64) / 0.9)
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_draft_sample_masked_and_one_hot_rows(orc):
    V = 16
    rows = np.full((3, V), -np.inf, np.float32)
    rows[0, 5] = 0.0                        # one finite logit: always that token, log q = 0
    rows[1, [2, 9]] = [1.0, 1.0]             # two equal logits: one of them, log q = -ln 2
    rows[2, :] = np.linspace(-3, 3, V)       # all finite
    rows[2, ::2] = -np.inf                   # masked tokens never drawn
    for t in range(40):
        out = orc.draft_sample(rows, 1.0, 3, t, 0)
        assert out["status"] == 0
        assert out["tokens"][0] == 5 and out["logq"][0] == 0.0
        assert out["tokens"][1] in (2, 9) and abs(out["logq"][1] + np.log(2.0)) < 1e-15
        assert out["tokens"][2] % 2 == 1


def test_verify_with_draft_logq_equals_reading_the_draft_rows(orc):
    """Reweighting with the log q the draft sampler emitted matches the verify that reads
    the draft rows: same tokens, log-weights within rounding."""
    rng = np.random.default_rng(8)
    nseq, K, V, T = 24, 4, 301, 0.8
    tgt = rng.normal(0, 2, (nseq, K + 1, V)).astype(np.float32)
    drf = (tgt[:, :K] + rng.normal(0, 1, (nseq, K, V))).astype(np.float32)
    toks = np.zeros((nseq, K), np.int32)
    logq = np.zeros((nseq, K))
    for k in range(K):
        d = orc.draft_sample(drf[:, k], T, 21, 4, k, rng_index=np.arange(nseq, dtype=np.int64))
        toks[:, k] = d["tokens"]
        logq[:, k] = d["logq"]
    lw0 = rng.normal(0, 1, nseq).astype(np.float32)
    a = orc.verify_smc(tgt, drf, toks, T, 1.0, 21, 5, lw0)
    b = orc.verify_smc(tgt, None, toks, T, 1.0, 21, 5, lw0, logq_in=logq)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.max(np.abs(a["lw"] - b["lw"])) < 1e-12
    assert np.max(np.abs(a["logq"] - b["logq"])) < 1e-12
    assert np.all(np.isnan(b["lse"][:, K + 1:]))
    assert np.array_equal(a["lse"][:, :K + 1], b["lse"][:, :K + 1])
