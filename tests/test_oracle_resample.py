"""Pins of the oracle's ESS + systematic resampling step - CPU only.

Closed forms for ESS, numpy.searchsorted for the systematic rule (textbook), the
offspring-count bounds floor/ceil(N W_j), and a Monte Carlo check that the expected
offspring count is N W_j (unbiasedness: the resampled population still represents
the weighted one, as the pages require when high-weight particles are copied and
low-weight ones dropped).
"""
import numpy as np
import pytest

from tests.helpers import rocrand_probe


def _ess_ref(lw):
    lw = np.asarray(lw, np.float64)
    w = np.exp(lw - lw.max())
    return min(max(w.sum() ** 2 / (w ** 2).sum(), 1.0), len(lw))


def test_ess_closed_forms(orc):
    N = 16
    out = orc.resample(np.zeros((1, N), np.float32), 0.5, 1, 0)
    assert out["ess"][0] == N and out["resampled"][0] == 0
    lw = np.full((1, N), -np.inf, np.float32)
    lw[0, 3] = 1.0
    out = orc.resample(lw, 0.5, 1, 0)
    assert out["ess"][0] == 1.0 and out["resampled"][0] == 1
    assert np.all(out["ancestors"][0] == 3)
    # two-level: k weights e^a, N-k weights 1  ->  (k e^a + N - k)^2 / (k e^{2a} + N - k)
    for k, a in [(1, 2.0), (4, 1.0), (15, -3.0)]:
        lw = np.zeros((1, N), np.float32)
        lw[0, :k] = a
        ea = np.exp(float(np.float32(a)))
        expect = (k * ea + N - k) ** 2 / (k * ea ** 2 + N - k)
        got = orc.resample(lw, 0.0, 1, 0)["ess"][0]
        assert got == pytest.approx(expect, rel=1e-14)


def test_ess_bounds_and_strict_threshold(orc):
    rng = np.random.default_rng(0)
    lw = rng.normal(0, 3, (64, 32)).astype(np.float32)
    out = orc.resample(lw, 0.5, 9, 4)
    assert np.all(out["ess"] >= 1.0) and np.all(out["ess"] <= 32.0)
    for b in range(64):
        assert out["ess"][b] == pytest.approx(_ess_ref(lw[b]), rel=1e-13)
        assert out["resampled"][b] == int(out["ess"][b] < 0.5 * 32)
    # equal weights: ESS = N exactly, tau = 1 is not "below"
    out = orc.resample(np.zeros((2, 8), np.float32), 1.0, 1, 1)
    assert np.all(out["resampled"] == 0)


@pytest.mark.skipif(not rocrand_probe.available(), reason="hipcc / rocRAND headers not present")
def test_systematic_matches_searchsorted(orc):
    rng = np.random.default_rng(1)
    B, N, seed, step = 40, 24, 0x1234_5678_9ABC, 31
    lw = rng.normal(0, 2, (B, N)).astype(np.float32)
    out = orc.resample(lw, 2.0, seed, step)        # tau > 1: every prompt resamples
    assert np.all(out["resampled"] == 1)
    ctr = np.array([[b, step, 0, 2] for b in range(B)], np.uint32)
    key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32), (B, 1))
    blocks = rocrand_probe.philox_blocks(ctr, key)
    for b in range(B):
        u0 = float(int(blocks[b, 0]) >> 8) / (1 << 24)
        w = np.exp(lw[b].astype(np.float64) - lw[b].max())
        C = np.cumsum(w) / w.sum()
        ref = np.minimum(np.searchsorted(C, (np.arange(N) + u0) / N, side="right"), N - 1)
        ok = out["margin_pos"][b] > 1e-12
        assert np.array_equal(out["ancestors"][b][ok], ref[ok])
        assert np.all(np.diff(out["ancestors"][b]) >= 0)            # non-decreasing
        assert np.all(out["lw"][b] == 0.0)                          # weights restart uniform


def test_offspring_counts_bounds(orc):
    rng = np.random.default_rng(2)
    B, N = 200, 16
    lw = rng.normal(0, 1.5, (B, N)).astype(np.float32)
    out = orc.resample(lw, 2.0, 77, 5)
    for b in range(B):
        w = np.exp(lw[b].astype(np.float64) - lw[b].max())
        W = w / w.sum()
        c = np.bincount(out["ancestors"][b], minlength=N)
        assert c.sum() == N
        assert np.all(c >= np.floor(N * W) - 1e-9) and np.all(c <= np.ceil(N * W) + 1e-9)


def test_identity_when_equal_weights_forced(orc):
    out = orc.resample(np.zeros((3, 10), np.float32), 1.5, 3, 3)
    assert np.all(out["resampled"] == 1)
    assert np.array_equal(out["ancestors"], np.tile(np.arange(10), (3, 1)))


def test_offspring_unbiased_monte_carlo(orc):
    """E[c_j] = N W_j over the resampling offset u0 (many rounds t)."""
    rng = np.random.default_rng(3)
    N = 8
    lw = rng.normal(0, 1.0, (1, N)).astype(np.float32)
    w = np.exp(lw[0].astype(np.float64) - lw[0].max())
    W = w / w.sum()
    reps = 4000
    lwB = np.repeat(lw, reps, 0)
    out = orc.resample(lwB, 2.0, 11, 0)          # prompts b = 0..reps-1 use distinct u0 streams
    c = np.stack([np.bincount(a, minlength=N) for a in out["ancestors"]]).mean(0)
    # c_j in {floor, ceil}: variance <= 1/4, so the mean's std <= 0.5/sqrt(reps)
    assert np.all(np.abs(c - N * W) < 6 * 0.5 / np.sqrt(reps))


def test_degenerate_weights_flagged(orc):
    lw = np.full((2, 4), -np.inf, np.float32)
    lw[1] = 0
    out = orc.resample(lw, 0.5, 1, 1)
    assert out["status"] & orc.ST_DEGENERATE_WEIGHTS
    assert out["resampled"][0] == 0 and np.array_equal(out["ancestors"][0], np.arange(4))
    assert out["ess"][1] == 4
