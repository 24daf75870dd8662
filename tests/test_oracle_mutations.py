"""The oracle's pins have power: each plausible mistake, planted in a private copy of
the oracle's C source (CPU only, never the HIP path), makes at least one pin fail.

Each case names a text substitution in smcsd_oracle.c (a dropped term, a wrong sign,
a wrong index or row, a transposed operand, a wrong comparison) and the pin tests
expected to catch it.  The variant library is compiled into a temporary directory
and swapped in for the duration of the case only.
"""
import contextlib
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_draft as dr
from tests import test_oracle_kv as kv
from tests import test_oracle_laws as laws
from tests import test_oracle_race as race
from tests import test_oracle_resample as rs
from tests import test_oracle_rng as rng_t
from tests import test_oracle_sps as sps
from tests import test_oracle_verify as vf
from tests.helpers import rocrand_probe

SRC = open(oracle.SRC).read()


@contextlib.contextmanager
def planted(old: str, new: str):
    assert SRC.count(old) >= 1, "mutation anchor not found: %r" % old
    src = SRC.replace(old, new)
    d = tempfile.mkdtemp(prefix="orc_mut_")
    c_path = os.path.join(d, "m.c")
    so_path = os.path.join(d, "m.so")
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    c_path, "-o", so_path, "-lm"], check=True)
    saved = oracle._load()
    oracle._lib = oracle.configure(ctypes.CDLL(so_path))
    try:
        yield
    finally:
        oracle._lib = saved


def _caught(pins) -> bool:
    for fn in pins:
        try:
            fn()
        except AssertionError:
            return True
    return False


O = oracle
NEEDS_PROBE = rocrand_probe.available()

CASES = [
    ("weight sign of log q", "incr += alpha * lp - lq;", "incr += alpha * lp + lq;",
     [lambda: vf.test_weight_identity_by_enumeration(O, 1.0)]),
    ("bonus term dropped (power mode)", "incr += (alpha - 1.0) * lpK;", "incr += 0.0 * lpK;",
     [lambda: vf.test_weight_identity_by_enumeration(O, 4.0)]),
    ("alpha on bonus instead of alpha-1", "incr += (alpha - 1.0) * lpK;", "incr += alpha * lpK;",
     [lambda: vf.test_weight_identity_by_enumeration(O, 1.0)]),
    ("LSE without the max shift", "return zmax + log(s);", "return log(s);",
     [lambda: vf.test_row_lse_matches_scipy_fp32(O, 1.0, 1000)]),
    ("temperature ignored in target gather",
     "lp = load_elem(trow, dtype, x) / T - L[k];",
     "lp = load_elem(trow, dtype, x) - L[k];",
     [lambda: vf.test_verify_gather_and_weights_vs_log_softmax(O, "f32", 1.0)]),
    ("log q gathered from the target row",
     "load_elem(row_ptr(drf, dtype, (int64_t)s * K + k, V), dtype, x) / T",
     "load_elem(trow, dtype, x) / T",
     [lambda: vf.test_verify_gather_and_weights_vs_log_softmax(O, "f32", 1.0)]),
    ("bonus drawn from row K-1",
     "const void *brow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + K, V);",
     "const void *brow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + K - 1, V);",
     [lambda: vf.test_bonus_chi_square_against_target(O)]),
    ("uniform loses its top bit", "(double)(out[word & 3] >> 8)", "(double)(out[word & 3] >> 9)",
     [lambda: rng_t.test_uniform_chi_square(O)]),
    ("Philox key bump uses the wrong Weyl constant", "k0 += weyl0;", "k0 += weyl1;",
     [lambda: rng_t.test_philox_known_answer_vectors(O)]
     + ([lambda: rng_t.test_philox_matches_rocrand_block_function(O)] if NEEDS_PROBE else [])),
    ("Philox round mixes the wrong high half", "uint32_t n0 = hi1 ^ c1 ^ k0;",
     "uint32_t n0 = hi0 ^ c1 ^ k0;",
     [lambda: rng_t.test_philox_known_answer_vectors(O)]
     + ([lambda: rng_t.test_philox_matches_rocrand_block_function(O)] if NEEDS_PROBE else [])),
    ("counter words t_hi and tag swapped",
     "uint32_t ctr[4] = {index, (uint32_t)t, (uint32_t)(t >> 32), tag};",
     "uint32_t ctr[4] = {index, (uint32_t)t, tag, (uint32_t)(t >> 32)};",
     [lambda: rng_t.test_uniform_counter_layout_matches_rocrand(O)] if NEEDS_PROBE else []),
    ("ESS without the square", "double e = s1 * s1 / s2;", "double e = s1 / s2;",
     [lambda: rs.test_ess_closed_forms(O)]),
    ("threshold not strict", "int do_res = e < tau * (double)N;", "int do_res = e <= tau * (double)N;",
     [lambda: rs.test_ess_bounds_and_strict_threshold(O)]),
    ("systematic offset dropped", "double pos = ((double)i + u0) / (double)N;",
     "double pos = ((double)i) / (double)N;",
     [lambda: rs.test_offspring_unbiased_monte_carlo(O)]),
    ("weights not reset after resampling",
     "for (int n = 0; n < N; ++n) lw_out[(int64_t)b * N + n] = 0.0;", "",
     [lambda: rs.test_systematic_matches_searchsorted(O)] if NEEDS_PROBE else []),
    ("refcount increments skipped for two offspring", "if (cnt[j] > 1)\n", "if (cnt[j] > 2)\n",
     [lambda: kv.test_block_tables_reproduce_deep_copy_model(O, True, 4, 2, 16, True)]),
    ("copy-on-write never done", "needs_cow[g] = 1;", "needs_cow[g] = 0;",
     [lambda: kv.test_block_tables_reproduce_deep_copy_model(O, False, 4, 2, 16, True)]),
    ("freed blocks pushed ascending", "return (x < y) - (x > y);", "return (x > y) - (x < y);",
     [lambda: kv.test_identity_is_noop_and_all_equal_ancestors(O)]),
    ("gather ignores the ancestors", "old[(int64_t)a[i] * nb_old + s]", "old[(int64_t)i * nb_old + s]",
     [lambda: kv.test_block_tables_reproduce_deep_copy_model(O, False, 4, 2, 16, True)]),
    ("SpS residual without the positive part", "double rho = p - q > 0.0 ? p - q : 0.0;",
     "double rho = fabs(p - q);", [lambda: laws.test_sps_law_equals_target(O)]),
    ("SpS accepts every draft", "if (!(r < ratio)) {", "if (!(r < 1.0)) {",
     [lambda: laws.test_sps_law_equals_target(O)]),
    ("SMC weight uses q/p", "incr += alpha * lp - lq;", "incr += lq - alpha * lp;",
     [lambda: laws.test_smc_round_follows_sir_law(O, 4, 1.0)]),
    ("draft uniform ignores the position", "ORC_TAG_DRAFT | ((uint32_t)pos << 8)", "ORC_TAG_DRAFT",
     [lambda: dr.test_draft_sample_is_the_textbook_inverse_cdf(O, "f32", 1.0)]),
    ("draft log q without the temperature",
     "logq[r] = x >= 0 ? load_elem(row, dtype, x) / T - L : NAN;",
     "logq[r] = x >= 0 ? load_elem(row, dtype, x) - L : NAN;",
     [lambda: dr.test_draft_sample_is_the_textbook_inverse_cdf(O, "f32", 0.8)]),
    ("draft log q of the wrong token", "logq[r] = x >= 0 ? load_elem(row, dtype, x) / T - L : NAN;",
     "logq[r] = x >= 0 ? load_elem(row, dtype, x > 0 ? x - 1 : x) / T - L : NAN;",
     [lambda: dr.test_draft_sample_is_the_textbook_inverse_cdf(O, "f32", 1.0)]),
    ("race key adds the log clock", "double key = z - log(orc_race_clock(", "double key = z + log(orc_race_clock(",
     [lambda: race.test_race_law_chi_square(O, 1.0)]),
    ("race key without the temperature", "double key = z - log(orc_race_clock(",
     "double key = z * T - log(orc_race_clock(", [lambda: race.test_race_law_chi_square(O, 0.7)]),
    ("race clocks share one Philox word", "(double)(out[v & 3] >> 9)", "(double)(out[0] >> 9)",
     [lambda: race.test_race_clocks_are_exponential_and_uncorrelated(O)]),
    ("race clocks repeat every block", "ORC_TAG_RACE | ((uint32_t)(v >> 2) << 8)", "ORC_TAG_RACE",
     [lambda: race.test_race_clocks_are_exponential_and_uncorrelated(O)]),
    ("verify ignores the race rule", "if (bonus_rule == ORC_BONUS_RACE)", "if (0)",
     [lambda: race.test_verify_race_bonus_is_the_race_and_reweights(O, 1.0)]),
    ("verify reads the wrong precomputed log q", "logq_in[(int64_t)s * K + k]", "logq_in[(int64_t)s * K]",
     [lambda: dr.test_verify_with_draft_logq_equals_reading_the_draft_rows(O)]),
    ("SpS acceptance reads word 0 for every draft",
     "ORC_TAG_SPS_ACCEPT | ((uint32_t)(k / 4) << 8), k % 4);",
     "ORC_TAG_SPS_ACCEPT | ((uint32_t)(k / 4) << 8), 0);",
     [lambda: _sps(sps.test_sps_accept_decisions_follow_the_rule, 4, 1.0)] if NEEDS_PROBE else []),
    ("SpS acceptance tag ignores k div 4",
     "ORC_TAG_SPS_ACCEPT | ((uint32_t)(k / 4) << 8), k % 4);", "ORC_TAG_SPS_ACCEPT, k % 4);",
     [lambda: _sps(sps.test_sps_accept_decisions_follow_the_rule, 6, 1.3)] if NEEDS_PROBE else []),
    ("SpS final draw with the acceptance tag", "orc_uniform(seed, g, t, ORC_TAG_SPS_FINAL, 0);",
     "orc_uniform(seed, g, t, ORC_TAG_SPS_ACCEPT, 0);",
     [lambda: _sps(sps.test_sps_final_draw_is_searchsorted_on_the_residual, 4, 1.0)]
     if NEEDS_PROBE else []),
    ("SpS residual q taken from the target row",
     "const void *qrow = row_ptr(drf, dtype, (int64_t)s * K + kstar, V);",
     "const void *qrow = row_ptr(tgt, dtype, (int64_t)s * (K + 1) + kstar, V);",
     [lambda: _sps(sps.test_sps_final_draw_is_searchsorted_on_the_residual, 4, 1.0)]
     if NEEDS_PROBE else []),
    ("SpS residual q - p instead of p - q", "double rho = p - q > 0.0 ? p - q : 0.0;",
     "double rho = q - p > 0.0 ? q - p : 0.0;",
     [lambda: _sps(sps.test_sps_final_draw_is_searchsorted_on_the_residual, 4, 0.8)]
     if NEEDS_PROBE else []),
    ("SpS empty residual draws nothing", "} else if (isfinite(L[kstar])) {", "} else if (0) {",
     [lambda: sps.test_sps_forced_rejection_and_empty_residual(O)] if NEEDS_PROBE else []),
    ("SpS drawn token's log p from the bonus row",
     "tok >= 0 ? load_elem(prow, dtype, tok) / T - L[kstar] : NAN;",
     "tok >= 0 ? load_elem(prow, dtype, tok) / T - L[K] : NAN;",
     [lambda: _sps(sps.test_sps_final_draw_is_searchsorted_on_the_residual, 4, 1.0)]
     if NEEDS_PROBE else []),
]


def _sps(fn, K, T):
    """An SpS pin on fresh oracle output (its cached run is computed before the swap)."""
    sps._run.cache_clear()
    try:
        fn(O, K, T)
    finally:
        sps._run.cache_clear()


@pytest.mark.parametrize("name,old,new,pins", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(name, old, new, pins):
    if not pins:
        pytest.skip("the pin for this case needs the rocRAND probe")
    with planted(old, new):
        assert _caught(pins), "planted mistake not caught: " + name
