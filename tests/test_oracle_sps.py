"""Exact, deterministic pins of the oracle's SpS verify (CPU only).

The speculative-sampling notes ("Accelerating Large Language Model Decoding with
Speculative Sampling"): section 1 - the draft proposes K tokens, the target scores them in
parallel, and each is kept or resampled so that the output follows the target exactly;
section 4.2 - the modified rejection rule: keep x_k with probability min(1, p(x_k)/q(x_k)),
and at the first rejection draw from the residual max(0, p - q) renormalised; section 6,
Theorem 1 - the emitted tokens follow the target distribution.

Pins, none of which re-uses the oracle's arithmetic:
  * every acceptance decision against the rule written with scipy's log_softmax and the
    uniforms of rocRAND's own Philox4x32-10 (counter (g, t lo, t hi, 3 | (k div 4) << 8),
    word k mod 4, u = (word >> 8) 2^-24), for K = 4 and K = 6 (words and tags past 4);
  * every final draw against numpy's searchsorted over the residual's cumulative sum (or
    p_K's, with no rejection), with rocRAND's uniform of tag 4, and the drawn token's log p;
  * a forced rejection (a draft token masked in the target row) and an empty residual
    (p = q in the rejected row, which falls back to p);
  * the law of the rule itself: enumerating every draft and every accept / reject branch
    on V = 8, K = 2 with prefix-dependent tables, the first three emitted tokens follow
    pi(y) = p(y1) p(y2 | y1) p(y3 | y1 y2) to 1e-12 (continuous uniforms), and to within the
    2^-24 grid of the 24-bit uniforms when the branch probabilities are those of that grid.
"""
import functools

import numpy as np
import pytest
from scipy import special

from tests.helpers import rocrand_probe
from tests.test_oracle_laws import _tables

needs_probe = pytest.mark.skipif(not rocrand_probe.available(),
                                 reason="hipcc / rocRAND headers not present")

TAG_ACCEPT, TAG_FINAL = 3, 4
SEED, STEP = 0x9E3779B97F4A7C15, (1 << 33) + 12345   # both key words and the step's high word used


def _uniforms(idx, tags, words):
    """rocRAND Philox4x32-10 uniforms for stream indices idx, tags and words (arrays)."""
    n = len(idx)
    ctr = np.stack([np.asarray(idx, np.uint64), np.full(n, STEP & 0xFFFFFFFF, np.uint64),
                    np.full(n, STEP >> 32, np.uint64), np.asarray(tags, np.uint64)],
                   1).astype(np.uint32)
    key = np.tile(np.array([SEED & 0xFFFFFFFF, SEED >> 32], np.uint64), (n, 1)).astype(np.uint32)
    blk = rocrand_probe.philox_blocks(ctr, key)
    w = blk[np.arange(n), np.asarray(words)].astype(np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) / float(1 << 24)


def _case(K, T, nseq=300, V=53, seed=0):
    """Logits and draft tokens: draft = target + noise, so some drafts are kept and some not;
    the draft tokens are drawn from the draft (as the Extend step would)."""
    rng = np.random.default_rng(1000 + 17 * K + seed)
    tgt = rng.normal(0, 1.5, (nseq, K + 1, V)).astype(np.float32)
    drf = (tgt[:, :K] + rng.normal(0, 1.0, (nseq, K, V))).astype(np.float32)
    q = special.softmax(drf.astype(np.float64) / T, axis=-1)
    c = np.cumsum(q, -1)
    u = rng.random((nseq, K, 1))
    toks = np.minimum((c < u * c[..., -1:]).sum(-1), V - 1).astype(np.int32)
    return tgt, drf, toks


def _expected(tgt, drf, toks, T, idx):
    """The rule of section 4.2 in fp64 with scipy's log_softmax and rocRAND's uniforms:
    (k*, final token, log p of it, smallest decision margin) per sequence."""
    nseq, K1, V = tgt.shape
    K = K1 - 1
    lpt = special.log_softmax(tgt.astype(np.float64) / T, axis=-1)
    lpd = special.log_softmax(drf.astype(np.float64) / T, axis=-1)
    ks = np.repeat(np.arange(K)[None], nseq, 0).reshape(-1)
    r = _uniforms(np.repeat(idx, K), TAG_ACCEPT | ((ks // 4) << 8), ks % 4).reshape(nseq, K)
    uf = _uniforms(idx, np.full(nseq, TAG_FINAL), np.zeros(nseq, np.int64))
    out = []
    np.seterr(invalid="ignore")  # a token masked in both rows: ratio 0/0 (no acceptance)
    for s in range(nseq):
        kstar, margin = K, np.inf
        for k in range(K):
            ratio = np.exp(lpt[s, k, toks[s, k]] - lpd[s, k, toks[s, k]])
            margin = min(margin, abs(r[s, k] - ratio))
            if not (r[s, k] < ratio):
                kstar = k
                break
        p = np.exp(lpt[s, kstar])
        w = p
        if kstar < K:
            rho = np.maximum(p - np.exp(lpd[s, kstar]), 0.0)
            if rho.sum() > 0.0:
                w = rho
        cdf = np.cumsum(w) / w.sum()
        tok = int(np.searchsorted(cdf, uf[s], side="right"))
        margin = min(margin, abs(uf[s] - cdf[tok]), abs(uf[s] - (cdf[tok - 1] if tok else 0.0)))
        out.append((kstar, tok, lpt[s, kstar, tok], margin))
    return out


@functools.lru_cache(maxsize=None)
def _run(K, T):
    import oracle
    oracle.build()
    tgt, drf, toks = _case(K, T)
    idx = np.arange(len(toks), dtype=np.int64) * 7 + 3
    o = oracle.verify_sps(tgt, drf, toks, T, SEED, STEP, rng_index=idx)
    return tgt, drf, toks, idx, o, _expected(tgt, drf, toks, T, idx)


@needs_probe
@pytest.mark.parametrize("K,T", [(4, 1.0), (4, 0.8), (6, 1.3)])
def test_sps_accept_decisions_follow_the_rule(orc, K, T):
    tgt, drf, toks, idx, o, exp = _run(K, T)
    kstars = []
    for s, (kstar, _, _, margin) in enumerate(exp):
        if margin < 1e-9:
            continue
        kstars.append(kstar)
        assert o["num_tokens"][s] == kstar + 1, s
        assert np.array_equal(o["tokens"][s, :kstar], toks[s, :kstar]), s
        assert np.all(o["tokens"][s, kstar + 1:] == -1), s
    # the cases reach every outcome: early rejections, late ones, all accepted
    assert len(kstars) > 0.98 * len(exp)
    assert set(range(K + 1)) <= set(kstars)


@needs_probe
@pytest.mark.parametrize("K,T", [(4, 1.0), (4, 0.8), (6, 1.3)])
def test_sps_final_draw_is_searchsorted_on_the_residual(orc, K, T):
    tgt, drf, toks, idx, o, exp = _run(K, T)
    checked = 0
    for s, (kstar, tok, lp, margin) in enumerate(exp):
        if margin < 1e-9:
            continue
        assert o["tokens"][s, kstar] == tok, s
        assert abs(o["logp"][s, K] - lp) <= 1e-12 * max(1.0, abs(lp)), s
        checked += 1
    assert checked > 0.98 * len(exp)


def _single(tgt, drf, toks, T=1.0):
    import oracle
    idx = np.arange(len(toks), dtype=np.int64)
    return oracle.verify_sps(tgt, drf, toks, T, SEED, STEP, rng_index=idx), \
        _expected(tgt, drf, toks, T, idx)


@needs_probe
def test_sps_forced_rejection_and_empty_residual(orc):
    K, T = 3, 1.0
    tgt, drf, toks = _case(K, T, nseq=64, V=29, seed=5)
    # forced rejection at k = 1: the target gives the draft token no mass
    a_t = tgt.copy()
    for s in range(64):
        a_t[s, 1, toks[s, 1]] = -np.inf
    o, exp = _single(a_t, drf, toks)
    for s, (kstar, tok, lp, margin) in enumerate(exp):
        assert kstar <= 1
        if margin >= 1e-9:
            assert o["num_tokens"][s] == kstar + 1 and o["tokens"][s, kstar] == tok
            assert o["tokens"][s, kstar] != toks[s, kstar] or kstar == 0
    assert np.mean([e[0] == 1 for e in exp]) > 0.3        # rejections at k = 1 do occur
    # empty residual: row 0 of draft and target identical, the draft token masked in both
    # (ratio 0/0 is no acceptance), so max(0, p - q) = 0 and the draw falls back to p
    b_t, b_d = tgt.copy(), drf.copy()
    b_d[:, 0] = b_t[:, 0]
    for s in range(64):
        b_t[s, 0, toks[s, 0]] = -np.inf
        b_d[s, 0, toks[s, 0]] = -np.inf
    o, exp = _single(b_t, b_d, toks)
    p = special.softmax(b_t[:, 0].astype(np.float64) / T, axis=-1)
    u = _uniforms(np.arange(64), np.full(64, TAG_FINAL), np.zeros(64, np.int64))
    for s in range(64):
        assert exp[s][0] == 0 and o["num_tokens"][s] == 1
        want = int(np.searchsorted(np.cumsum(p[s]), u[s], side="right"))
        if exp[s][3] >= 1e-9:
            assert o["tokens"][s, 0] == want == exp[s][1]
        assert o["tokens"][s, 0] != toks[s, 0]              # the masked token has p = 0
    assert o["status"] == 0


# --------------------------------------------------------------------------- the law
V8, K2 = 8, 2


def _sm(x):
    return special.softmax(x.astype(np.float64), axis=-1)


def _grid(pr):
    """Probability that a 24-bit uniform u = j 2^-24 satisfies u < pr (pr in [0, 1])."""
    n = float(1 << 24)
    return np.minimum(np.ceil(pr * n), n) / n


def _grid_draw(w):
    """Law of searchsorted(cumsum(w)/sum(w), u, 'right') for u on the 2^-24 grid."""
    n = float(1 << 24)
    c = np.concatenate([[0.0], np.cumsum(w) / w.sum()])
    c[-1] = 1.0
    return np.diff(np.minimum(np.ceil(c * n), n)) / n


def _round_law(tgt, drf, code, d, grid):
    """{emitted tuple: probability} of one SpS round from the prefix with index `code` at
    depth d: x1 ~ q, x2 ~ q(.|x1); keep x_k with probability min(1, p/q) (P(u < p/q) on the
    grid); at the first rejection draw from max(0, p - q) renormalised (p if empty); with
    none, draw from p(.|x1 x2)."""
    acc = (lambda pr: _grid(pr)) if grid else (lambda pr: np.minimum(1.0, pr))
    draw = _grid_draw if grid else (lambda w: w / w.sum())
    law = {}

    def add(key, pr):
        law[key] = law.get(key, 0.0) + pr

    p1, q1 = _sm(tgt[d][code]), _sm(drf[d][code])
    rho1 = np.maximum(p1 - q1, 0.0)
    r1 = draw(rho1 if rho1.sum() > 0 else p1)
    for x1 in range(V8):
        a1 = acc(p1[x1] / q1[x1])
        for y in range(V8):
            add((y,), q1[x1] * (1 - a1) * r1[y])
        c1 = code * V8 + x1
        p2, q2 = _sm(tgt[d + 1][c1]), _sm(drf[d + 1][c1])
        rho2 = np.maximum(p2 - q2, 0.0)
        r2 = draw(rho2 if rho2.sum() > 0 else p2)
        for x2 in range(V8):
            a2 = acc(p2[x2] / q2[x2])
            for y in range(V8):
                add((x1, y), q1[x1] * a1 * q2[x2] * (1 - a2) * r2[y])
            p3 = draw(_sm(tgt[d + 2][c1 * V8 + x2]))
            for y in range(V8):
                add((x1, x2, y), q1[x1] * a1 * q2[x2] * a2 * p3[y])
    return law


def _first_three_law(tgt, drf, grid):
    """Law of the first three emitted tokens over as many rounds as they take."""
    out = np.zeros(V8 ** 3)
    stack = [((), 1.0)]
    while stack:
        prefix, pr = stack.pop()
        code = 0
        for v in prefix:
            code = code * V8 + v
        for em, pe in _round_law(tgt, drf, code, len(prefix), grid).items():
            y = prefix + em
            if len(y) >= 3:
                out[y[0] * 64 + y[1] * 8 + y[2]] += pr * pe
            else:
                stack.append((y, pr * pe))
    return out


def _pi(tgt):
    p0, p1, p2 = _sm(tgt[0][0]), _sm(tgt[1]), _sm(tgt[2])
    pi = np.zeros((V8, V8, V8))
    for a in range(V8):
        for b in range(V8):
            pi[a, b] = p0[a] * p1[a, b] * p2[a * V8 + b]
    return pi.reshape(-1)


@pytest.mark.parametrize("seed", [2024, 7, 31337])
def test_sps_rule_is_exact_by_enumeration(seed):
    tgt, drf = _tables(seed)
    pi = _pi(tgt)
    law = _first_three_law(tgt, drf, grid=False)
    assert abs(law.sum() - 1.0) < 1e-12
    assert np.max(np.abs(law - pi)) < 1e-12
    # with the 24-bit uniforms the oracle draws, each branch probability moves by at most
    # 2^-24: the law stays within a few grid steps of the target
    lawg = _first_three_law(tgt, drf, grid=True)
    assert abs(lawg.sum() - 1.0) < 1e-12
    assert np.max(np.abs(lawg - pi)) < 2.0 ** -20
    # the draft alone is far from the target: the rule does the correcting
    q = np.zeros((V8, V8, V8))
    q0, q1 = _sm(drf[0][0]), _sm(drf[1])
    p2 = _sm(tgt[2])
    for a in range(V8):
        for b in range(V8):
            q[a, b] = q0[a] * q1[a, b] * p2[a * V8 + b]
    assert np.abs(q.reshape(-1) - pi).sum() > 0.05
