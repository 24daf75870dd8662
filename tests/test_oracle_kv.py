"""Pins of the oracle's refcounted block-table pointer exchange - CPU only.

Brute force: a deep-copy model keeps every particle's token list explicitly; the
block-table model (the oracle) plus a per-block token store, written through the
tables and patched with the oracle's copy-on-write list, must reproduce every list
after every round.  A block freed while still referenced, a wrong gather, a missing
copy-on-write or a double allocation all corrupt some particle's tokens.
Invariants: rc[b] = number of table references; live and free blocks partition the
pool; no table entry has rc = 0; identity ancestors leave the tables unchanged.
"""
import math

import numpy as np
import pytest


def _initial(B, N, M, bs, P, ctx0, shared):
    T = np.full((B * N, M), -1, np.int32)
    rc = np.zeros(P, np.int32)
    fl = np.arange(P - 1, -1, -1, dtype=np.int32)
    nb0 = math.ceil(ctx0 / bs)
    nxt = 0
    if shared:
        for b in range(B):
            T[b * N:(b + 1) * N, :nb0] = np.arange(nxt, nxt + nb0)
            rc[nxt:nxt + nb0] = N
            nxt += nb0
    else:
        for g in range(B * N):
            T[g, :nb0] = np.arange(nxt, nxt + nb0)
            rc[nxt:nxt + nb0] = 1
            nxt += nb0
    return T, rc, fl, P - nxt


def _check_invariants(st, P):
    T, rc, fl, top = st["tables"], st["refcounts"], st["free_list"], st["free_top"]
    refs = np.bincount(T[T >= 0], minlength=P)
    assert np.array_equal(refs, rc), "refcount != number of table references"
    free = fl[:top]
    assert len(np.unique(free)) == top, "duplicate block on the free stack"
    assert np.all(rc[free] == 0), "a free block is still referenced"
    live = np.nonzero(rc)[0]
    assert len(live) + top == P, "live and free blocks do not partition the pool"


def _tokens_via_tables(store, T, g, L, bs):
    return [store[T[g, p // bs]][p % bs] for p in range(L)]


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("bs,K,ctx0", [(4, 2, 16), (16, 4, 35), (3, 5, 7), (8, 7, 0)])
@pytest.mark.parametrize("sorted_ancestors", [True, False])
def test_block_tables_reproduce_deep_copy_model(orc, shared, bs, K, ctx0, sorted_ancestors):
    rng = np.random.default_rng(hash((shared, bs, K, ctx0, sorted_ancestors)) & 0xFFFF)
    B, N, rounds = 3, 6, 25
    R = K + 1
    M = math.ceil((ctx0 + (rounds + 1) * R) / bs)
    P = B * N * M
    T, rc, fl, top = _initial(B, N, M, bs, P, ctx0, shared)
    # token store per block; prompt tokens written through the initial tables
    store = np.full((P, bs), -1, np.int64)
    tokens = []
    for g in range(B * N):
        b = g // N
        prompt = [1000 * b + p for p in range(ctx0)]
        tokens.append(list(prompt))
        for p, tkn in enumerate(prompt):
            store[T[g, p // bs], p % bs] = tkn
    L = ctx0
    # reservation before round 0 (identity ancestors)
    st = orc.kv_reassign(np.tile(np.arange(N), (B, 1)), np.zeros(B), T, bs, L, R, rc, fl, top)
    assert st["status"] == 0
    for src, dst, n in st["cow"]:
        store[dst, :n] = store[src, :n]
    _check_invariants(st, P)
    for rnd in range(rounds):
        T = st["tables"]
        # the round writes K+1 new tokens per particle into its reserved slots
        for g in range(B * N):
            new = [int(x) for x in rng.integers(0, 10**6, R)]
            for j, tkn in enumerate(new):
                p = L + j
                store[T[g, p // bs], p % bs] = tkn
            tokens[g].extend(new)
        L += R
        resampled = (rng.random(B) < 0.6).astype(np.int32)
        if sorted_ancestors:
            anc = np.sort(rng.integers(0, N, (B, N)), axis=1).astype(np.int32)
        else:
            anc = rng.integers(0, N, (B, N)).astype(np.int32)
        before = T.copy()
        st = orc.kv_reassign(anc, resampled, T, bs, L, R, st["refcounts"], st["free_list"],
                             st["free_top"])
        assert st["status"] == 0
        for src, dst, n in st["cow"]:
            assert n == L % bs
            store[dst, :n] = store[src, :n]
        new_tokens = []
        for g in range(B * N):
            b, i = divmod(g, N)
            a = anc[b, i] if resampled[b] else i
            new_tokens.append(list(tokens[b * N + a]))
        tokens = new_tokens
        _check_invariants(st, P)
        for g in range(B * N):
            assert _tokens_via_tables(store, st["tables"], g, L, bs) == tokens[g]
        # identity prompts keep their committed slots; nobody rewrites full blocks below floor(L/bs)
        for b in range(B):
            if not resampled[b]:
                rows = slice(b * N, (b + 1) * N)
                assert np.array_equal(st["tables"][rows, :L // bs], before[rows, :L // bs])


def test_identity_is_noop_and_all_equal_ancestors(orc):
    B, N, bs, M = 1, 4, 4, 10
    P = B * N * M
    T, rc, fl, top = _initial(B, N, M, bs, P, 8, False)
    st = orc.kv_reassign(np.tile(np.arange(N), (B, 1)), np.ones(B), T, bs, 8, 0, rc, fl, top)
    assert np.array_equal(st["tables"], T) and np.array_equal(st["refcounts"], rc)
    st = orc.kv_reassign(np.full((1, N), 2), np.ones(1), T, bs, 8, 0, rc, fl, top)
    for g in range(N):
        assert np.array_equal(st["tables"][g], T[2])
    assert np.all(st["refcounts"][T[2, :2]] == N)
    # six blocks freed (particles 0, 1, 3), pushed in descending order: pops return ascending
    assert st["free_top"] == top + 6
    assert list(st["free_list"][top:top + 6]) == sorted(
        [int(x) for x in T[[0, 1, 3], :2].ravel()], reverse=True)


def test_hand_worked_round():
    """A round worked by hand from the rules (no oracle involved in the expectation).
    B=1, N=3, bs=4, L=6 (slots 0,1 allocated; slot 1 is a partial tail with 2 tokens),
    tables: g0 -> [0, 1], g1 -> [2, 3], g2 -> [4, 5]; rc = 1 for blocks 0..5;
    free stack (bottom..top) = [9, 8, 7, 6] so pops return 6, 7, 8, 9, ...
    Ancestors (0, 0, 2): c = (2, 0, 1).
      increments: blocks 0, 1 -> rc 2.  decrements: blocks 2, 3 -> rc 0 -> freed.
      push descending: stack = [9, 8, 7, 6, 3, 2] (top = 2).
      tables: g0 -> [0, 1], g1 -> [0, 1], g2 -> [4, 5].
    Reserve R=3 positions 6..8: tail slot 1 (L mod bs = 2), fresh slot 2.
      g0: block 1 has rc 2 and g1 > g0 also holds it -> COW: pop 2, rc[1] = 1,
          rc[2] = 1, g0 slot 1 = 2, emit (1, 2, 2); fresh slot 2: pop 3.
      g1: block 1 now has rc 1 but the decision uses the post-exchange state
          (rc 2, no higher holder) -> keep; fresh slot 2: pop 6.
      g2: block 5 rc 1 -> keep; fresh slot 2: pop 7.
    Final tables: [0, 2, 3], [0, 1, 6], [4, 5, 7]; top = 6 - 4 = ... stack length 6 -> 2."""
    import oracle
    T = np.full((3, 4), -1, np.int32)
    T[0, :2] = [0, 1]
    T[1, :2] = [2, 3]
    T[2, :2] = [4, 5]
    rc = np.zeros(10, np.int32)
    rc[:6] = 1
    fl = np.zeros(10, np.int32)
    fl[:4] = [9, 8, 7, 6]
    st = oracle.kv_reassign(np.array([[0, 0, 2]]), np.array([1]), T, 4, 6, 3, rc, fl, 4)
    assert st["tables"][:, :3].tolist() == [[0, 2, 3], [0, 1, 6], [4, 5, 7]]
    assert st["cow"].tolist() == [[1, 2, 2]]
    assert st["free_top"] == 2 and st["free_list"][:2].tolist() == [9, 8]
    expect_rc = np.zeros(10, np.int32)
    expect_rc[[0]] = 2
    expect_rc[[1, 2, 3, 4, 5, 6, 7]] = 1
    assert st["refcounts"].tolist() == expect_rc.tolist()


def test_nospace_is_reported(orc):
    B, N, bs, M = 1, 2, 4, 6
    T, rc, fl, top = _initial(B, N, M, bs, 5, 4, False)   # pool of 5: 2 used, 3 free
    st = orc.kv_reassign(np.tile(np.arange(N), (B, 1)), np.zeros(B), T, bs, 4, 9, rc, fl, top)
    # each sequence needs 3 fresh slots (positions 4..12 -> slots 1..3): 6 > 3 free
    assert st["status"] & orc.ST_NOSPACE
    assert st["free_top"] == 0
    assert st["tables"][0, 1:4].tolist() == [2, 3, 4] and st["tables"][1, 1:4].tolist() == [-1, -1, -1]


def test_slots_left_by_nospace_are_flagged_and_skipped(orc):
    """After a NOSPACE call some allocated slots hold -1; a later resampling call flags
    BAD_INPUT, changes only the counts of real blocks and keeps rc = references."""
    B, N, bs, M, P = 1, 2, 4, 6, 5
    T, rc, fl, top = _initial(B, N, M, bs, P, 4, False)          # blocks 0, 1 used; 3 free
    st = orc.kv_reassign(np.tile(np.arange(N), (B, 1)), np.zeros(B), T, bs, 4, 9, rc, fl, top)
    assert st["status"] == orc.ST_NOSPACE
    assert st["tables"][:, :4].tolist() == [[0, 2, 3, 4], [1, -1, -1, -1]]
    # particle 0 dropped, particle 1 duplicated, one more token reserved (same slot count)
    s2 = orc.kv_reassign(np.array([[1, 1]]), np.array([1]), st["tables"], bs, 13, 1,
                         st["refcounts"], st["free_list"], st["free_top"])
    assert s2["status"] == orc.ST_BAD_INPUT
    assert s2["tables"][:, :4].tolist() == [[1, -1, -1, -1], [1, -1, -1, -1]]
    assert s2["refcounts"].tolist() == [0, 2, 0, 0, 0]
    assert s2["free_top"] == 4 and s2["free_list"][:4].tolist() == [4, 3, 2, 0]
    assert s2["cow_count"] == 0                                   # a -1 tail is not shared


def test_bad_ancestor_leaves_its_prompt_unexchanged(orc):
    B, N, bs, M = 2, 3, 4, 8
    P = B * N * M
    T, rc, fl, top = _initial(B, N, M, bs, P, 8, False)
    anc = np.array([[2, 2, 0], [0, 1, N + 1]], np.int32)
    st = orc.kv_reassign(anc, np.array([1, 1]), T, bs, 8, 4, rc, fl, top)
    good = orc.kv_reassign(np.array([[2, 2, 0], [0, 1, 2]], np.int32), np.array([1, 0]), T, bs, 8,
                           4, rc, fl, top)
    assert st["status"] == orc.ST_BAD_INPUT and good["status"] == 0
    for k in ("tables", "refcounts", "free_list"):
        assert np.array_equal(st[k], good[k]), k
    assert st["free_top"] == good["free_top"]


def test_corrupt_free_stack_entry_is_flagged(orc):
    """A popped id outside [0, P) leaves its slot as it was; a copy-on-write that pops one
    is listed with destination -1 and changes no count."""
    B, N, bs, M = 1, 2, 4, 6
    P = 12
    T, rc, fl, top = _initial(B, N, M, bs, P, 6, True)            # tail slot 1 shared by both
    fl = fl.copy()
    fl[top - 1] = P + 7                                          # the first pop (g = 0's copy)
    st = orc.kv_reassign(np.tile(np.arange(N), (B, 1)), np.zeros(B), T, bs, 6, 1, rc, fl, top)
    assert st["status"] == orc.ST_BAD_INPUT
    assert st["cow_count"] == 1 and st["cow"].tolist() == [[1, -1, 2]]
    assert np.array_equal(st["refcounts"], rc) and np.array_equal(st["tables"], T)
    assert st["free_top"] == top - 1


def test_out_of_vocabulary_draft_token_is_flagged(orc):
    rng = np.random.default_rng(3)
    S, K, V = 3, 2, 40
    tgt = rng.normal(size=(S, K + 1, V)).astype(np.float32)
    drf = rng.normal(size=(S, K, V)).astype(np.float32)
    toks = np.array([[1, 2], [V, 3], [-1, 0]], np.int32)
    o = orc.verify_smc(tgt, drf, toks, 1.0, 1.0, 5, 0, np.zeros(S, np.float32))
    assert o["status"] == orc.ST_BAD_INPUT
    assert np.isfinite(o["lw"][0]) and np.isnan(o["lw"][1]) and np.isnan(o["lw"][2])
    assert np.array_equal(o["tokens"][:, :K], toks)
    assert np.isnan(o["logp"][1, 0]) and np.isnan(o["logq"][2, 0]) and np.isfinite(o["logp"][1, 1])
    s = orc.verify_sps(tgt, drf, toks, 1.0, 5, 0)
    assert s["status"] == orc.ST_BAD_INPUT
    assert s["num_tokens"][1] == 1 and s["num_tokens"][2] == 1      # a NaN ratio is no acceptance


def test_kv_check_definition_on_a_hand_built_state():
    """The invariant counts on a hand-built pool of 8 blocks: two sequences sharing block 0,
    each with a private block, the other five on the free stack; then one corruption at a
    time, each with the count it must give."""
    import oracle

    T = np.array([[0, 1, -1], [0, 2, -1]], np.int32)
    rc = np.array([2, 1, 1, 0, 0, 0, 0, 0], np.int32)
    fl = np.array([7, 6, 5, 4, 3, 0, 0, 0], np.int32)
    assert oracle.kv_check(T, 2, rc, fl, 5).tolist() == [0, 0, 0, 0, 0]
    r = rc.copy(); r[1] = 2                                     # a refcount one too high
    assert oracle.kv_check(T, 2, r, fl, 5).tolist() == [1, 0, 0, 0, 0]
    t = T.copy(); t[1, 1] = 9                                   # an id past the pool
    assert oracle.kv_check(t, 2, rc, fl, 5).tolist() == [1, 1, 0, 0, 0]
    t = T.copy(); t[1, 1] = -1                                  # an unfilled slot: allowed
    assert oracle.kv_check(t, 2, rc, fl, 5).tolist() == [1, 0, 0, 0, 0]
    f = fl.copy(); f[5] = 3                                     # block 3 pushed twice
    assert oracle.kv_check(T, 2, rc, f, 6).tolist() == [0, 0, 1, 0, 0]
    f = fl.copy(); f[5] = 0                                     # a live block on the stack
    assert oracle.kv_check(T, 2, rc, f, 6).tolist() == [0, 0, 0, 1, 0]
    assert oracle.kv_check(T, 2, rc, fl, 4).tolist() == [0, 0, 0, 0, 1]   # block 3 leaked
    f = fl.copy(); f[2] = -3                                    # a corrupt stack entry
    assert oracle.kv_check(T, 2, rc, f, 5).tolist() == [0, 0, 1, 0, 1]   # and 5 is lost
    # a top past the pool (1), clamped to 8: block 0 three times on the stack (2 extra) and
    # live (1)
    assert oracle.kv_check(T, 2, rc, fl, 9).tolist() == [0, 0, 3, 1, 0]
    assert oracle.kv_check(T, 3, rc, fl, 5).tolist() == [0, 0, 0, 0, 0]  # -1 slots skipped
    r = rc.copy(); r[2] = 0                                     # a live block's count lost
    assert oracle.kv_check(T, 2, r, fl, 5).tolist() == [1, 0, 0, 0, 1]


@pytest.mark.parametrize("shared", [False, True])
def test_kv_check_is_clean_after_oracle_rounds(orc, shared):
    """Every state the oracle's exchange leaves passes the invariant check, rounds with
    and without resampling, with copy-on-write and fresh reservations."""
    import oracle

    rng = np.random.default_rng(7 + shared)
    B, N, bs, K, ctx0, rounds = 3, 6, 4, 3, 9, 12
    R = K + 1
    M = math.ceil((ctx0 + (rounds + 1) * R) / bs)
    P = B * N * M
    T, rc, fl, top = _initial(B, N, M, bs, P, ctx0, shared)
    L = ctx0
    st = orc.kv_reassign(np.tile(np.arange(N, dtype=np.int32), (B, 1)), np.zeros(B, np.int32), T,
                         bs, L, R, rc, fl, top)
    assert oracle.kv_check(st["tables"], math.ceil((L + R) / bs), st["refcounts"], st["free_list"],
                           st["free_top"]).tolist() == [0] * 5
    for t in range(rounds):
        L += R
        anc = np.sort(rng.integers(0, N, (B, N)), axis=1).astype(np.int32)
        res = (rng.random(B) < 0.7).astype(np.int32)
        st = orc.kv_reassign(anc, res, st["tables"], bs, L, R, st["refcounts"], st["free_list"],
                             st["free_top"])
        assert oracle.kv_check(st["tables"], math.ceil((L + R) / bs), st["refcounts"],
                               st["free_list"], st["free_top"]).tolist() == [0] * 5, t
        _check_invariants(st, P)
