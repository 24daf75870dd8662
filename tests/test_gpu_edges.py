"""GPU edge cases, each checked against the oracle through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm
from tests import gpu_harness as H
from workloads import configs as C
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def _verify_case(target, draft, toks, K, V, T, alpha, seed, step, lw0, row_stride=None,
                 mode=sm.MODE_SMC):
    """One SMC verify on the GPU vs the oracle; returns (gpu dict, oracle dict)."""
    S = toks.shape[0]
    out = dict(tokens=_i32(S, K + 1), num=_i32(S), logp=_f32(S, K + 1), logq=_f32(S, max(K, 1)),
               lse=_f32(S, 2 * K + 1), status=_i32(1))
    lw = torch.tensor(lw0, dtype=torch.float32, device="cuda")
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, S, 1, K, V)
    sm.verify(target, draft, toks, S, 1, K, V, T, alpha, mode, seed, step, out["tokens"],
              out["status"], ws, log_weights=lw, out_num_tokens=out["num"], out_logp=out["logp"],
              out_logq=out["logq"], out_lse=out["lse"], row_stride=row_stride)
    torch.cuda.synchronize()
    rs = V if row_stride is None else row_stride
    th = H.host_logits(target).reshape(S, K + 1, rs)[:, :, :V]
    dh = H.host_logits(draft).reshape(S, K, rs)[:, :, :V] if K else \
        np.zeros((S, 0, V), th.dtype)
    o = oracle.verify_smc(np.ascontiguousarray(th), np.ascontiguousarray(dh),
                          toks.cpu().numpy(), float(np.float32(T)), float(np.float32(alpha)), seed,
                          step, np.asarray(lw0, np.float32),
                          bonus="race" if mode == sm.MODE_SMC_RACE else "cdf")
    g = {k: v.cpu().numpy() for k, v in out.items()}
    g["lw"] = lw.cpu().numpy()
    return g, o


def _assert_verify_parity(g, o, K, margin=H.MARGIN):
    assert int(g["status"][0]) == o["status"]
    assert np.array_equal(g["tokens"][:, :K], o["tokens"][:, :K])
    for i in range(len(o["lw"])):
        if o["margin"][i] >= margin:
            assert g["tokens"][i, K] == o["tokens"][i, K], (i, o["margin"][i])
            assert abs(g["lw"][i] - o["lw"][i]) <= H.TOL_LW
    fin = np.isfinite(o["lse"])
    assert np.all(np.abs(g["lse"][fin] - o["lse"][fin]) <= H.TOL_LSE_REL * np.abs(o["lse"][fin]))


@pytest.mark.parametrize("dtype,V,pad", [("bf16", 1001, 0), ("bf16", 1001, 3), ("f32", 37, 2),
                                         ("bf16", 1, 0), ("f32", 5, 0), ("bf16", 16385, 1),
                                         ("f32", 8193, 0), ("bf16", 32768, 0),
                                         ("bf16", 65536, 0), ("bf16", 65535, 0), ("bf16", 65537, 5),
                                         ("f32", 16384, 0), ("f32", 16383, 1),
                                         ("bf16", 32767, 0), ("bf16", 32769, 3),
                                         ("f32", 32768, 0), ("f32", 32767, 0), ("f32", 32769, 1),
                                         ("f32", 65537, 0)])
def test_ragged_and_misaligned_rows(dtype, V, pad):
    """Rows whose length or stride is not a multiple of the 16-byte vector (so rows start
    misaligned), single-element rows, and tiles split one element past a boundary; rows
    made only of whole load groups (8 vectors per lane over the workgroup) and rows one
    element short of or past them; rows at one or two times the big-tile bound (32768
    elements) and one element short of or past it, where a row's big tiles share it
    equally (32769 elements: two tiles of 16392 and 16377, whole vectors each; with a
    padded stride every tile also starts misaligned)."""
    K, S = 3, 5
    rs = V + pad
    g = torch.Generator(device="cuda").manual_seed(V * 7 + pad)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tgt = (2 * torch.randn((S, K + 1, rs), generator=g, device="cuda")).to(dt)
    drf = (tgt[:, :K].float() + torch.randn((S, K, rs), generator=g, device="cuda")).to(dt)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _verify_case(tgt, drf, toks, K, V, 0.8, 1.0, 77, 5, np.zeros(S), row_stride=rs)
    _assert_verify_parity(gg, o, K)


@pytest.mark.parametrize("K", [0, 1, 32])
def test_k_extremes(K):
    S, V = 4, 3000
    g = torch.Generator(device="cuda").manual_seed(K + 11)
    tgt = torch.randn((S, K + 1, V), generator=g, device="cuda").to(torch.bfloat16)
    drf = torch.randn((S, max(K, 1), V), generator=g, device="cuda").to(torch.bfloat16)[:, :K]
    drf = drf.contiguous()
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _verify_case(tgt, drf, toks, K, V, 1.0, 4.0, 3, 9, np.full(S, 0.25))
    _assert_verify_parity(gg, o, K)


def test_masked_empty_and_nan_rows():
    S, K, V = 4, 2, 700
    tgt = torch.zeros((S, K + 1, V), dtype=torch.float32, device="cuda")
    drf = torch.zeros((S, K, V), dtype=torch.float32, device="cuda")
    tgt[0, K, :] = -math.inf
    tgt[0, K, 123] = 2.0                    # one-hot bonus row
    tgt[1, K, :] = -math.inf
    tgt[1, K, [5, 600]] = 0.0              # two tokens, everything else masked
    toks = torch.zeros((S, K), dtype=torch.int32, device="cuda")
    gg, o = _verify_case(tgt, drf, toks, K, V, 1.0, 1.0, 1, 2, np.zeros(S))
    _assert_verify_parity(gg, o, K)
    assert gg["tokens"][0, K] == 123 and gg["tokens"][1, K] in (5, 600)
    # an all -inf draft row -> EMPTY_ROW; a NaN -> NAN_INPUT (same bits on both sides)
    drf[2, 1, :] = -math.inf
    tgt[3, 0, 17] = math.nan
    gg, o = _verify_case(tgt, drf, toks, K, V, 1.0, 1.0, 1, 2, np.zeros(S))
    assert int(gg["status"][0]) == o["status"] == sm.ST_EMPTY_ROW | sm.ST_NAN_INPUT


def test_bad_token_flagged_not_faulting():
    S, K, V = 2, 2, 100
    tgt = torch.zeros((S, K + 1, V), dtype=torch.float32, device="cuda")
    drf = torch.zeros((S, K, V), dtype=torch.float32, device="cuda")
    toks = torch.tensor([[0, 1], [V, -1]], dtype=torch.int32, device="cuda")
    st = _i32(1)
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, S, 1, K, V)
    sm.verify(tgt, drf, toks, S, 1, K, V, 1.0, 1.0, sm.MODE_SMC, 0, 0, _i32(S, K + 1), st, ws,
              log_weights=_f32(S))
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) & sm.ST_BAD_INPUT


def test_philox_bit_exact_against_oracle():
    rng = np.random.default_rng(4)
    n = 4096
    ctr = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, (n, 2), dtype=np.uint64).astype(np.uint32)
    out = _i32(n, 4)
    sm.philox4x32_10(torch.from_numpy(ctr.view(np.int32)).cuda(),
                     torch.from_numpy(key.view(np.int32)).cuda(), out)
    got = out.cpu().numpy().view(np.uint32)
    ref = np.stack([oracle.philox4x32_10(c, k) for c, k in zip(ctr, key)])
    assert np.array_equal(got, ref)


def test_philox_known_answer_vectors_on_device():
    from tests.test_oracle_rng import load_kat
    ctr, key, ref = load_kat()
    out = _i32(len(ctr), 4)
    sm.philox4x32_10(torch.from_numpy(ctr.view(np.int32)).cuda(),
                     torch.from_numpy(key.view(np.int32)).cuda(), out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref)


@pytest.mark.parametrize("N", [1, 2, 3, 64, 1000, 1024])
def test_resample_particle_counts(N):
    B = 7
    rng = np.random.default_rng(N)
    lw0 = rng.normal(0, 2.0, (B, N)).astype(np.float32)
    lw0[1] = 0.0                            # equal weights: ESS = N exactly
    lw0[2] = -np.inf
    lw0[2, N // 2] = 0.0                    # one live particle
    for tau in (0.5, 1.5):
        lw = torch.from_numpy(lw0.copy()).cuda()
        anc, ess, res, st = _i32(B, N), _f32(B), _i32(B), _i32(1)
        sm.resample(lw, B, N, tau, 99, 3, anc, ess, res, st)
        torch.cuda.synchronize()
        o = oracle.resample(lw0, float(np.float32(tau)), 99, 3)
        assert int(st.cpu()[0]) == o["status"]
        gres, ganc = res.cpu().numpy(), anc.cpu().numpy()
        for b in range(B):
            if o["margin_ess"][b] >= H.MARGIN:
                assert gres[b] == o["resampled"][b]
                if gres[b]:
                    ok = o["margin_pos"][b] >= H.MARGIN
                    assert np.array_equal(ganc[b][ok], o["ancestors"][b][ok])
            assert abs(ess.cpu().numpy()[b] - o["ess"][b]) <= 1e-6 * o["ess"][b]


def test_resample_degenerate_weights():
    lw0 = np.full((2, 8), -np.inf, np.float32)
    lw0[1, 3] = np.nan
    lw = torch.from_numpy(lw0).cuda()
    anc, ess, res, st = _i32(2, 8), _f32(2), _i32(2), _i32(1)
    sm.resample(lw, 2, 8, 0.5, 1, 1, anc, ess, res, st)
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == sm.ST_DEGENERATE_WEIGHTS
    assert np.array_equal(anc.cpu().numpy(), np.tile(np.arange(8), (2, 1)))
    assert np.all(res.cpu().numpy() == 0)


_KV_WS = {}


def _kv_gpu(anc, res, B, N, T, bs, L, R, rc, fl, top):
    """One smcsd_kv_reassign call on copies of the given state.  The workspace of a shape is
    reused across calls (as a caller would), so successive calls alternate its buffers."""
    tables = torch.from_numpy(T.copy()).cuda()
    rcd = torch.from_numpy(rc.copy()).cuda()
    fld = torch.from_numpy(fl.copy()).cuda()
    topd = torch.tensor([top], dtype=torch.int32, device="cuda")
    cow, ncow, st = _i32(B * N, 3), _i32(1), _i32(1)
    key = (B, N, rc.size)
    if key not in _KV_WS:
        _KV_WS[key] = sm.alloc_workspace(sm.OP_KV, B, N, P=rc.size)
    ws = _KV_WS[key]
    sm.kv_reassign(torch.from_numpy(anc).cuda(), torch.from_numpy(res).cuda(), B, N, tables, bs, L,
                   R, rcd, fld, topd, cow, ncow, st, ws)
    torch.cuda.synchronize()
    n = int(ncow.cpu()[0])
    return dict(tables=tables.cpu().numpy(), refcounts=rcd.cpu().numpy(),
                free_list=fld.cpu().numpy(), free_top=int(topd.cpu()[0]), cow=cow.cpu().numpy()[:n],
                cow_count=n, status=int(st.cpu()[0]))


def _kv_equal(g, o):
    top = o["free_top"]
    return (g["status"] == o["status"] and g["free_top"] == top and g["cow_count"] == o["cow_count"]
            and np.array_equal(g["tables"], o["tables"])
            and np.array_equal(g["refcounts"], o["refcounts"])
            and np.array_equal(g["free_list"][:top], o["free_list"][:top])
            and np.array_equal(g["cow"], o["cow"]))


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("N", [1, 5, 128, 1024])
def test_kv_random_rounds(shared, N):
    """Random (also unsorted) ancestor maps over several rounds, bit-exact vs the oracle."""
    B, bs, K, ctx0, rounds = 3, 4, 2, 10, 6
    R = K + 1
    M = math.ceil((ctx0 + (rounds + 1) * R) / bs)
    cfg = C.C1.scaled(B=B, N=N, K=K, ctx0=ctx0, block_size=bs, shared_prefix=shared,
                      iters=rounds)
    kv = synth.initial_kv(cfg)
    T, rc, fl, top, L = kv["tables"], kv["refcounts"], kv["free_list"], int(kv["free_top"][0]), ctx0
    assert T.shape[1] == M
    rng = np.random.default_rng(N * 3 + shared)
    ident = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    o = oracle.kv_reassign(ident, np.zeros(B, np.int32), T, bs, L, R, rc, fl, top)
    g = _kv_gpu(ident, np.zeros(B, np.int32), B, N, T, bs, L, R, rc, fl, top)
    assert _kv_equal(g, o)
    for r in range(rounds):
        T, rc, fl, top = o["tables"], o["refcounts"], o["free_list"], o["free_top"]
        L += R
        anc = rng.integers(0, N, (B, N)).astype(np.int32)
        if r % 2 == 0:
            anc.sort(axis=1)
        res = (rng.random(B) < 0.7).astype(np.int32)
        o = oracle.kv_reassign(anc, res, T, bs, L, R, rc, fl, top)
        g = _kv_gpu(anc, res, B, N, T, bs, L, R, rc, fl, top)
        assert _kv_equal(g, o), r


def test_kv_nospace_and_bad_ancestor():
    B, N, bs, M = 1, 2, 4, 6
    cfg = C.C1.scaled(B=B, N=N, K=8, ctx0=4, block_size=bs, iters=0)
    kv = synth.initial_kv(cfg)
    P = 5
    T = kv["tables"][:, :M].copy()
    rc = np.zeros(P, np.int32)
    rc[[0, 1]] = 1
    fl = np.arange(P - 1, -1, -1, dtype=np.int32)
    ident = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    o = oracle.kv_reassign(ident, np.zeros(B, np.int32), T, bs, 4, 9, rc, fl, 3)
    g = _kv_gpu(ident, np.zeros(B, np.int32), B, N, T, bs, 4, 9, rc, fl, 3)
    assert o["status"] == sm.ST_NOSPACE and _kv_equal(g, o)
    bad = np.array([[0, 7]], np.int32)
    g = _kv_gpu(bad, np.ones(B, np.int32), B, N, T, bs, 4, 0, rc, fl, 3)
    assert g["status"] & sm.ST_BAD_INPUT
    assert np.array_equal(g["tables"], T)


@pytest.mark.parametrize("N,shared", [(2, False), (5, True), (16, True), (40, False), (40, True)])
def test_kv_after_nospace_and_bad_indices_match_the_oracle(N, shared):
    """A pool too small for the reservations: NOSPACE leaves -1 in allocated slots, which
    later resampling rounds (random ancestors) must flag and skip exactly as the oracle does;
    then an out-of-range ancestor and a corrupt free-stack entry.  Bit-exact every call."""
    B, bs, K, ctx0, rounds = 3, 4, 2, 9, 6
    R = K + 1
    M = math.ceil((ctx0 + (rounds + 2) * R) / bs)
    cfg = C.C1.scaled(B=B, N=N, K=K, ctx0=ctx0, block_size=bs, shared_prefix=shared,
                      iters=rounds + 1)
    assert cfg.M_cap == M
    kv = synth.initial_kv(cfg)
    used = int(kv["refcounts"].astype(bool).sum())
    P = used + (B * N) // 2 + 1                              # room for about half a round
    T = kv["tables"][:, :M].copy()
    rc = kv["refcounts"][:P].copy()
    fl = np.arange(P - 1, -1, -1, dtype=np.int32)
    top, L = P - used, ctx0
    rng = np.random.default_rng(N * 7 + shared)
    ident = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    seen = 0
    for r in range(rounds + 2):
        if r == 0:
            anc, res = ident, np.zeros(B, np.int32)
        else:
            L += R
            anc = np.sort(rng.integers(0, N, (B, N)), axis=1).astype(np.int32)
            res = np.ones(B, np.int32)
            if r == rounds:
                anc[1, 0] = N + 2                            # prompt 1: a bad ancestor
            if r == rounds + 1 and top > 0:
                fl = fl.copy()
                fl[top - 1] = P + 9                          # a corrupt entry on the stack
        o = oracle.kv_reassign(anc, res, T, bs, L, R, rc, fl, top)
        g = _kv_gpu(anc, res, B, N, T, bs, L, R, rc, fl, top)
        assert _kv_equal(g, o), (r, g["status"], o["status"])
        seen |= o["status"]
        T, rc, fl, top = o["tables"], o["refcounts"], o["free_list"], o["free_top"]
    assert seen & sm.ST_NOSPACE and seen & sm.ST_BAD_INPUT


def test_empty_batch_is_noop():
    st = _i32(1)
    sm.verify(_f32(1, 2, 4), _f32(1, 1, 4), _i32(1, 1), 0, 4, 1, 4, 1.0, 1.0, sm.MODE_SMC, 0, 0,
              _i32(1, 2), st, sm.alloc_workspace(sm.OP_VERIFY_SMC, 1, 1, 1, 4),
              log_weights=_f32(1))
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == 0


def _final_state(p):
    return [x.cpu().numpy().copy() for x in (p.lw, p.tables, p.rc, p.free_list, p.free_top,
                                             p.tokens, p.anc)]


def test_determinism_and_resume():
    """Two runs are bit-identical; 6 rounds + copy of the state + 6 rounds equals 12 rounds
    straight (the counter-based RNG depends only on seed, round and index)."""
    cfg = C.downsized(C.C3, B=2, V=50000, iters=12)
    a = H.Pipeline(cfg, check=False)
    for t in range(12):
        a.round(t)
    b = H.Pipeline(cfg, check=False)
    for t in range(12):
        b.round(t)
    torch.cuda.synchronize()
    for x, y in zip(_final_state(a), _final_state(b)):
        assert np.array_equal(x, y)
    c = H.Pipeline(cfg, check=False)
    for t in range(6):
        c.round(t)
    torch.cuda.synchronize()
    saved = {k: getattr(c, k).clone() for k in ("lw", "tables", "rc", "free_list", "free_top")}
    L = c.L
    d = H.Pipeline(cfg, check=False)
    for k, v in saved.items():
        getattr(d, k).copy_(v)
    d.L = L
    for t in range(6, 12):
        d.round(t)
    torch.cuda.synchronize()
    for x, y in zip(_final_state(a), _final_state(d)):
        assert np.array_equal(x, y)


def test_kv_more_sequences_than_the_lds_prefix():
    """B*N above the 8192 sequences whose allocation offsets fit in LDS: the pops take the
    per-thread path."""
    B, N, bs, K, ctx0, rounds = 9, 1024, 4, 2, 6, 3
    R = K + 1
    cfg = C.C1.scaled(B=B, N=N, K=K, ctx0=ctx0, block_size=bs, shared_prefix=True, iters=rounds)
    kv = synth.initial_kv(cfg)
    T, rc, fl, top, L = kv["tables"], kv["refcounts"], kv["free_list"], int(kv["free_top"][0]), ctx0
    rng = np.random.default_rng(5)
    ident = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    o = oracle.kv_reassign(ident, np.zeros(B, np.int32), T, bs, L, R, rc, fl, top)
    g = _kv_gpu(ident, np.zeros(B, np.int32), B, N, T, bs, L, R, rc, fl, top)
    assert _kv_equal(g, o)
    for r in range(rounds):
        T, rc, fl, top = o["tables"], o["refcounts"], o["free_list"], o["free_top"]
        L += R
        anc = np.sort(rng.integers(0, N, (B, N)), axis=1).astype(np.int32)
        res = (rng.random(B) < 0.8).astype(np.int32)
        o = oracle.kv_reassign(anc, res, T, bs, L, R, rc, fl, top)
        g = _kv_gpu(anc, res, B, N, T, bs, L, R, rc, fl, top)
        assert _kv_equal(g, o), r


def test_many_chunks_per_sequence():
    """K=32 with a long fp32 row: more chunk pairs per sequence than the finalize stages in
    LDS, so it reads them in place."""
    S, K, V = 2, 32, 140001
    g = torch.Generator(device="cuda").manual_seed(3)
    tgt = torch.randn((S, K + 1, V), generator=g, device="cuda")
    drf = tgt[:, :K] + torch.randn((S, K, V), generator=g, device="cuda")
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _verify_case(tgt, drf.contiguous(), toks, K, V, 0.8, 1.0, 5, 6, np.zeros(S))
    _assert_verify_parity(gg, o, K)


@pytest.mark.parametrize("dtype,mode", [("bf16", sm.MODE_SMC), ("f32", sm.MODE_SMC),
                                        ("bf16", sm.MODE_SMC_RACE)])
def test_maximum_vocabulary(dtype, mode):
    """V = 2^24, the largest vocabulary the library takes: 1024 (bf16) or 2048 (fp32) chunks
    per row, so the finalize's chunk terms fill their LDS array and the slab sums are read in
    place; in race mode the clock counters reach (v div 4) = 2^22 - 1."""
    S, K, V = 2, 1, 1 << 24
    g = torch.Generator(device="cuda").manual_seed(24)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tgt = (torch.randn((S, K + 1, V), generator=g, device="cuda") * 1.5).to(dt)
    drf = (torch.randn((S, K, V), generator=g, device="cuda") * 1.5).to(dt)
    toks = torch.tensor([[V - 1], [12345]], dtype=torch.int32, device="cuda")
    gg, o = _verify_case(tgt, drf, toks, K, V, 0.9, 2.0, 13, 4, np.array([0.0, -1.0]), mode=mode)
    _assert_verify_parity(gg, o, K, margin=1e-4 if mode == sm.MODE_SMC_RACE else H.MARGIN)
    assert np.all((gg["tokens"][:, K] >= 0) & (gg["tokens"][:, K] < V))


@pytest.mark.parametrize("L,R", [(12, 0), (8, 4), (10, 2), (9, 0)])
def test_kv_table_filled_to_capacity(L, R):
    """The reservation reaches the last slot (or the table is already full): one sequence
    whose table has exactly M_cap slots."""
    B, N, bs, M = 1, 1, 4, 3
    P = 8
    T = np.full((1, M), -1, np.int32)
    nb = math.ceil(L / bs)
    T[0, :nb] = np.arange(nb)
    rc = np.zeros(P, np.int32)
    rc[:nb] = 1
    fl = np.zeros(P, np.int32)
    free = list(range(P - 1, nb - 1, -1))
    fl[:len(free)] = free
    anc = np.zeros((1, 1), np.int32)
    for res in (0, 1):
        o = oracle.kv_reassign(anc, np.array([res], np.int32), T, bs, L, R, rc, fl, len(free))
        g = _kv_gpu(anc, np.array([res], np.int32), B, N, T, bs, L, R, rc, fl, len(free))
        assert _kv_equal(g, o)


def _tiny_rows(n, rows, V, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((n, rows, V), generator=g, device="cuda") * 1.5


@pytest.mark.parametrize("mode", ["smc", "sps", "resample_wave", "resample_block"])
def test_batches_beyond_one_dispatch(mode):
    """Batches whose one-workgroup-per-item kernels would need more than 2^32 threads (the
    width of a dispatch): the kernels stride over their items with a capped grid, and every
    item's result still matches the oracle."""
    V = 8
    if mode == "smc":                      # finalize: 256 threads per sequence
        S, K = (1 << 24) + 1000, 0
        tgt = _tiny_rows(S, 1, V, 1)
        drf = torch.zeros((S, 0, V), device="cuda")
        toks = _i32(S, 0)
        out, st = _i32(S, 1), _i32(1)
        lw = torch.zeros(S, device="cuda")
        ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, S, 1, K, V)
        sm.verify(tgt, drf, toks, S, 1, K, V, 1.0, 1.0, sm.MODE_SMC, 3, 4, out, st, ws, log_weights=lw)
        torch.cuda.synchronize()
        o = oracle.verify_smc(tgt.cpu().numpy(), np.zeros((S, 0, V), np.float32),
                              np.zeros((S, 0), np.int32), 1.0, 1.0, 3, 4, np.zeros(S, np.float32))
        ok = o["margin"] >= H.MARGIN
        g = out.cpu().numpy()[:, 0]
        assert int(st.cpu()[0]) == o["status"] == 0
        assert np.array_equal(g[ok], o["tokens"][ok, 0]) and (g >= 0).all()
        assert np.max(np.abs(lw.cpu().numpy() - o["lw"])) <= H.TOL_LW
    elif mode == "sps":                    # SpS residual + draw: 256 threads per sequence
        S, K = (1 << 24) + 300, 1
        tgt = _tiny_rows(S, K + 1, V, 2)
        drf = (tgt[:, :K] + _tiny_rows(S, K, V, 3)).contiguous()
        toks = torch.randint(0, V, (S, K), device="cuda", dtype=torch.int32)
        out, num, st = _i32(S, K + 1), _i32(S), _i32(1)
        ws = sm.alloc_workspace(sm.OP_VERIFY_SPS, S, 1, K, V)
        sm.verify(tgt, drf, toks, S, 1, K, V, 1.0, 1.0, sm.MODE_SPS, 5, 6, out, st, ws,
                  out_num_tokens=num)
        torch.cuda.synchronize()
        o = oracle.verify_sps(tgt.cpu().numpy(), drf.cpu().numpy(), toks.cpu().numpy(), 1.0, 5, 6)
        ok = np.minimum(o["margin_accept"], o["margin_final"]) >= H.MARGIN
        assert int(st.cpu()[0]) == o["status"]
        assert np.array_equal(num.cpu().numpy()[ok], o["num_tokens"][ok])
        assert np.array_equal(out.cpu().numpy()[ok], o["tokens"][ok])
    else:                                  # resample: one wave or one workgroup per prompt
        N = 2 if mode == "resample_wave" else 65
        B = (1 << 24) + 77 if mode == "resample_wave" else (1 << 22) + 77
        g = torch.Generator(device="cuda").manual_seed(B)
        lw = torch.randn((B, N), generator=g, device="cuda") * 2.0
        lw_in = lw.cpu().numpy()
        anc, ess, res, st = _i32(B, N), torch.zeros(B, device="cuda"), _i32(B), _i32(1)
        sm.resample(lw, B, N, 0.6, 7, 8, anc, ess, res, st)
        torch.cuda.synchronize()
        o = oracle.resample(lw_in, float(np.float32(0.6)), 7, 8)
        ok = o["margin_ess"] >= H.MARGIN
        assert np.array_equal(res.cpu().numpy()[ok], o["resampled"][ok])
        a = anc.cpu().numpy()
        both = ok & (o["resampled"] == 1)
        okp = both[:, None] & (o["margin_pos"] >= H.MARGIN)
        assert np.array_equal(a[okp], o["ancestors"][okp])
        kept = ok & (o["resampled"] == 0)
        assert (a[kept] == np.arange(N)[None, :]).all()
        e = ess.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(e - o["ess"]) / o["ess"]) <= H.TOL_ESS_REL
