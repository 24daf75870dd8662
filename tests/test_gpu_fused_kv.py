"""smcsd_resample_kv_reassign against smcsd_resample followed by smcsd_kv_reassign.

Two copies of the same state run the same rounds, one through the fused entry point and
one through the two separate calls; every output must be bit-identical after every
round: ancestors, ESS, decisions, reset log-weights, block tables, refcounts, free stack,
copy-on-write list and status.  Covers the one-wave resample (N <= 64: one column segment
for N <= 16, several above) and the workgroup resample (N > 64), shared and unshared
prefixes, prompts with degenerate (NaN) weights, the many-sequence KV path, the two forms
alternating on one workspace, and the exact KV shapes of the benchmark's workloads (B = 32,
N = 16, 16-token blocks, shared 2048-token prefix, tables of 128 to 285 columns in one
column tile; B = 8, N = 128, 256 shared blocks, split over several workgroups per prompt).
Every round of the fused form is also checked against the oracle in lock-step: the
resample against the oracle's on the same log-weights (a differing decision or ancestor is
allowed only where the oracle's margin is below 1e-6), the KV state against the oracle's
reassign given the ancestors the GPU drew.
"""

import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm
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


class _State:
    def __init__(self, kv, B, N, P):
        self.tables = torch.from_numpy(kv["tables"].copy()).cuda()
        self.rc = torch.from_numpy(kv["refcounts"].copy()).cuda()
        self.fl = torch.from_numpy(kv["free_list"].copy()).cuda()
        self.top = torch.from_numpy(kv["free_top"].copy()).cuda()
        self.cow, self.ncow, self.st = _i32(B * N, 3), _i32(1), _i32(1)
        self.anc, self.res = _i32(B, N), _i32(B)
        self.ess = torch.zeros(B, device="cuda")
        self.ws = sm.alloc_workspace(sm.OP_KV, B, N, P=P)

    def snapshot(self, lw):
        n = int(self.ncow.cpu()[0])
        return dict(anc=self.anc.cpu().numpy(), res=self.res.cpu().numpy(),
                    ess=self.ess.cpu().numpy(), lw=lw.cpu().numpy(),
                    tables=self.tables.cpu().numpy(), rc=self.rc.cpu().numpy(),
                    top=int(self.top.cpu()[0]), fl=self.fl.cpu().numpy(), cow=self.cow.cpu().numpy()[:n],
                    ncow=n, st=int(self.st.cpu()[0]))


def _equal(a, b):
    top = a["top"]
    for k in ("anc", "res", "ess", "lw", "tables", "rc", "cow"):
        # NaN log-weights of a degenerate prompt stay NaN on both sides
        if not np.array_equal(a[k], b[k], equal_nan=a[k].dtype.kind == "f"):
            return k
    for k in ("top", "ncow", "st"):
        if a[k] != b[k]:
            return k
    if not np.array_equal(a["fl"][:top], b["fl"][:top]):
        return "fl"
    return None


@pytest.mark.parametrize("B,N,shared", [(3, 16, True), (2, 5, False), (3, 40, True), (2, 64, False),
                                        (2, 128, True), (40, 256, False)])
def test_fused_equals_separate_calls(B, N, shared):
    _fused_vs_separate(B, N, shared, bs=4, ctx0=10)


@pytest.mark.parametrize("B,N,shared,bs,ctx0", [(3, 128, True, 4, 300), (2, 64, False, 2, 300),
                                                (2, 16, True, 1, 600), (1, 1024, False, 4, 40),
                                                (2, 40, True, 3, 700), (40, 256, False, 4, 160)])
def test_fused_equals_separate_calls_split_tables(B, N, shared, bs, ctx0):
    """Tables of more than one 32 KiB column tile per prompt (N * blocks > 8192): the exchange
    runs in several workgroups per prompt, each resampling the prompt itself, and the pop
    kernel resets the log-weights; every output must equal the two separate calls'.  The last
    case also takes the many-sequence pop path (B * N > 8192)."""
    assert N * (ctx0 // bs) > 8192
    _fused_vs_separate(B, N, shared, bs=bs, ctx0=ctx0)


@pytest.mark.parametrize("ctx0", [2048, 2600, 3700, 4530])
def test_fused_equals_separate_calls_c3_kv_shape(ctx0):
    """B = 32 prompts of N = 16 particles, K = 4, 16-token blocks and a shared prefix: the
    benchmark's C3 step, at contexts from its first round (128 columns) to its last (285
    columns, one 32 KiB column tile per prompt, several columns per thread)."""
    _fused_vs_separate(32, 16, True, bs=16, ctx0=ctx0, K=4, rounds=5, tau=0.5)


def test_fused_equals_separate_calls_c5_kv_shape():
    """B = 8 prompts of N = 128, K = 5, 4096-token shared prefixes in 16-token blocks (256
    blocks per particle), tau = 0.3: the C5 step, split over several workgroups per prompt."""
    _fused_vs_separate(8, 128, True, bs=16, ctx0=4096, K=5, rounds=4, tau=0.3)


def _fused_vs_separate(B, N, shared, bs, ctx0, K=2, rounds=6, tau=0.6):
    R = K + 1
    cfg = C.C1.scaled(B=B, N=N, K=K, ctx0=ctx0, block_size=bs, shared_prefix=shared, iters=rounds)
    kv = synth.initial_kv(cfg)
    P = kv["refcounts"].size
    A, F = _State(kv, B, N, P), _State(kv, B, N, P)
    ident = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    zero = _i32(B)
    L = ctx0
    for s in (A, F):
        sm.kv_reassign(ident, zero, B, N, s.tables, bs, L, R, s.rc, s.fl, s.top, s.cow, s.ncow, s.st,
                       s.ws)
    g = torch.Generator(device="cuda").manual_seed(B * 1000 + N)
    lw_a = torch.zeros(B * N, device="cuda")
    lw_f = torch.zeros(B * N, device="cuda")
    tau32 = float(np.float32(tau))
    saw_degenerate = False
    for r in range(rounds):
        L += R
        A.st.zero_()
        F.st.zero_()
        inc = torch.randn(B * N, generator=g, device="cuda") * (0.3 + r)
        if r == 2:
            inc[:N] = float("nan")            # prompt 0: degenerate weights this round
        lw_a += inc
        lw_f += inc
        lw_in = lw_f.cpu().numpy().copy()
        tables_in, rc_in = F.tables.cpu().numpy(), F.rc.cpu().numpy()
        fl_in, top_in = F.fl.cpu().numpy(), int(F.top.cpu()[0])
        sm.resample(lw_a.view(B, N), B, N, tau32, 77, r, A.anc, A.ess, A.res, A.st)
        sm.kv_reassign(A.anc, A.res, B, N, A.tables, bs, L, R, A.rc, A.fl, A.top, A.cow, A.ncow,
                       A.st, A.ws)
        if r % 3 == 1:   # F's workspace also serves the separate calls between fused ones
            sm.resample(lw_f.view(B, N), B, N, tau32, 77, r, F.anc, F.ess, F.res, F.st)
            sm.kv_reassign(F.anc, F.res, B, N, F.tables, bs, L, R, F.rc, F.fl, F.top, F.cow,
                           F.ncow, F.st, F.ws)
        else:
            sm.resample_kv_reassign(lw_f.view(B, N), B, N, tau32, 77, r, F.anc, F.ess, F.res,
                                    F.tables, bs, L, R, F.rc, F.fl, F.top, F.cow, F.ncow, F.st,
                                    F.ws)
        torch.cuda.synchronize()
        a, f = A.snapshot(lw_a), F.snapshot(lw_f)
        bad = _equal(a, f)
        assert bad is None, (r, bad)
        # lock-step against the oracle, every round
        o = oracle.resample(lw_in.reshape(B, N), tau32, 77, r)
        for b in range(B):
            if o["margin_ess"][b] >= 1e-6:
                assert f["res"][b] == o["resampled"][b], (r, b)
            if f["res"][b] == o["resampled"][b] and o["resampled"][b]:
                m = o["margin_pos"][b] >= 1e-6
                assert np.array_equal(f["anc"][b][m], o["ancestors"][b][m]), (r, b)
        ok = oracle.kv_reassign(f["anc"], f["res"], tables_in, bs, L, R, rc_in, fl_in, top_in)
        assert np.array_equal(f["tables"], ok["tables"]), r
        assert np.array_equal(f["rc"], ok["refcounts"]), r
        assert f["top"] == ok["free_top"] and f["ncow"] == ok["cow_count"], r
        assert np.array_equal(f["fl"][:f["top"]], ok["free_list"][:f["top"]]), r
        assert np.array_equal(f["cow"], ok["cow"]), r
        assert f["st"] == o["status"] | ok["status"], (r, f["st"], o["status"], ok["status"])
        saw_degenerate |= bool(f["st"] & sm.ST_DEGENERATE_WEIGHTS)
    if N <= 64:
        assert (a["res"] == 1).any()          # the rounds did resample
    assert saw_degenerate


def test_fused_rejects_what_either_call_rejects():
    B, N, P = 2, 4, 64
    lw = torch.zeros(B * N, device="cuda")
    anc, res, ess = _i32(B, N), _i32(B), torch.zeros(B, device="cuda")
    tables = torch.full((B * N, 8), -1, dtype=torch.int32, device="cuda")
    rc, fl, top = _i32(P), _i32(P), _i32(1)
    cow, ncow, st = _i32(B * N, 3), _i32(1), _i32(1)
    ws = sm.alloc_workspace(sm.OP_KV, B, N, P=P)
    with pytest.raises(sm.SmcsdError):
        sm.resample_kv_reassign(lw, B, N, float("nan"), 1, 0, anc, ess, res, tables, 4, 0, 1, rc, fl,
                                top, cow, ncow, st, ws)
    with pytest.raises(sm.SmcsdError):      # reservation beyond M_cap
        sm.resample_kv_reassign(lw, B, N, 0.5, 1, 0, anc, ess, res, tables, 4, 30, 8, rc, fl, top,
                                cow, ncow, st, ws)
    with pytest.raises(sm.SmcsdError):      # workspace too small
        sm.resample_kv_reassign(lw, B, N, 0.5, 1, 0, anc, ess, res, tables, 4, 0, 1, rc, fl, top,
                                cow, ncow, st, ws[:64])
