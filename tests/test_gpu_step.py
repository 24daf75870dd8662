"""smcsd_step (one whole SMC-SD round: verify, then resample + KV exchange) against
smcsd_verify followed by smcsd_resample_kv_reassign on a copy of the same state: every
output must be bit-identical after every round - tokens, counts, log-probabilities, row
normalisers, log-weights, ancestors, ESS, decisions, block tables, refcounts, free stack,
copy-on-write list and status.  The shapes cover the benchmark's C3 shape, small N, the
race bonus, fp32 logits, the draft's log q, K = 0, a NaN row, N > 16, tables split over
several workgroups and more than 8192 sequences.  Lock-step parity of smcsd_step against
the oracle at full size is in the harness (every third round)."""
import numpy as np
import pytest
import torch

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


class _Copy:
    """One copy of the round's state and outputs."""

    def __init__(self, cfg, kv, lw0, dev="cuda"):
        B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.lw = lw0.clone()
        self.tables = torch.from_numpy(kv["tables"].copy()).to(dev)
        self.rc = torch.from_numpy(kv["refcounts"].copy()).to(dev)
        self.fl = torch.from_numpy(kv["free_list"].copy()).to(dev)
        self.top = torch.from_numpy(kv["free_top"].copy()).to(dev)
        self.tok, self.num = torch.zeros((S, K + 1), **i32), torch.zeros(S, **i32)
        self.logp, self.logq = torch.zeros((S, K + 1), **f32), torch.zeros((S, max(K, 1)), **f32)
        self.lse = torch.zeros((S, 2 * K + 1), **f32)
        self.anc, self.ess, self.res = torch.zeros((B, N), **i32), torch.zeros(B, **f32), torch.zeros(B, **i32)
        self.cow, self.ncow, self.st = torch.zeros((S, 3), **i32), torch.zeros(1, **i32), torch.zeros(1, **i32)
        self.ws_v = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
        self.ws_kv = sm.alloc_workspace(sm.OP_KV, B, N, P=cfg.pool)

    def snapshot(self):
        n = int(self.ncow.cpu()[0])
        top = int(self.top.cpu()[0])
        d = {k: getattr(self, k).cpu().numpy() for k in
             ("lw", "tables", "rc", "tok", "num", "logp", "logq", "lse", "anc", "ess", "res")}
        d.update(fl=self.fl.cpu().numpy()[:top], top=top, cow=self.cow.cpu().numpy()[:n], st=int(self.st.cpu()[0]))
        return d


def _same(a, b):
    for k in a:
        x, y = a[k], b[k]
        if isinstance(x, np.ndarray):
            if x.dtype.kind == "f":
                x, y = x.view(np.int32), y.view(np.int32)   # bit-identical, NaN included
            if not np.array_equal(x, y):
                return k
        elif x != y:
            return k
    return None


def _run(cfg, rounds, mode=sm.MODE_SMC, draft_logq=False, nan_row=False):
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    base = synth.zipf_base(cfg, "cuda") if cfg.target_kind == "zipf" else None
    sets = []
    for s in range(cfg.n_sets):
        t, d = synth.make_logit_set(cfg, s, "cuda", base)
        if nan_row and s == 0:
            t[1, K, 5] = float("nan")
        x = synth.sample_draft_tokens(cfg, d, s)
        lq = None
        if draft_logq and K:
            lq = torch.randn((S, K), device="cuda") - 4.0     # any log q values will do
        sets.append((t, d, x, lq))
    kv = synth.initial_kv(cfg)
    g = torch.Generator(device="cuda").manual_seed(S + K)
    lw0 = torch.randn(S, generator=g, device="cuda")
    A, F = _Copy(cfg, kv, lw0), _Copy(cfg, kv, lw0)
    L = int(kv["seq_len"])
    ident = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    for c in (A, F):
        sm.kv_reassign(ident, torch.zeros(B, dtype=torch.int32, device="cuda"), B, N, c.tables,
                       cfg.block_size, L, K + 1, c.rc, c.fl, c.top, c.cow, c.ncow, c.st, c.ws_kv)
    resampled_any = False
    for t in range(rounds):
        tgt, drf, x, lq = sets[t % cfg.n_sets]
        L += K + 1
        for c in (A, F):
            c.st.zero_()
        # A: smcsd_verify, then smcsd_resample_kv_reassign
        sm.verify(tgt, None if lq is not None else drf, x, B, N, K, V, cfg.temperature, cfg.alpha,
                  mode, cfg.rng_seed, t, A.tok, A.st, A.ws_v, log_weights=A.lw, out_num_tokens=A.num,
                  out_logp=A.logp, out_logq=A.logq, out_lse=A.lse, logq_in=lq)
        sm.resample_kv_reassign(A.lw.view(B, N), B, N, cfg.tau, cfg.rng_seed, t, A.anc, A.ess, A.res,
                                A.tables, cfg.block_size, L, K + 1, A.rc, A.fl, A.top, A.cow, A.ncow,
                                A.st, A.ws_kv)
        # F: smcsd_step
        sm.step(tgt, None if lq is not None else drf, x, B, N, K, V, cfg.temperature, cfg.alpha, mode,
                cfg.tau, cfg.rng_seed, t, F.lw, F.tok, F.anc, F.ess, F.res, F.tables, cfg.block_size, L,
                K + 1, F.rc, F.fl, F.top, F.cow, F.ncow, F.st, F.ws_v, F.ws_kv, out_num_tokens=F.num,
                out_logp=F.logp, out_logq=F.logq, out_lse=F.lse, logq_in=lq)
        torch.cuda.synchronize()
        a, f = A.snapshot(), F.snapshot()
        bad = _same(a, f)
        assert bad is None, (t, bad)
        resampled_any |= bool(a["res"].any())
        if nan_row and t % cfg.n_sets == 0:
            assert a["st"] & sm.ST_NAN_INPUT
    assert resampled_any


@pytest.mark.parametrize("case", ["c3_shape", "n5_unshared", "race", "fp32", "draft_logq", "k0",
                                  "nan_row", "n40", "split_tables", "many_sequences"])
def test_step_equals_verify_then_fused_resample_kv(case):
    if case == "c3_shape":          # the benchmark's step shape at 4 prompts
        _run(C.C3.scaled(name="s", B=4, n_sets=2, iters=8), 6)
    elif case == "n5_unshared":
        _run(C.C2.scaled(name="s", B=3, N=5, V=20011, n_sets=2, iters=8), 6)
    elif case == "race":
        _run(C.C3.scaled(name="s", B=3, V=40000, n_sets=2, iters=8), 6, mode=sm.MODE_SMC_RACE)
    elif case == "fp32":
        _run(C.C4.scaled(name="s", B=3, N=16, V=30011, n_sets=2, iters=8, ctx0=256), 6)
    elif case == "draft_logq":
        _run(C.C3.scaled(name="s", B=3, V=30011, n_sets=2, iters=8), 6, draft_logq=True)
    elif case == "k0":
        _run(C.C2.scaled(name="s", B=3, K=0, V=5000, n_sets=2, iters=8, tau=0.9), 6)
    elif case == "nan_row":
        _run(C.C3.scaled(name="s", B=2, V=20011, n_sets=2, iters=8), 4, nan_row=True)
    elif case == "n40":              # N > 16: the exchange over a workgroup-wide resample
        _run(C.C3.scaled(name="s", B=2, N=40, V=20011, n_sets=2, iters=8), 5)
    elif case == "split_tables":     # tables over several column tiles (C5-like)
        _run(C.C5.scaled(name="s", B=1, N=128, V=20011, n_sets=2, iters=6), 4)
    else:                            # more than 8192 sequences: the many-sequence pop path
        _run(C.C2.scaled(name="s", B=1100, N=8, V=300, n_sets=2, iters=8, ctx0=40), 4)


def _graph_run(cfg, rounds, passes=2):
    """Rounds of smcsd_step recorded in HIP graphs (one graph per round, captured once with
    nothing executing) and replayed in order, against the same rounds called directly: every
    output bit-identical after every replay.  The replays are run `passes` times from the
    initial state, restored by eager copies between passes, so replays after the first one
    are checked too; the status word is cleared eagerly before each round on both sides."""
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    base = synth.zipf_base(cfg, "cuda") if cfg.target_kind == "zipf" else None
    sets = []
    for s in range(cfg.n_sets):
        t, d = synth.make_logit_set(cfg, s, "cuda", base)
        sets.append((t, d, synth.sample_draft_tokens(cfg, d, s)))
    kv = synth.initial_kv(cfg)
    lw0 = torch.randn(S, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
    A, G = _Copy(cfg, kv, lw0), _Copy(cfg, kv, lw0)
    L0 = int(kv["seq_len"])
    ident = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    for c in (A, G):
        sm.kv_reassign(ident, torch.zeros(B, dtype=torch.int32, device="cuda"), B, N, c.tables,
                       cfg.block_size, L0, K + 1, c.rc, c.fl, c.top, c.cow, c.ncow, c.st, c.ws_kv)
    torch.cuda.synchronize()
    state_names = ("lw", "tables", "rc", "fl", "top")
    init = {k: getattr(G, k).clone() for k in state_names}
    ws_kv0 = G.ws_kv.clone()

    def call(c, t):
        tgt, drf, x = sets[t % cfg.n_sets]
        sm.step(tgt, drf, x, B, N, K, V, cfg.temperature, cfg.alpha, sm.MODE_SMC, cfg.tau,
                cfg.rng_seed, t, c.lw, c.tok, c.anc, c.ess, c.res, c.tables, cfg.block_size,
                L0 + (t + 1) * (K + 1), K + 1, c.rc, c.fl, c.top, c.cow, c.ncow, c.st, c.ws_v,
                c.ws_kv, out_num_tokens=c.num, out_logp=c.logp, out_logq=c.logq, out_lse=c.lse)

    want = []
    for t in range(rounds):
        A.st.zero_()
        call(A, t)
        torch.cuda.synchronize()
        want.append(A.snapshot())
    graphs = []
    for t in range(rounds):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(G, t)
        graphs.append(g)
    torch.cuda.synchronize()
    for p in range(passes):
        for k in state_names:
            getattr(G, k).copy_(init[k])
        G.ws_kv.copy_(ws_kv0)
        for t in range(rounds):
            G.st.zero_()
            graphs[t].replay()
            torch.cuda.synchronize()
            bad = _same(want[t], G.snapshot())
            assert bad is None, (p, t, bad)
    assert any(w["res"].any() for w in want)


@pytest.mark.parametrize("name", ["c1_tiny", "c2_single_prompt", "c3_small"])
def test_step_graph_replays_equal_direct_calls(name):
    """The launch-bound shapes (C1, C2 at full size) and C3 at 4 prompts, replayed from HIP
    graphs: the form that removes the host's per-call cost."""
    if name == "c1_tiny":
        _graph_run(C.C1.scaled(name="g", iters=10), 8)
    elif name == "c2_single_prompt":
        _graph_run(C.C2.scaled(name="g", iters=10, n_sets=8), 8)
    else:
        _graph_run(C.C3.scaled(name="g", B=4, n_sets=2, iters=8), 6)


def test_rounds_on_two_streams_do_not_interfere():
    """The library keeps no state: two independent batches, each with its own workspaces
    and state, stepped on two streams at once (default priority) give the bits of the same
    rounds run one after the other on the default stream."""
    cfg = C.C3.scaled(name="s2", B=3, V=30011, n_sets=2, iters=8)
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    base = synth.zipf_base(cfg, "cuda")
    sets = []
    for s in range(cfg.n_sets):
        t, d = synth.make_logit_set(cfg, s, "cuda", base)
        sets.append((t, d, synth.sample_draft_tokens(cfg, d, s)))
    kv = synth.initial_kv(cfg)
    lw0 = torch.zeros(S, device="cuda")

    def fresh():
        c = _Copy(cfg, kv, lw0)
        ident = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
        sm.kv_reassign(ident, torch.zeros(B, dtype=torch.int32, device="cuda"), B, N, c.tables,
                       cfg.block_size, int(kv["seq_len"]), K + 1, c.rc, c.fl, c.top, c.cow, c.ncow,
                       c.st, c.ws_kv)
        return c

    def rounds(c, seed, stream=None):
        L = int(kv["seq_len"])
        for t in range(5):
            tgt, drf, x = sets[t % cfg.n_sets]
            L += K + 1
            sm.step(tgt, drf, x, B, N, K, V, cfg.temperature, cfg.alpha, sm.MODE_SMC, cfg.tau, seed, t,
                    c.lw, c.tok, c.anc, c.ess, c.res, c.tables, cfg.block_size, L, K + 1, c.rc, c.fl,
                    c.top, c.cow, c.ncow, c.st, c.ws_v, c.ws_kv, out_num_tokens=c.num,
                    out_logp=c.logp, out_lse=c.lse, stream=stream)

    ref = [fresh(), fresh()]
    torch.cuda.synchronize()
    rounds(ref[0], 11)
    rounds(ref[1], 12)
    torch.cuda.synchronize()
    par = [fresh(), fresh()]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for c, seed, st in zip(par, (11, 12), streams):
        with torch.cuda.stream(st):
            rounds(c, seed, stream=st)
    torch.cuda.synchronize()
    for a, b in zip(ref, par):
        bad = _same(a.snapshot(), b.snapshot())
        assert bad is None, bad
    assert _same(ref[0].snapshot(), ref[1].snapshot()) is not None   # the seeds differ
