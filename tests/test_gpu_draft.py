"""GPU parity of the draft-side sampler and of the verify that takes the draft's log q.

smcsd_draft_sample (one draft position per call) against the oracle's draft_sample, and
smcsd_verify with logq_in against the oracle's verify with logq_in, on seeded rows that
span several vocabulary chunks with a ragged tail and misaligned row starts.  Tokens
must match exactly except at draws whose oracle CDF margin is below 1e-6; log q within
1e-5 * max(1, |ref|); log-weights within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def _host(x):
    x = x.contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def _gpu_draft(rows, V, T, seed, step, pos, row_stride=None):
    n = rows.shape[0]
    tok, st = _i32(n), _i32(1)
    lq = torch.zeros(n, dtype=torch.float32, device="cuda")
    ws = sm.alloc_workspace(sm.OP_DRAFT, n, 1, 0, V)
    flat = rows.reshape(-1)
    sm.draft_sample(flat, n, V, T, seed, step, pos, tok, st, ws, out_logq=lq,
                    row_stride=row_stride)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lq.cpu().numpy(), int(st.cpu()[0])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,T,pos", [(40000, 0.8, 0), (40000, 1.3, 7), (8193, 1.0, 3), (5, 1.0, 0)])
def test_draft_sample_matches_oracle(dtype, V, T, pos):
    g = torch.Generator(device="cuda").manual_seed(V + pos)
    n, stride = 96, V + 3                    # odd stride: rows start misaligned
    buf = torch.randn((n, stride), generator=g, device="cuda") * 2.0
    buf[:, ::11] -= 6.0
    buf = buf.to(dtype)
    tok, lq, st = _gpu_draft(buf, V, T, 17, 1234, pos, row_stride=stride)
    assert st == 0
    rows = _host(buf)[:, :V]
    o = oracle.draft_sample(np.ascontiguousarray(rows), float(np.float32(T)), 17, 1234, pos)
    flagged = o["margin"] < MARGIN
    assert np.array_equal(tok[~flagged], o["tokens"][~flagged])
    same = tok == o["tokens"]
    assert np.all(np.abs(lq[same] - o["logq"][same]) <= 1e-5 * np.maximum(1.0, np.abs(o["logq"][same])))
    assert np.all((tok >= 0) & (tok < V))


def test_draft_sample_maximum_vocabulary():
    """V = 2^24 rows (1024 one-step tiles per row): tokens and log q against the oracle."""
    V, n = 1 << 24, 3
    g = torch.Generator(device="cuda").manual_seed(99)
    rows = (torch.randn((n, V), generator=g, device="cuda") * 1.5).to(torch.bfloat16)
    tok, lq, st = _gpu_draft(rows, V, 0.7, 5, 8, 2)
    assert st == 0
    o = oracle.draft_sample(_host(rows), float(np.float32(0.7)), 5, 8, 2)
    flagged = o["margin"] < MARGIN
    assert np.array_equal(tok[~flagged], o["tokens"][~flagged])
    same = tok == o["tokens"]
    assert np.all(np.abs(lq[same] - o["logq"][same]) <= 1e-5 * np.maximum(1.0, np.abs(o["logq"][same])))


def test_draft_sample_masked_one_hot_and_empty_rows():
    V = 20000
    rows = torch.full((4, V), float("-inf"), device="cuda")
    rows[0, 12345] = 0.0                     # one finite logit
    rows[1, 7] = 1.0
    rows[1, 19999] = 1.0                     # two equal logits at both ends
    rows[2] = torch.linspace(-3, 3, V, device="cuda")
    rows[2, ::2] = float("-inf")             # masked tokens are never drawn
    for t in range(5):
        tok, lq, st = _gpu_draft(rows[:3].contiguous(), V, 1.0, 3, t, 1)
        assert st == 0
        assert tok[0] == 12345 and lq[0] == 0.0
        assert tok[1] in (7, 19999) and abs(lq[1] + np.log(2.0)) < 1e-6
        assert tok[2] % 2 == 1
    tok, lq, st = _gpu_draft(rows[3:].contiguous(), V, 1.0, 3, 0, 0)
    assert tok[0] == -1 and st & sm.ST_EMPTY_ROW


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_with_draft_logq_matches_oracle(dtype):
    g = torch.Generator(device="cuda").manual_seed(11)
    B, N, K, V, T = 2, 8, 4, 30011, 0.8
    S = B * N
    tgt = (torch.randn((S, K + 1, V), generator=g, device="cuda") * 2.0).to(dtype)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    logq = -torch.rand((S, K), generator=g, device="cuda") * 9.0
    lw = torch.randn(S, generator=g, device="cuda")
    lw0 = lw.cpu().numpy().copy()
    out, num, st = _i32(S, K + 1), _i32(S), _i32(1)
    lp = torch.zeros((S, K + 1), device="cuda")
    lse = torch.zeros((S, 2 * K + 1), device="cuda")
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    sm.verify(tgt, None, toks, B, N, K, V, T, 1.0, sm.MODE_SMC, 5, 9, out, st, ws, log_weights=lw,
              out_num_tokens=num, out_logp=lp, out_lse=lse, logq_in=logq)
    torch.cuda.synchronize()
    assert int(st.cpu()[0]) == 0
    o = oracle.verify_smc(_host(tgt), None, toks.cpu().numpy(), float(np.float32(T)), 1.0, 5, 9,
                          lw0, logq_in=logq.cpu().numpy().astype(np.float64))
    got = out.cpu().numpy()
    flagged = o["margin"] < MARGIN
    assert np.array_equal(got[~flagged], o["tokens"][~flagged])
    assert np.max(np.abs(lw.cpu().numpy() - o["lw"])) < 1e-4
    assert np.all(num.cpu().numpy() == K + 1)
    l = lse.cpu().numpy()
    assert np.all(np.isnan(l[:, K + 1:]))
    assert np.allclose(l[:, :K + 1], o["lse"][:, :K + 1], rtol=1e-5, atol=0)


def test_draft_logq_path_equals_reading_the_draft_rows():
    """Draft tokens and log q from smcsd_draft_sample, one position at a time, then the
    verify with logq_in against the verify that reads the draft rows: same tokens, same
    log-weights within rounding."""
    g = torch.Generator(device="cuda").manual_seed(23)
    B, N, K, V, T = 4, 16, 4, 128256, 0.8
    S = B * N
    tgt = (torch.randn((S, K + 1, V), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    drf = (tgt[:, :K].float() + torch.randn((S, K, V), generator=g, device="cuda")).to(torch.bfloat16)
    toks = _i32(S, K)
    logq = torch.zeros((S, K), device="cuda")
    flat = drf.reshape(-1)
    ws_d = sm.alloc_workspace(sm.OP_DRAFT, S, 1, 0, V)
    st = _i32(1)
    for k in range(K):
        tk, lk = _i32(S), torch.zeros(S, device="cuda")
        sm.draft_sample(flat[k * V:], S, V, T, 77, 3, k, tk, st, ws_d, out_logq=lk, row_stride=K * V)
        toks[:, k] = tk
        logq[:, k] = lk
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    outs = []
    for use_logq in (False, True):
        lw = torch.zeros(S, device="cuda")
        out = _i32(S, K + 1)
        lq = torch.zeros((S, K), device="cuda")
        sm.verify(tgt, None if use_logq else drf, toks, B, N, K, V, T, 1.0, sm.MODE_SMC, 77, 4, out,
                  st, ws, log_weights=lw, out_logq=lq, logq_in=logq if use_logq else None)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lw.cpu().numpy(), lq.cpu().numpy()))
    assert int(st.cpu()[0]) == 0
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.max(np.abs(outs[0][1] - outs[1][1])) < 1e-4
    assert np.max(np.abs(outs[0][2] - outs[1][2])) < 1e-4


def test_draft_side_round_at_the_benchmark_shape():
    """The --draft-logq flow of bench.py at the C3 shape (32 prompts x 16 particles, K = 4,
    V = 128256, bf16 Zipf logits), every sequence against the oracle: the K draft positions
    from smcsd_draft_sample (strided rows of the draft tensor, as the benchmark passes them)
    against oracle.draft_sample, then smcsd_verify with those log q against the oracle's
    verify with logq_in."""
    from workloads import configs as C
    from workloads import synth

    cfg = C.C3
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    tgt, drf = synth.make_logit_set(cfg, 0, "cuda", synth.zipf_base(cfg, "cuda"))
    T32 = float(np.float32(cfg.temperature))
    dh = _host(drf)
    toks, lq = _i32(S, K), torch.zeros((S, K), device="cuda")
    flat = drf.reshape(-1)
    ws_d = sm.alloc_workspace(sm.OP_DRAFT, S, 1, 0, V)
    st = _i32(1)
    for k in range(K):
        tk, lk = _i32(S), torch.zeros(S, device="cuda")
        sm.draft_sample(flat[k * V:], S, V, cfg.temperature, cfg.rng_seed, 0, k, tk, st, ws_d,
                        out_logq=lk, row_stride=K * V)
        torch.cuda.synchronize()
        o = oracle.draft_sample(np.ascontiguousarray(dh[:, k]), T32, cfg.rng_seed, 0, k)
        ok = o["margin"] >= MARGIN
        assert ok.mean() > 0.9        # ~3 % of Zipf draws land within 1e-6 of a CDF step
        assert np.array_equal(tk.cpu().numpy()[ok], o["tokens"][ok]), k
        d = np.abs(lk.cpu().numpy().astype(np.float64) - o["logq"])
        assert np.all(d[ok] <= 1e-5 * np.maximum(1.0, np.abs(o["logq"][ok]))), k
        toks[:, k] = torch.from_numpy(o["tokens"]).cuda()     # the oracle's draws feed both sides
        lq[:, k] = lk
    assert int(st.cpu()[0]) == 0
    lw = torch.zeros(S, device="cuda")
    out, num = _i32(S, K + 1), _i32(S)
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    sm.verify(tgt, None, toks, B, N, K, V, cfg.temperature, cfg.alpha, sm.MODE_SMC, cfg.rng_seed, 1,
              out, st, ws, log_weights=lw, out_num_tokens=num, logq_in=lq)
    torch.cuda.synchronize()
    o = oracle.verify_smc(_host(tgt), None, toks.cpu().numpy(), T32, float(np.float32(cfg.alpha)),
                          cfg.rng_seed, 1, np.zeros(S, np.float32),
                          logq_in=lq.cpu().numpy().astype(np.float64))
    ok = o["margin"] >= MARGIN
    assert int(st.cpu()[0]) == o["status"] == 0
    assert np.array_equal(out.cpu().numpy()[ok], o["tokens"][ok])
    assert np.max(np.abs(lw.cpu().numpy() - o["lw"])) <= 1e-4
    assert np.all(num.cpu().numpy() == K + 1)
