"""GPU parity of the SMC verify with the exponential-race bonus (SMCSD_MODE_SMC_RACE).

The bonus token is argmax_v (z_v - ln E_v) with Philox clocks (the exponential-races
summary page, key design); the GPU evaluates the keys in fp32 inside the LSE pass, the
oracle in fp64.  Bar: bonus tokens equal except where the oracle's gap between the two
largest keys is below 2e-5 nats.  Bound on an fp32 key's error (keys of magnitude <= ~30 in
log2 units): the fp32 rounding of c = log2(e)/T times |x c| (<= 1.8e-6), one ulp of each
of the two hardware logarithms at that magnitude (<= 1.9e-6 each) and of the final
multiply-add (<= 1.9e-6): ~5.5e-6 log2 units = 3.8e-6 nats per key, 7.6e-6 on a gap of two;
2e-5 is 2.6 times that.  Measured (test_race_key_error_is_far_below_the_flag_threshold):
at most 1.4e-6 nats over the winners of 64 sequences of the C3 vocabulary.
draft tokens echoed exactly; log-weights within 1e-4; log p of the bonus within
1e-5 * max(1, |ref|) where the tokens agree.  Covers several chunks with a ragged tail,
row starts that are not 16-byte aligned (the one-at-a-time path), bf16 and fp32, the
full C3 shape on sampled sequences, masked / one-hot / empty / NaN rows, and the equality
of every non-bonus output with SMC mode.
"""
import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm
from workloads import configs, synth

pytestmark = pytest.mark.gpu

MARGIN = 2e-5


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


def _run(tgt, drf, toks, B, N, K, V, T, alpha, seed, step, lw0, mode, row_stride=None):
    S = B * N
    lw = lw0.clone()
    out, num, st = _i32(S, K + 1), _i32(S), _i32(1)
    lp = torch.zeros((S, K + 1), device="cuda")
    lse = torch.zeros((S, 2 * K + 1), device="cuda")
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    sm.verify(tgt, drf, toks, B, N, K, V, T, alpha, mode, seed, step, out, st, ws, log_weights=lw,
              out_num_tokens=num, out_logp=lp, out_lse=lse, row_stride=row_stride)
    torch.cuda.synchronize()
    return dict(tokens=out.cpu().numpy(), num=num.cpu().numpy(), lw=lw.cpu().numpy(),
                logp=lp.cpu().numpy(), lse=lse.cpu().numpy(), status=int(st.cpu()[0]))


def _check(got, o, K):
    flagged = o["margin"] < MARGIN
    assert np.array_equal(got["tokens"][:, :K], o["tokens"][:, :K])
    bad = (got["tokens"][:, K] != o["tokens"][:, K]) & ~flagged
    assert not bad.any(), (np.nonzero(bad)[0][:8], o["margin"][bad][:8])
    same = got["tokens"][:, K] == o["tokens"][:, K]
    assert np.max(np.abs(got["lw"][same] - o["lw"][same])) < 1e-4
    ref = o["logp"][same, K]
    assert np.all(np.abs(got["logp"][same, K] - ref) <= 1e-5 * np.maximum(1.0, np.abs(ref)))
    return int(flagged.sum())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,pad,T,alpha", [(40000, 0, 0.8, 1.0), (40000, 3, 1.3, 4.0),
                                           (8193, 1, 1.0, 1.0), (5, 0, 1.0, 2.0),
                                           (65537, 0, 1.0, 1.0), (32769, 2, 0.9, 1.0)])
def test_race_verify_matches_oracle(dtype, V, pad, T, alpha):
    g = torch.Generator(device="cuda").manual_seed(V + pad)
    B, N, K = 4, 12, 2
    S, stride = B * N, V + pad            # pad > 0: row starts not 16-byte aligned
    buf = torch.randn((S, K + 1, stride), generator=g, device="cuda") * 2.0
    buf[..., ::7] -= 5.0
    dbuf = buf[:, :K] + torch.randn((S, K, stride), generator=g, device="cuda")
    buf, dbuf = buf.to(dtype), dbuf.to(dtype)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    lw0 = torch.randn(S, generator=g, device="cuda")
    got = _run(buf.reshape(-1), dbuf.reshape(-1), toks, B, N, K, V, T, alpha, 19, 77, lw0,
               sm.MODE_SMC_RACE, row_stride=stride)
    assert got["status"] == 0
    assert np.all(got["num"] == K + 1)
    o = oracle.verify_smc(np.ascontiguousarray(_host(buf)[..., :V]),
                          np.ascontiguousarray(_host(dbuf)[..., :V]), toks.cpu().numpy(),
                          float(np.float32(T)), alpha, 19, 77, lw0.cpu().numpy(), bonus="race")
    assert _check(got, o, K) <= 2


def test_race_verify_full_c3_shape_sampled():
    """C3 (B=32, N=16, K=4, V=128256, bf16 Zipf logits) in race mode; 64 sampled sequences
    against the oracle, and every bonus token a finite-logit id."""
    cfg = configs.C3
    B, N, K, V, S = cfg.B, cfg.N, cfg.K, cfg.V, cfg.S
    base = synth.zipf_base(cfg, "cuda")
    tgt, drf = synth.make_logit_set(cfg, 1, "cuda", base)
    toks = synth.sample_draft_tokens(cfg, drf, 1)
    lw0 = torch.zeros(S, device="cuda")
    got = _run(tgt, drf, toks, B, N, K, V, cfg.temperature, cfg.alpha, cfg.rng_seed, 5, lw0,
               sm.MODE_SMC_RACE)
    assert got["status"] == 0
    bon = got["tokens"][:, K]
    assert np.all((bon >= 0) & (bon < V))
    pick = np.random.default_rng(0).choice(S, 64, replace=False)
    pt = torch.from_numpy(pick).cuda()
    o = oracle.verify_smc(_host(tgt.view(S, K + 1, V)[pt]), _host(drf.view(S, K, V)[pt]),
                          toks.view(S, K)[pt].cpu().numpy(), float(np.float32(cfg.temperature)),
                          cfg.alpha, cfg.rng_seed, 5, np.zeros(64), rng_index=pick.astype(np.int64),
                          bonus="race")
    sub = {k: got[k][pick] for k in ("tokens", "lw", "logp")}
    assert _check(sub, o, K) <= 2


def test_race_mode_matches_smc_mode_apart_from_the_bonus():
    """Race and inverse-CDF modes on the same inputs: the bonus row is cut into the same
    tiles in both but reduced in a different order (the inverse-CDF tiles carry their slab
    sums through a two-phase reduction, the race tiles their race winners through a
    butterfly), and the other rows into larger big tiles in race mode, so the normalisers,
    the gathered log-probabilities and the log-weights agree to rounding (checked ten times
    tighter than the oracle bar)."""
    g = torch.Generator(device="cuda").manual_seed(4)
    B, N, K, V = 2, 16, 4, 50000
    S = B * N
    tgt = (torch.randn((S, K + 1, V), generator=g, device="cuda") * 2).to(torch.bfloat16)
    drf = (tgt[:, :K].float() + torch.randn((S, K, V), generator=g, device="cuda")).to(torch.bfloat16)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    lw0 = torch.randn(S, generator=g, device="cuda")
    a = _run(tgt, drf, toks, B, N, K, V, 0.9, 1.0, 3, 8, lw0, sm.MODE_SMC)
    b = _run(tgt, drf, toks, B, N, K, V, 0.9, 1.0, 3, 8, lw0, sm.MODE_SMC_RACE)
    assert a["status"] == 0 and b["status"] == 0
    assert np.array_equal(a["tokens"][:, :K], b["tokens"][:, :K])
    lse_a, lse_b = a["lse"].reshape(S, 2 * K + 1), b["lse"].reshape(S, 2 * K + 1)
    assert np.all(np.abs(lse_a[:, K] - lse_b[:, K]) <= 1e-6 * np.abs(lse_a[:, K]))
    assert np.all(np.abs(lse_a - lse_b) <= 1e-6 * np.abs(lse_a))
    assert np.max(np.abs(a["logp"][:, :K] - b["logp"][:, :K])) <= 1e-6 * max(1.0, np.max(np.abs(a["logp"][:, :K])))
    assert np.max(np.abs(a["lw"] - b["lw"])) <= 1e-5  # alpha = 1: the bonus adds nothing
    assert (a["tokens"][:, K] != b["tokens"][:, K]).any()


def test_race_masked_one_hot_empty_and_nan_rows():
    B, N, K, V = 1, 5, 1, 20000
    S = B * N
    tgt = torch.randn((S, K + 1, V), device="cuda")
    drf = torch.randn((S, K, V), device="cuda")
    tgt[0, K] = float("-inf")
    tgt[0, K, 12345] = 0.0                 # one finite logit
    tgt[1, K, ::2] = float("-inf")         # masked tokens never win
    tgt[2, K] = float("-inf")              # empty row: no bonus, EMPTY_ROW
    toks = torch.zeros((S, K), dtype=torch.int32, device="cuda")
    for step in range(4):
        got = _run(tgt, drf, toks, B, N, K, V, 1.0, 1.0, 9, step, torch.zeros(S, device="cuda"),
                   sm.MODE_SMC_RACE)
        assert got["tokens"][0, K] == 12345 and got["logp"][0, K] == 0.0
        assert got["tokens"][1, K] % 2 == 1
        assert got["tokens"][2, K] == -1 and got["status"] & sm.ST_EMPTY_ROW
        assert 0 <= got["tokens"][3, K] < V
    tgt[4, K, 777] = float("nan")
    got = _run(tgt, drf, toks, B, N, K, V, 1.0, 1.0, 9, 0, torch.zeros(S, device="cuda"),
               sm.MODE_SMC_RACE)
    assert got["status"] & sm.ST_NAN_INPUT
    assert got["tokens"][4, K] == -1


def test_race_mode_with_the_drafts_log_q():
    """Race mode with logq_in (the draft rows not read) against race mode reading them:
    same tokens, log-weights within rounding (the tile order differs between the two)."""
    g = torch.Generator(device="cuda").manual_seed(31)
    B, N, K, V, T = 2, 16, 4, 70001, 0.8
    S = B * N
    tgt = (torch.randn((S, K + 1, V), generator=g, device="cuda") * 2).to(torch.bfloat16)
    drf = (tgt[:, :K].float() + torch.randn((S, K, V), generator=g, device="cuda")).to(torch.bfloat16)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    ref = oracle.verify_smc(_host(tgt), _host(drf), toks.cpu().numpy(), float(np.float32(T)), 1.0,
                            6, 2, np.zeros(S), bonus="race")
    lq = torch.from_numpy(ref["logq"].astype(np.float32)).cuda()
    outs = []
    for use in (False, True):
        lw = torch.zeros(S, device="cuda")
        out, st = _i32(S, K + 1), _i32(1)
        ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
        sm.verify(tgt, None if use else drf, toks, B, N, K, V, T, 1.0, sm.MODE_SMC_RACE, 6, 2, out,
                  st, ws, log_weights=lw, logq_in=lq if use else None)
        torch.cuda.synchronize()
        assert int(st.cpu()[0]) == 0
        outs.append((out.cpu().numpy(), lw.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.max(np.abs(outs[0][1] - outs[1][1])) < 1e-4
    flagged = ref["margin"] < MARGIN
    assert np.array_equal(outs[1][0][~flagged], ref["tokens"][~flagged])


def _race_winner_keys(ws, S, K, V, dtype):
    """The race winners (key, id) the LSE pass left in the verify workspace, best per
    sequence.  Layout of the workspace (256-byte aligned regions): the row partials (float2
    per sequence, row and 8192-element chunk), the bonus slab sums (8 floats per sequence and
    chunk), then one (key bits, id) pair per sequence and bonus tile."""
    cmin = -(-V // 8192)
    a256 = lambda x: (x + 255) & ~255  # noqa: E731
    off = a256(8 * S * (2 * K + 1) * cmin) + a256(4 * S * cmin * 8)
    ce = 16384 if dtype == torch.bfloat16 else 8192
    chunks = -(-V // ce)
    raw = ws[off:off + 8 * S * chunks].view(torch.int32).view(S, chunks, 2).cpu().numpy()
    keys = raw[:, :, 0].copy().view(np.float32).astype(np.float64)
    ids = raw[:, :, 1]
    best = np.lexsort((ids, -keys), axis=1)[:, 0]
    r = np.arange(S)
    return keys[r, best], ids[r, best]


@pytest.mark.parametrize("dtype,T", [(torch.bfloat16, 0.8), (torch.float32, 1.0)])
def test_race_key_error_is_far_below_the_flag_threshold(dtype, T):
    """The fp32 keys the GPU races with, against the oracle's fp64 key of the same token:
    the largest difference over 64 sequences of the C3 vocabulary (printed) must sit well
    inside the 2e-5 flag threshold, as the rounding bound in the module docstring says."""
    cfg = configs.C3.scaled(name="race_keys", B=4, dtype="bf16" if dtype == torch.bfloat16 else "f32",
                            temperature=T, n_sets=1)
    B, N, K, V = cfg.B, cfg.N, cfg.K, cfg.V
    S = B * N
    base = synth.zipf_base(cfg, "cuda")
    tgt, drf = synth.make_logit_set(cfg, 0, "cuda", base)
    toks = synth.sample_draft_tokens(cfg, drf, 0)
    out, st = _i32(S, K + 1), _i32(1)
    ws = sm.alloc_workspace(sm.OP_VERIFY_SMC, B, N, K, V)
    seed, step = 31, 9
    sm.verify(tgt, drf, toks, B, N, K, V, T, 1.0, sm.MODE_SMC_RACE, seed, step, out, st, ws,
              log_weights=torch.zeros(S, device="cuda"))
    torch.cuda.synchronize()
    key2, ids = _race_winner_keys(ws, S, K, V, dtype)
    tok = out.cpu().numpy()[:, K]
    assert np.array_equal(ids, tok)
    rows = _host(tgt)[:, K]
    z = (rows.astype(np.uint32) << 16).view(np.float32) if dtype == torch.bfloat16 else rows
    T32 = float(np.float32(T))
    key_o = np.array([float(z[g, tok[g]]) / T32 - np.log(oracle.race_clock(seed, g, step, int(tok[g])))
                      for g in range(S)])
    # the GPU key is log2(e) (z - ln E) + log2(ln 2) in log2 units
    key_g = (key2 - np.log2(np.log(2.0))) * np.log(2.0)
    err = np.abs(key_g - key_o)
    print("\n[race keys] %s T=%g: max |key_gpu - key_oracle| = %.3g nats over %d sequences "
          "(keys up to %.1f)" % (cfg.dtype, T, err.max(), S, np.abs(key_o).max()), flush=True)
    assert err.max() < MARGIN / 5
