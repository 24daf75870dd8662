"""SpS verify edge cases against the oracle, through the C ABI: ragged and misaligned rows
(the residual pass's element loads), rows that end inside a slab or a chunk, rows of more
chunk pairs than the per-workgroup decision takes (then a separate decide kernel runs
first), K at 0 and 32, a draft equal to the target and a forced rejection, masked rows,
given row log-normalisers (lse_in: no LSE pass) and the static-scratch entry point."""
import math

import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm
from tests import gpu_harness as H

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


def _sps_case(tgt, drf, toks, K, V, T, seed, step, row_stride=None, lse_in=None, static=False):
    S = toks.shape[0]
    out = dict(tokens=_i32(S, K + 1), num=_i32(S), logp=_f32(S, K + 1), logq=_f32(S, max(K, 1)),
               lse=_f32(S, 2 * K + 1), status=_i32(1))
    kw = dict(out_num_tokens=out["num"], out_logp=out["logp"], out_logq=out["logq"],
              out_lse=out["lse"], lse_in=lse_in, row_stride=row_stride)
    if static:
        sm.verify_static(tgt, drf, toks, S, 1, K, V, T, 1.0, sm.MODE_SPS, seed, step, out["tokens"],
                         out["status"], **kw)
    else:
        ws = sm.alloc_workspace(sm.OP_VERIFY_SPS, S, 1, K, V)
        sm.verify(tgt, drf, toks, S, 1, K, V, T, 1.0, sm.MODE_SPS, seed, step, out["tokens"],
                  out["status"], ws, **kw)
    torch.cuda.synchronize()
    rs = V if row_stride is None else row_stride
    th = H.host_logits(tgt).reshape(S, K + 1, rs)[:, :, :V]
    dh = H.host_logits(drf).reshape(S, K, rs)[:, :, :V] if K else np.zeros((S, 0, V), th.dtype)
    o = oracle.verify_sps(np.ascontiguousarray(th), np.ascontiguousarray(dh), toks.cpu().numpy(),
                          float(np.float32(T)), seed, step)
    return {k: v.cpu().numpy() for k, v in out.items()}, o


def _assert_sps(g, o, K, lse=True, min_ok=0.5):
    assert int(g["status"][0]) == o["status"]
    ok = np.minimum(o["margin_accept"], o["margin_final"]) >= H.MARGIN
    assert ok.mean() >= min_ok
    assert np.array_equal(g["num"][ok], o["num_tokens"][ok])
    assert np.array_equal(g["tokens"][ok], o["tokens"][ok])
    acc = o["margin_accept"] >= H.MARGIN
    for name in ("logp", "logq"):
        gv, ov = g[name][acc, :K].astype(np.float64), o[name][acc, :K]
        fin = np.isfinite(ov)
        assert np.all(np.abs(gv[fin] - ov[fin]) <= H.TOL_LOGP * np.maximum(1.0, np.abs(ov[fin])))
    # log p of the drawn token, where it is the oracle's
    lpK = g["logp"][ok, K].astype(np.float64)
    olpK = o["logp"][ok, K]
    fin = np.isfinite(olpK)
    assert np.all(np.abs(lpK[fin] - olpK[fin]) <= H.TOL_LOGP * np.maximum(1.0, np.abs(olpK[fin])))
    if lse:
        fin = np.isfinite(o["lse"])
        assert np.all(np.abs(g["lse"][fin] - o["lse"][fin]) <= H.TOL_LSE_REL * np.abs(o["lse"][fin]))


def _rows(S, K, rs, dtype, seed, close=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tgt = (2 * torch.randn((S, K + 1, rs), generator=g, device="cuda")).to(dt)
    drf = (tgt[:, :K].float() + close * torch.randn((S, K, rs), generator=g, device="cuda")).to(dt)
    return tgt, drf.contiguous(), g


@pytest.mark.parametrize("dtype,V,pad", [
    ("f32", 37, 2), ("bf16", 1001, 3), ("f32", 2047, 0), ("f32", 2049, 1), ("bf16", 4097, 0),
    ("f32", 8193, 0), ("bf16", 16385, 1), ("f32", 20011, 0), ("bf16", 40000, 0),
    ("f32", 262144, 0), ("f32", 262145, 0), ("bf16", 524289, 2)])
def test_sps_rows(dtype, V, pad):
    """Rows ending one element short of or past a slab (2048 fp32 / 4096 bf16 elements) and
    a chunk, misaligned rows (the element-load path), rows of exactly 32 chunks (the last
    shape whose decision runs in every residual workgroup) and of 33 or more."""
    S, K = 6, 4
    rs = V + pad
    tgt, drf, g = _rows(S, K, rs, dtype, V * 3 + pad, close=0.5)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _sps_case(tgt, drf, toks, K, V, 0.9, 11, 3, row_stride=rs)
    _assert_sps(gg, o, K)


@pytest.mark.parametrize("K", [0, 1, 32])
def test_sps_k_extremes(K):
    S, V = 5, 3001
    tgt, drf, g = _rows(S, K, V, "bf16", K + 5, close=0.3)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _sps_case(tgt, drf, toks, K, V, 1.0, 4, 9)
    _assert_sps(gg, o, K)


def test_sps_accept_all_and_forced_reject():
    """Draft rows equal to the target rows: p = q, every test passes (r < 1) and the draw is
    the bonus token from p_K.  Then the first draft token made far likelier under q than
    under p: the first test fails and the token comes from the residual of that row pair."""
    S, K, V = 8, 3, 5000
    g = torch.Generator(device="cuda").manual_seed(17)
    tgt = torch.randn((S, K + 1, V), generator=g, device="cuda")
    drf = tgt[:, :K].clone().contiguous()
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    gg, o = _sps_case(tgt, drf, toks, K, V, 1.0, 2, 2)
    _assert_sps(gg, o, K, min_ok=0.9)
    assert (o["num_tokens"] == K + 1).all()
    toks[:, 0] = 5
    drf[:, 0, 5] = tgt[:, 0, 5] + 30.0
    gg, o = _sps_case(tgt, drf, toks, K, V, 1.0, 2, 3)
    _assert_sps(gg, o, K, min_ok=0.9)
    assert (o["num_tokens"] == 1).all()


def test_sps_masked_rows_and_flags():
    S, K, V = 4, 2, 700
    tgt = torch.zeros((S, K + 1, V), dtype=torch.float32, device="cuda")
    drf = torch.zeros((S, K, V), dtype=torch.float32, device="cuda")
    tgt[0, K, :] = -math.inf
    tgt[0, K, 123] = 2.0                    # one-hot bonus row
    tgt[1, 0, :] = -math.inf                # target row 0 masked but its draft token
    tgt[1, 0, 9] = 0.0
    toks = torch.zeros((S, K), dtype=torch.int32, device="cuda")
    toks[1, 0] = 9
    gg, o = _sps_case(tgt, drf, toks, K, V, 1.0, 1, 2)
    _assert_sps(gg, o, K)
    drf[2, 1, :] = -math.inf
    tgt[3, 0, 17] = math.nan
    gg, o = _sps_case(tgt, drf, toks, K, V, 1.0, 1, 2)
    assert int(gg["status"][0]) == o["status"] == sm.ST_EMPTY_ROW | sm.ST_NAN_INPUT


@pytest.mark.parametrize("V", [3001, 300001])
def test_sps_given_row_normalisers(V):
    """lse_in: the row log-normalisers are given (here the oracle's, rounded to fp32) and
    the LSE pass does not run; the per-workgroup decision and the separate decide kernel
    (V = 300001 fp32: 37 chunks) both take them."""
    S, K = 5, 3
    tgt, drf, g = _rows(S, K, V, "f32", V, close=0.5)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    th, dh = H.host_logits(tgt), H.host_logits(drf)
    o0 = oracle.verify_sps(th, dh, toks.cpu().numpy(), float(np.float32(0.8)), 6, 1)
    lse = torch.from_numpy(o0["lse"].astype(np.float32)).cuda()
    gg, o = _sps_case(tgt, drf, toks, K, V, 0.8, 6, 1, lse_in=lse)
    _assert_sps(gg, o, K, lse=False)
    assert np.all(np.abs(gg["lse"] - o["lse"]) <= H.TOL_LSE_REL * np.abs(o["lse"]))


def test_sps_static_entry_point():
    S, K, V = 3, 4, 20011
    tgt, drf, g = _rows(S, K, V, "bf16", 5, close=0.5)
    toks = torch.randint(0, V, (S, K), generator=g, device="cuda", dtype=torch.int32)
    for step in (1, 2):
        gg, o = _sps_case(tgt, drf, toks, K, V, 0.7, 8, step, static=True)
        _assert_sps(gg, o, K)
