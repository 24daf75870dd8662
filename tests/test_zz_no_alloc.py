"""smcsd_verify_static (the verify entry point that allocates nothing, for callers that
cannot allocate device memory) against smcsd_verify with a caller workspace: the same
kernels on the same inputs, so every output must be bit-identical.  Two calls in a row
share the library's scratch array, the second on a smaller batch and vocabulary; both SMC
modes, the SpS mode, bf16 and fp32; plus the host-side rejection of a call whose scratch
would exceed the array."""
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


def _inputs(cfg, s):
    base = synth.zipf_base(cfg, "cuda") if cfg.target_kind == "zipf" else None
    t, d = synth.make_logit_set(cfg, s, "cuda", base)
    return t, d, synth.sample_draft_tokens(cfg, d, s)


def _call(fn, cfg, t, d, x, mode, step, ws=None):
    B, N, K, V = cfg.B, cfg.N, cfg.K, cfg.V
    S = B * N if mode != sm.MODE_SPS else B
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = dict(tok=torch.full((S, K + 1), -7, **i32), num=torch.zeros(S, **i32),
               logp=torch.zeros((S, K + 1), **f32), logq=torch.zeros((S, K), **f32),
               lse=torch.zeros((S, 2 * K + 1), **f32), st=torch.zeros(1, **i32),
               lw=torch.linspace(-3.0, 1.0, S, **f32))
    kw = dict(log_weights=out["lw"] if mode != sm.MODE_SPS else None, out_num_tokens=out["num"],
              out_logp=out["logp"], out_logq=out["logq"], out_lse=out["lse"])
    if mode == sm.MODE_SPS:
        args = (t, d, x, B, 1, K, V, cfg.temperature, 1.0, mode, cfg.rng_seed, step, out["tok"],
                out["st"])
        kw["seq_step"] = N
    else:
        args = (t, d, x, B, N, K, V, cfg.temperature, cfg.alpha, mode, cfg.rng_seed, step,
                out["tok"], out["st"])
    if fn is sm.verify:
        fn(*args[:14], ws, **kw)
    else:
        fn(*args, **kw)
    return out


def _same(a, b):
    for k in a:
        assert torch.equal(a[k].view(torch.int32) if a[k].dtype == torch.float32 else a[k],
                           b[k].view(torch.int32) if b[k].dtype == torch.float32 else b[k]), k


@pytest.mark.parametrize("mode", [sm.MODE_SMC, sm.MODE_SMC_RACE, sm.MODE_SPS])
def test_static_matches_workspace_two_calls(mode):
    big = C.C3.scaled(name="c3_noalloc", B=4, n_sets=1)            # 64 sequences, V = 128256
    small = C.C2.scaled(name="c2_noalloc", B=2, V=20011, n_sets=1)  # 16 sequences, V = 20011
    if mode == sm.MODE_SPS:
        big = big.scaled(dtype="f32")
    for step, cfg in enumerate((big, small)):
        t, d, x = _inputs(cfg, step)
        op = sm.OP_VERIFY_SPS if mode == sm.MODE_SPS else sm.OP_VERIFY_SMC
        nseq = cfg.B if mode == sm.MODE_SPS else cfg.B * cfg.N
        assert sm.workspace_bytes(op, nseq, 1, cfg.K, cfg.V) <= sm.STATIC_SCRATCH_BYTES
        ws = sm.alloc_workspace(op, nseq, 1, cfg.K, cfg.V)
        ref = _call(sm.verify, cfg, t, d, x, mode, 11 + step, ws)
        got = _call(sm.verify_static, cfg, t, d, x, mode, 11 + step)
        torch.cuda.synchronize()
        _same(ref, got)
        assert int(got["st"].cpu()[0]) == 0
        assert (got["tok"][:, 0] >= 0).all()


def test_static_rejects_beyond_its_array():
    # 1024 sequences x 17 rows at V = 128256 need ~2.9 MB; 4096 sequences need more than 4 MiB
    K, V = 8, 128256
    assert sm.workspace_bytes(sm.OP_VERIFY_SMC, 64, 64, K, V) > sm.STATIC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    lw = torch.zeros(16, dtype=torch.float32, device="cuda")
    tok = torch.zeros(16, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = sm.load_library().smcsd_verify_static(
        t.data_ptr(), t.data_ptr(), sm.DTYPE_BF16, V, 1, x.data_ptr(), 64, 64, K, V, 1.0, 1.0,
        sm.MODE_SMC, 0, 0, None, None, lw.data_ptr(), tok.data_ptr(), None, None, None, None,
        st.data_ptr(), None)
    assert rc == -5
    assert "static array" in sm.status_string(-5)
