"""smcsd_kv_check, the debugging check of the block-table state, against the oracle's
definition of a consistent state (oracle.kv_check) on the same arrays: the states the
library's own rounds leave (all counts zero), one injected corruption at a time (each
kind of violation, with exact counts), pools beyond one workgroup's reach, and the
binding's debug mode (SMCSD_DEBUG_CHECK=1), which raises after a KV call that leaves an
inconsistent state."""
import math

import numpy as np
import pytest
import torch

import oracle
import smc_verification_resampling_amd as sm
from tests import gpu_harness as H
from workloads import configs as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _gpu_check(T, slots, rc, fl, top):
    """The library's counts and status bit for host arrays (copied to the device)."""
    dev = "cuda"
    P = rc.shape[0]
    viol = torch.full((sm.KV_CHECK_KINDS,), 77, dtype=torch.int32, device=dev)  # overwritten
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = sm.alloc_workspace(sm.OP_KV_CHECK, 0, 0, P=P)
    ws.fill_(0x5A)                                    # any contents
    sm.kv_check(torch.from_numpy(np.ascontiguousarray(T)).to(dev), slots,
                torch.from_numpy(rc).to(dev), torch.from_numpy(fl).to(dev),
                torch.tensor([top], dtype=torch.int32, device=dev), viol, st, ws)
    torch.cuda.synchronize()
    return viol.cpu().numpy().astype(np.int64), int(st.cpu()[0])


def _agree(T, slots, rc, fl, top):
    g, st = _gpu_check(T, slots, rc, fl, top)
    o = oracle.kv_check(T, slots, rc, fl, top)
    assert np.array_equal(g, o), (g, o)
    assert (st == sm.ST_KV_INCONSISTENT) == bool(o.any())
    return o


def _pipeline_state(cfg, rounds):
    p = H.Pipeline(cfg, check=False)
    for t in range(rounds):
        p.round(t)
    torch.cuda.synchronize()
    slots = math.ceil((p.L + cfg.K + 1) / cfg.block_size)
    return (p.tables.cpu().numpy(), slots, p.rc.cpu().numpy(), p.free_list.cpu().numpy(),
            int(p.free_top.cpu()[0]))


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_library_rounds_leave_a_consistent_state(name):
    cfg = C.downsized(C.C3 if name == "c3" else C.C5, B=2, V=20011, iters=8)
    T, slots, rc, fl, top = _pipeline_state(cfg, 6)
    assert _agree(T, slots, rc, fl, top).tolist() == [0] * 5


def test_each_injected_corruption_is_counted():
    cfg = C.downsized(C.C3, B=2, V=20011, iters=8)
    T, slots, rc, fl, top = _pipeline_state(cfg, 5)
    P = rc.shape[0]
    live = np.nonzero(rc)[0]
    shared = live[np.argmax(rc[live])]        # a prefix block, rc = N
    private = live[np.argmin(rc[live])]
    cases = []
    r = rc.copy(); r[shared] += 1; cases.append((T, r, fl, top))            # refcount off by one
    r = rc.copy(); r[private] = 0; cases.append((T, r, fl, top))            # and leaked
    t = T.copy(); t[3, 0] = P + 5; cases.append((t, rc, fl, top))           # id past the pool
    t = T.copy(); t[3, slots - 1] = -7; cases.append((t, rc, fl, top))      # a corrupt slot
    f = fl.copy(); f[top] = f[0]; cases.append((T, rc, f, top + 1))         # pushed twice
    f = fl.copy(); f[top] = private; cases.append((T, rc, f, top + 1))      # live block freed
    cases.append((T, rc, fl, top - 3))                                      # three blocks lost
    f = fl.copy(); f[1] = -1; cases.append((T, rc, f, top))                 # corrupt stack entry
    cases.append((T, rc, fl, P + 1))                                        # top past the pool
    cases.append((T, rc, fl, -2))                                           # negative top
    for i, (t, r, f, tp) in enumerate(cases):
        o = _agree(t, slots, r, f, tp)
        assert o.any(), i


def test_pools_beyond_one_launch_row():
    """A pool of 3M blocks and 70,000 sequences (several workgroups per item kind), with a
    few corruptions scattered over it."""
    rng = np.random.default_rng(5)
    S, M, slots, P = 70000, 40, 37, 3_000_000
    T = np.full((S, M), -1, np.int32)
    ids = rng.permutation(P)[: S * slots].astype(np.int32).reshape(S, slots)
    T[:, :slots] = ids
    rc = np.zeros(P, np.int32)
    rc[ids.ravel()] = 1
    free = np.setdiff1d(np.arange(P, dtype=np.int32), ids.ravel())[::-1].copy()
    fl = np.zeros(P, np.int32)
    fl[: free.size] = free
    top = free.size
    assert _agree(T, slots, rc, fl, top).tolist() == [0] * 5
    rc[ids[123, 4]] = 2
    rc[ids[69999, 36]] = 0
    fl[top - 10] = ids[5, 5]
    assert _agree(T, slots, rc, fl, top).tolist() == [2, 0, 0, 1, 2]


def test_debug_mode_raises_after_an_inconsistent_kv_call(monkeypatch):
    cfg = C.downsized(C.C3, B=2, V=20011, iters=8)
    p = H.Pipeline(cfg, check=False)
    for t in range(3):
        p.round(t)
    torch.cuda.synchronize()
    monkeypatch.setenv("SMCSD_DEBUG_CHECK", "1")
    B, N, K = cfg.B, cfg.N, cfg.K
    ident = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    none = torch.zeros(B, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = p.L + K + 1
    sm.kv_reassign(ident, none, B, N, p.tables, cfg.block_size, L, K + 1, p.rc, p.free_list,
                   p.free_top, p.cow, p.cow_count, st, p.ws_kv)            # consistent: no raise
    torch.cuda.synchronize()
    rcv = p.rc.cpu().numpy()
    b = int(np.nonzero(rcv)[0][0])
    p.rc[b] += 1                                                           # corrupt one count
    with pytest.raises(sm.SmcsdError, match="refcount"):
        sm.kv_reassign(ident, none, B, N, p.tables, cfg.block_size, L + K + 1, K + 1, p.rc,
                       p.free_list, p.free_top, p.cow, p.cow_count, st, p.ws_kv)
