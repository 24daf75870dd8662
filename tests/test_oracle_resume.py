"""Checkpoint / resume on the oracle (CPU).

A round's state is small: the particles' log-weights, the block tables, refcounts, free
stack and its top, the sequence length and the round counter (with the seed).  Every
random draw depends only on (seed, round, index, tag) - the counter-based generator - so
ten rounds, a dump of that state to disk and a reload into fresh arrays, then ten more
rounds, must give the same bits as twenty rounds straight: tokens, log-weights, ESS,
ancestors, decisions, tables, refcounts, free stack and copy-on-write lists.  The GPU
form of the same property is in test_gpu_edges.py (determinism and resume).
"""
import math

import numpy as np
import pytest

import oracle
from workloads import configs as C
from workloads import synth


def _host(x):
    import torch

    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def _round(cfg, st, t, sets):
    """One oracle round on `st` (modified in place); returns this round's outputs."""
    B, N, K = cfg.B, cfg.N, cfg.K
    tgt, drf, x = sets[t % len(sets)]
    v = oracle.verify_smc(tgt, drf, x, float(np.float32(cfg.temperature)),
                          float(np.float32(cfg.alpha)), cfg.rng_seed, t, st["lw"])
    lw = v["lw"].astype(np.float32)                      # the library keeps fp32 weights
    r = oracle.resample(lw.reshape(B, N), float(np.float32(cfg.tau)), cfg.rng_seed, t)
    st["L"] += K + 1
    kv = oracle.kv_reassign(r["ancestors"], r["resampled"], st["tables"], cfg.block_size,
                            st["L"], K + 1, st["refcounts"], st["free_list"], st["free_top"])
    st["lw"] = r["lw"].astype(np.float32).reshape(-1)
    st["tables"], st["refcounts"] = kv["tables"], kv["refcounts"]
    st["free_list"], st["free_top"] = kv["free_list"], kv["free_top"]
    return {"tokens": v["tokens"], "lw_post": lw, "ess": r["ess"], "ancestors": r["ancestors"],
            "resampled": r["resampled"], "cow": kv["cow"], "status": v["status"] | r["status"] |
            kv["status"]}


def _start(cfg):
    kv = synth.initial_kv(cfg)
    st = {"lw": synth.initial_log_weights(cfg), "tables": kv["tables"],
          "refcounts": kv["refcounts"], "free_list": kv["free_list"],
          "free_top": int(kv["free_top"][0]), "L": int(kv["seq_len"])}
    B, N, K = cfg.B, cfg.N, cfg.K
    first = oracle.kv_reassign(np.tile(np.arange(N, dtype=np.int32), (B, 1)),
                               np.zeros(B, np.int32), st["tables"], cfg.block_size, st["L"],
                               K + 1, st["refcounts"], st["free_list"], st["free_top"])
    st["tables"], st["refcounts"] = first["tables"], first["refcounts"]
    st["free_list"], st["free_top"] = first["free_list"], first["free_top"]
    return st


def _same(a, b):
    for k in a:
        x, y = np.asarray(a[k]), np.asarray(b[k])
        if x.dtype.kind == "f":
            assert np.array_equal(x.view(np.int64 if x.itemsize == 8 else np.int32),
                                  y.view(np.int64 if y.itemsize == 8 else np.int32)), k
        else:
            assert np.array_equal(x, y), k


@pytest.mark.parametrize("name", ["c3_small", "c5_small"])
def test_resume_from_a_dump_equals_straight_rounds(name, tmp_path):
    base = C.C3 if name == "c3_small" else C.C5
    cfg = C.downsized(base, B=2, V=3001, iters=20).scaled(N=min(base.N, 12), n_sets=3)
    raw = []
    bs = synth.zipf_base(cfg, "cpu") if cfg.target_kind == "zipf" else None
    for s in range(cfg.n_sets):
        t, d = synth.make_logit_set(cfg, s, "cpu", bs)
        raw.append((_host(t), _host(d), synth.sample_draft_tokens(cfg, d, s).numpy()))

    straight = _start(cfg)
    outs_a = [_round(cfg, straight, t, raw) for t in range(20)]

    first = _start(cfg)
    outs_b = [_round(cfg, first, t, raw) for t in range(10)]
    path = tmp_path / "state.npz"
    np.savez(path, lw=first["lw"], tables=first["tables"], refcounts=first["refcounts"],
             free_list=first["free_list"], free_top=np.int64(first["free_top"]),
             L=np.int64(first["L"]), t=np.int64(10), seed=np.uint64(cfg.rng_seed))
    del first
    z = np.load(path)                                    # no pickle
    resumed = {"lw": z["lw"].copy(), "tables": z["tables"].copy(),
               "refcounts": z["refcounts"].copy(), "free_list": z["free_list"].copy(),
               "free_top": int(z["free_top"]), "L": int(z["L"])}
    assert int(z["t"]) == 10 and int(z["seed"]) == cfg.rng_seed
    outs_b += [_round(cfg, resumed, t, raw) for t in range(10, 20)]

    assert any(o["resampled"].any() for o in outs_a)
    for t, (a, b) in enumerate(zip(outs_a, outs_b)):
        _same(a, b)
    _same({k: straight[k] for k in ("lw", "tables", "refcounts", "free_list")},
          {k: resumed[k] for k in ("lw", "tables", "refcounts", "free_list")})
    assert straight["free_top"] == resumed["free_top"] and straight["L"] == resumed["L"]
    assert oracle.kv_check(resumed["tables"], math.ceil((resumed["L"] + cfg.K + 1) / cfg.block_size),
                           resumed["refcounts"], resumed["free_list"],
                           resumed["free_top"]).tolist() == [0] * 5
