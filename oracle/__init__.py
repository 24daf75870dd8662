"""CPU oracle for the SMC-SD verify / resample / KV pointer-exchange path.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``smc_verification_resampling_amd``) never imports it, and this package never
imports the product path: the two share no code.

The arithmetic lives in ``smcsd_oracle.c`` (plain C99, fp64, ascending-order sums);
this module only builds it with gcc and marshals numpy arrays through ctypes.
bf16 logits are passed as their uint16 bit patterns (dtype code 1); fp32 as float32
(dtype code 0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "smcsd_oracle.c")
LIB = os.path.join(HERE, "liboracle_smcsd.so")

ST_NAN_INPUT = 1
ST_EMPTY_ROW = 2
ST_NOSPACE = 4
ST_DEGENERATE_WEIGHTS = 8
ST_BAD_INPUT = 16
ST_KV_INCONSISTENT = 32

TAG_BONUS = 1
TAG_RESAMPLE = 2
TAG_SPS_ACCEPT = 3
TAG_SPS_FINAL = 4
TAG_DRAFT = 5
TAG_RACE = 6

BONUS_RULES = {"cdf": 0, "race": 1}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i64, u64, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_philox4x32_10.restype = None
    lib.orc_uniform.argtypes = [u64, ctypes.c_uint32, u64, ctypes.c_uint32, ctypes.c_int]
    lib.orc_uniform.restype = dbl
    lib.orc_row_lse.argtypes = [P, ctypes.c_int, i64, dbl, P]
    lib.orc_row_lse.restype = dbl
    lib.orc_verify_smc.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_int, P, ctypes.c_int, P,
                                   dbl, dbl, u64, u64, P, P, ctypes.c_int, P, P, P, P, P, P, P,
                                   P]
    lib.orc_verify_smc.restype = ctypes.c_int
    lib.orc_verify_sps.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_int, P, ctypes.c_int, P,
                                   dbl, u64, u64, P, P, P, P, P, P, P, P]
    lib.orc_verify_sps.restype = ctypes.c_int
    lib.orc_draft_sample.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, P, ctypes.c_int, dbl,
                                     u64, u64, P, P, P, P]
    lib.orc_draft_sample.restype = ctypes.c_int
    lib.orc_race_clock.argtypes = [u64, ctypes.c_uint32, u64, i64]
    lib.orc_race_clock.restype = dbl
    lib.orc_race_sample.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, P, dbl, u64, u64, P, P]
    lib.orc_race_sample.restype = ctypes.c_int
    lib.orc_resample.argtypes = [P, ctypes.c_int, ctypes.c_int, dbl, u64, u64,
                                 P, P, P, P, P, P, P]
    lib.orc_resample.restype = ctypes.c_int
    lib.orc_kv_reassign.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
                                    ctypes.c_int, i64, ctypes.c_int, P, P, P, ctypes.c_int,
                                    P, P, P]
    lib.orc_kv_reassign.restype = ctypes.c_int
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = configure(ctypes.CDLL(LIB))
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls (the default is every core)."""
    _load().orc_set_threads(int(n))


def _logit_array(x: np.ndarray):
    """(contiguous array, dtype code): float32 -> 0, uint16 (bf16 bits) -> 1."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:
        return x, 1
    raise TypeError("logits must be float32 or uint16 (bf16 bit patterns), got %s" % x.dtype)


# --------------------------------------------------------------------------- RNG
def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def uniform(seed: int, index: int, t: int, tag: int, word: int = 0) -> float:
    return float(_load().orc_uniform(seed, index, t, tag, word))


# --------------------------------------------------------------------------- rows
def row_lse(row: np.ndarray, T: float = 1.0):
    """(LSE of z = row / T in fp64, status bits)."""
    r, code = _logit_array(row.reshape(-1))
    st = np.zeros(1, dtype=np.int32)
    val = _load().orc_row_lse(_p(r), code, r.shape[0], T, _p(st))
    return float(val), int(st[0])


# --------------------------------------------------------------------------- verify
def verify_smc(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
               T: float, alpha: float, seed: int, t: int, lw_in: np.ndarray,
               rng_index: Optional[np.ndarray] = None,
               logq_in: Optional[np.ndarray] = None, bonus: str = "cdf") -> Dict[str, np.ndarray]:
    """SMC verify for nseq sequences.  target [nseq, K+1, V], draft [nseq, K, V]; with
    logq_in [nseq, K] (the draft's log-probabilities of its tokens) the draft rows are not
    read and draft may be None.  bonus: "cdf" (inverse CDF) or "race" (exponential race);
    with "race", margin is the gap between the two largest race keys."""
    tg, code = _logit_array(target)
    nseq, K1, V = tg.shape
    K = K1 - 1
    if logq_in is None:
        dr, code2 = _logit_array(draft.reshape(nseq, K, V))
        assert code == code2
        lq_in = None
    else:
        dr = np.zeros(1, np.float32)
        lq_in = np.ascontiguousarray(logq_in, dtype=np.float64).reshape(nseq, K)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(nseq, K)
    idx = np.arange(nseq, dtype=np.int64) if rng_index is None else \
        np.ascontiguousarray(rng_index, dtype=np.int64)
    lw = np.ascontiguousarray(lw_in, dtype=np.float64).reshape(nseq)
    out = {
        "lw": np.zeros(nseq, np.float64),
        "tokens": np.zeros((nseq, K + 1), np.int32),
        "logp": np.zeros((nseq, K + 1), np.float64),
        "lse": np.zeros((nseq, 2 * K + 1), np.float64),
        "u": np.zeros(nseq, np.float64),
        "margin": np.zeros(nseq, np.float64),
        "status": np.zeros(1, np.int32),
    }
    logq_buf = np.zeros((nseq, max(K, 1)), np.float64)
    _load().orc_verify_smc(_p(tg), _p(dr), code, V, nseq, _p(idx), K, _p(tok), T, alpha, seed, t,
                           _p(lw), None if lq_in is None else _p(lq_in), BONUS_RULES[bonus],
                           _p(out["lw"]),
                           _p(out["tokens"]), _p(out["logp"]),
                           _p(logq_buf), _p(out["lse"]), _p(out["u"]), _p(out["margin"]),
                           _p(out["status"]))
    out["logq"] = logq_buf[:, :K].copy()
    out["status"] = int(out["status"][0])
    return out


def draft_sample(rows: np.ndarray, T: float, seed: int, t: int, pos: int,
                 rng_index: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Draft-side sampler: one token per row from softmax(rows / T) and its log q.
    rows [n, V]; the RNG stream index of row r is rng_index[r] (default r)."""
    rw, code = _logit_array(rows)
    n, V = rw.shape
    idx = np.arange(n, dtype=np.int64) if rng_index is None else \
        np.ascontiguousarray(rng_index, dtype=np.int64)
    out = {"tokens": np.zeros(n, np.int32), "logq": np.zeros(n, np.float64),
           "margin": np.zeros(n, np.float64), "status": np.zeros(1, np.int32)}
    _load().orc_draft_sample(_p(rw), code, V, n, _p(idx), pos, T, seed, t, _p(out["tokens"]),
                             _p(out["logq"]), _p(out["margin"]), _p(out["status"]))
    out["status"] = int(out["status"][0])
    return out


def race_clock(seed: int, index: int, t: int, v: int) -> float:
    """E_v = -ln u_v, the exponential clock of token v in stream (seed; index, t)."""
    return float(_load().orc_race_clock(seed, index, t, v))


def race_sample(rows: np.ndarray, T: float, seed: int, t: int,
                rng_index: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Exponential-race draw, one token per row from softmax(rows / T).  rows [n, V];
    margin = gap between the two largest keys z_v - ln E_v."""
    rw, code = _logit_array(rows)
    n, V = rw.shape
    idx = np.arange(n, dtype=np.int64) if rng_index is None else \
        np.ascontiguousarray(rng_index, dtype=np.int64)
    out = {"tokens": np.zeros(n, np.int32), "margin": np.zeros(n, np.float64)}
    _load().orc_race_sample(_p(rw), code, V, n, _p(idx), T, seed, t, _p(out["tokens"]),
                            _p(out["margin"]))
    return out


def verify_sps(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray, T: float,
               seed: int, t: int, rng_index: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """SpS modified-rejection verify.  target [nseq, K+1, V], draft [nseq, K, V]."""
    tg, code = _logit_array(target)
    nseq, K1, V = tg.shape
    K = K1 - 1
    dr, code2 = _logit_array(draft.reshape(nseq, K, V))
    assert code == code2
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(nseq, K)
    idx = np.arange(nseq, dtype=np.int64) if rng_index is None else \
        np.ascontiguousarray(rng_index, dtype=np.int64)
    out = {
        "tokens": np.zeros((nseq, K + 1), np.int32),
        "num_tokens": np.zeros(nseq, np.int32),
        "logp": np.zeros((nseq, K + 1), np.float64),
        "lse": np.zeros((nseq, 2 * K + 1), np.float64),
        "margin_accept": np.zeros(nseq, np.float64),
        "margin_final": np.zeros(nseq, np.float64),
        "status": np.zeros(1, np.int32),
    }
    logq_buf = np.zeros((nseq, max(K, 1)), np.float64)
    _load().orc_verify_sps(_p(tg), _p(dr), code, V, nseq, _p(idx), K, _p(tok), T, seed, t,
                           _p(out["tokens"]), _p(out["num_tokens"]), _p(out["logp"]),
                           _p(logq_buf), _p(out["lse"]), _p(out["margin_accept"]),
                           _p(out["margin_final"]), _p(out["status"]))
    out["logq"] = logq_buf[:, :K].copy()
    out["status"] = int(out["status"][0])
    return out


# --------------------------------------------------------------------------- resample
def resample(lw_in: np.ndarray, tau: float, seed: int, t: int) -> Dict[str, np.ndarray]:
    """ESS + systematic resampling per prompt.  lw_in float32 [B, N]."""
    lw = np.ascontiguousarray(lw_in, dtype=np.float32)
    B, N = lw.shape
    out = {
        "lw": np.zeros((B, N), np.float64),
        "ancestors": np.zeros((B, N), np.int32),
        "ess": np.zeros(B, np.float64),
        "resampled": np.zeros(B, np.int32),
        "margin_ess": np.zeros(B, np.float64),
        "margin_pos": np.zeros((B, N), np.float64),
        "status": np.zeros(1, np.int32),
    }
    rc = _load().orc_resample(_p(lw), B, N, tau, seed, t, _p(out["lw"]), _p(out["ancestors"]),
                              _p(out["ess"]), _p(out["resampled"]), _p(out["margin_ess"]),
                              _p(out["margin_pos"]), _p(out["status"]))
    if rc != 0:
        raise MemoryError("orc_resample failed")
    out["status"] = int(out["status"][0])
    return out


# --------------------------------------------------------------------------- KV
def kv_reassign(ancestors: np.ndarray, resampled: np.ndarray, tables: np.ndarray, block_size: int,
                seq_len: int, reserve: int, refcounts: np.ndarray, free_list: np.ndarray,
                free_top: int) -> Dict[str, np.ndarray]:
    """Refcounted block-table pointer exchange + reservation.  Returns new copies."""
    anc = np.ascontiguousarray(ancestors, dtype=np.int32)
    B, N = anc.shape
    res = np.ascontiguousarray(resampled, dtype=np.int32).reshape(B)
    T = np.array(tables, dtype=np.int32, copy=True, order="C")
    S, M = T.shape
    assert S == B * N
    rc = np.array(refcounts, dtype=np.int32, copy=True)
    fl = np.array(free_list, dtype=np.int32, copy=True)
    P = rc.shape[0]
    top = np.array([free_top], dtype=np.int32)
    cow = np.full((S, 3), -1, dtype=np.int32)
    ncow = np.zeros(1, dtype=np.int32)
    st = np.zeros(1, dtype=np.int32)
    r = _load().orc_kv_reassign(_p(anc), _p(res), B, N, _p(T), M, block_size, seq_len, reserve,
                                _p(rc), _p(fl), _p(top), P, _p(cow), _p(ncow), _p(st))
    if r != 0:
        raise ValueError("orc_kv_reassign rejected its arguments (capacity or allocation)")
    return {"tables": T, "refcounts": rc, "free_list": fl, "free_top": int(top[0]),
            "cow": cow[: int(ncow[0])].copy(), "cow_count": int(ncow[0]), "status": int(st[0])}


def kv_check(tables: np.ndarray, slots: int, refcounts: np.ndarray, free_list: np.ndarray,
             free_top: int) -> np.ndarray:
    """The block-table state's invariants, counted by kind (SMC explainers, "system
    optimisation design": blocks shared by pointer and released by reference count).  The
    definition, in numpy, of what a consistent state is:
      [0] blocks whose refcount differs from the number of allocated slots naming them;
      [1] allocated slots holding an id outside [0, P) other than the -1 of an unfilled slot;
      [2] free-stack entries outside [0, P), extra occurrences of a block on the stack, and
          a top outside [0, P] (counted once, then clamped);
      [3] blocks on the free stack whose refcount is positive;
      [4] blocks whose refcount is <= 0 and that are not on the free stack.
    All zero: live and free blocks partition the pool and every count is exact."""
    T = np.asarray(tables, dtype=np.int64)[:, :slots]
    rc = np.asarray(refcounts, dtype=np.int64)
    P = rc.shape[0]
    v = np.zeros(5, dtype=np.int64)
    ids = T.ravel()
    inr = (ids >= 0) & (ids < P)
    v[1] = np.count_nonzero(~inr & (ids != -1))
    refs = np.bincount(ids[inr], minlength=P)
    v[0] = np.count_nonzero(refs != rc)
    top = int(free_top)
    if top < 0 or top > P:
        v[2] += 1
        top = min(max(top, 0), P)
    fr = np.asarray(free_list, dtype=np.int64)[:top]
    okf = (fr >= 0) & (fr < P)
    v[2] += np.count_nonzero(~okf)
    occ = np.bincount(fr[okf], minlength=P)
    v[2] += int(np.maximum(occ - 1, 0).sum())
    v[3] = np.count_nonzero((occ > 0) & (rc > 0))
    v[4] = np.count_nonzero((occ == 0) & (rc <= 0))
    return v
