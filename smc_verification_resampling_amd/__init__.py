"""Python binding of libsmcsd.so - the MI355X (gfx950) SMC-SD verify / resample / KV path.

Argument marshalling only: every step of the path runs in the library's HIP kernels.
Tensors must be device (HIP) tensors; this module checks placement, dtype, contiguity
and sizes so that no host pointer or short buffer reaches a kernel, passes raw pointers
and the current torch stream, and turns negative return codes into ``SmcsdError``.
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmcsd.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
MODE_SMC, MODE_SPS, MODE_SMC_RACE = 0, 1, 2  # MODE_SMC_RACE: SMC with the exponential-race bonus
OP_VERIFY_SMC, OP_VERIFY_SPS, OP_KV, OP_DRAFT, OP_KV_CHECK = 0, 1, 2, 3, 4
STATIC_SCRATCH_BYTES = 4 << 20  # smcsd_verify_static's per-GPU scratch array

ST_NAN_INPUT = 1
ST_EMPTY_ROW = 2
ST_NOSPACE = 4
ST_DEGENERATE_WEIGHTS = 8
ST_BAD_INPUT = 16
ST_KV_INCONSISTENT = 32
KV_CHECK_KINDS = 5
STREAM_READ_TILE_BYTES = 131072
KV_CHECK_NAMES = ("refcount != table references", "table id out of range",
                  "free-stack entry out of range or repeated", "referenced block on the free stack",
                  "unreferenced block not on the free stack")

EXPORTED = ("smcsd_version", "smcsd_status_string", "smcsd_workspace_bytes", "smcsd_verify",
            "smcsd_verify_static", "smcsd_draft_sample", "smcsd_resample", "smcsd_kv_reassign",
            "smcsd_resample_kv_reassign", "smcsd_step", "smcsd_kv_check", "smcsd_philox4x32_10",
            "smcsd_stream_read")

_DT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


class SmcsdError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsmcsd.so and declare the C signatures (no GPU work)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise SmcsdError("libsmcsd.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    P, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_float, ctypes.c_size_t)
    lib.smcsd_version.restype = i32
    lib.smcsd_status_string.argtypes = [i32]
    lib.smcsd_status_string.restype = ctypes.c_char_p
    lib.smcsd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i64]
    lib.smcsd_workspace_bytes.restype = sz
    lib.smcsd_verify.argtypes = [P, P, i32, i64, i32, P, i32, i32, i32, i32, f32, f32, i32, u64,
                                 u64, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.smcsd_verify.restype = i32
    lib.smcsd_verify_static.argtypes = [P, P, i32, i64, i32, P, i32, i32, i32, i32, f32, f32, i32,
                                        u64, u64, P, P, P, P, P, P, P, P, P, P]
    lib.smcsd_verify_static.restype = i32
    lib.smcsd_draft_sample.argtypes = [P, i32, i64, i32, i32, f32, u64, u64, i32, P, P, P, P, sz, P]
    lib.smcsd_draft_sample.restype = i32
    lib.smcsd_resample.argtypes = [P, i32, i32, f32, u64, u64, P, P, P, P, P]
    lib.smcsd_resample.restype = i32
    lib.smcsd_kv_reassign.argtypes = [P, P, i32, i32, P, i32, i32, i64, i32, P, P, P, i64, P, P,
                                      P, P, sz, P]
    lib.smcsd_kv_reassign.restype = i32
    lib.smcsd_resample_kv_reassign.argtypes = [P, i32, i32, f32, u64, u64, P, P, P, P, i32, i32, i64,
                                               i32, P, P, P, i64, P, P, P, P, sz, P]
    lib.smcsd_resample_kv_reassign.restype = i32
    lib.smcsd_step.argtypes = [P, P, i32, i64, P, i32, i32, i32, i32, f32, f32, i32, f32, u64, u64,
                               P, P, P, P, P, P, P, P, P, P, P, i32, i32, i64, i32, P, P, P, i64,
                               P, P, P, P, sz, P, sz, P]
    lib.smcsd_step.restype = i32
    lib.smcsd_kv_check.argtypes = [P, i64, i32, i32, P, P, P, i64, P, P, P, sz, P]
    lib.smcsd_kv_check.restype = i32
    lib.smcsd_philox4x32_10.argtypes = [P, P, i32, P, P]
    lib.smcsd_philox4x32_10.restype = i32
    lib.smcsd_stream_read.argtypes = [P, i64, P, P]
    lib.smcsd_stream_read.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _L():
    return _lib if _lib is not None else load_library()


def _check(rc: int, what: str):
    if rc != 0:
        raise SmcsdError("%s failed: %s (%d)" % (what, _L().smcsd_status_string(rc).decode(), rc))


def status_string(code: int) -> str:
    return _L().smcsd_status_string(code).decode()


def version() -> int:
    return int(_L().smcsd_version())


def workspace_bytes(op: int, B: int, N: int, K: int = 0, V: int = 1, P: int = 0) -> int:
    return int(_L().smcsd_workspace_bytes(op, B, N, K, V, P))


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, min_numel: int = 0,
         contiguous: bool = True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SmcsdError("%s must be a device tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise SmcsdError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if contiguous and not t.is_contiguous():
        raise SmcsdError("%s must be contiguous" % name)
    if t.numel() < min_numel:
        raise SmcsdError("%s holds %d elements, needs %d" % (name, t.numel(), min_numel))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def alloc_workspace(op: int, B: int, N: int, K: int = 0, V: int = 1, P: int = 0,
                    device=None) -> torch.Tensor:
    """Zero-filled device workspace of the size the library asks for."""
    n = workspace_bytes(op, B, N, K, V, P)
    if n == 0:
        raise SmcsdError("invalid workspace sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def verify(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
           B: int, N: int, K: int, V: int, temperature: float, alpha: float, mode: int, seed: int,
           step: int, out_tokens: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
           log_weights: Optional[torch.Tensor] = None, out_num_tokens=None, out_logp=None,
           out_logq=None, out_lse=None, lse_in=None, seq_step: int = 1,
           row_stride: Optional[int] = None, stream=None, logq_in=None) -> None:
    """smcsd_verify.  target [*, K+1, row_stride], draft [*, K, row_stride] (bf16 or fp32).
    mode: MODE_SMC (bonus by inverse CDF), MODE_SMC_RACE (bonus by the exponential race)
    or MODE_SPS.  With logq_in [*, K] fp32 (the draft's log q of its tokens; SMC modes)
    draft may be None."""
    if target.dtype not in _DT:
        raise SmcsdError("logits must be bfloat16 or float32")
    rs = V if row_stride is None else int(row_stride)
    S = B * N
    nsrc = (S - 1) * seq_step + 1 if S > 0 else 0
    tp = _dev(target, "target", target.dtype, nsrc * (K + 1) * rs - (rs - V) if S else 0)
    dp = _dev(draft, "draft", target.dtype, nsrc * K * rs - (rs - V) if S and K else 0) \
        if K > 0 and (draft is not None or logq_in is None) else None
    xp = _dev(draft_tokens, "draft_tokens", torch.int32, nsrc * K) if K > 0 else None
    lw = _dev(log_weights, "log_weights", torch.float32, S)
    rc = _L().smcsd_verify(
        tp, dp, _DT[target.dtype], rs, seq_step, xp, B, N, K, V, float(temperature), float(alpha),
        mode, int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
        _dev(lse_in, "lse_in", torch.float32, nsrc * (2 * K + 1)),
        _dev(logq_in, "logq_in", torch.float32, nsrc * K), lw,
        _dev(out_tokens, "out_tokens", torch.int32, S * (K + 1)),
        _dev(out_num_tokens, "out_num_tokens", torch.int32, S),
        _dev(out_logp, "out_logp", torch.float32, S * (K + 1)),
        _dev(out_logq, "out_logq", torch.float32, S * K),
        _dev(out_lse, "out_lse", torch.float32, S * (2 * K + 1)),
        _dev(status, "status", torch.int32, 1),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(rc, "smcsd_verify")


def verify_static(target: torch.Tensor, draft: Optional[torch.Tensor],
                  draft_tokens: Optional[torch.Tensor], B: int, N: int, K: int, V: int,
                  temperature: float, alpha: float, mode: int, seed: int, step: int,
                  out_tokens: torch.Tensor, status: torch.Tensor,
                  log_weights: Optional[torch.Tensor] = None, out_num_tokens=None, out_logp=None,
                  out_logq=None, out_lse=None, lse_in=None, seq_step: int = 1,
                  row_stride: Optional[int] = None, stream=None, logq_in=None) -> None:
    """smcsd_verify_static: smcsd_verify with the library's own per-GPU scratch array instead
    of a workspace (for callers that cannot allocate); same arguments otherwise.  Calls that
    overlap in time on one GPU race on that array."""
    if target.dtype not in _DT:
        raise SmcsdError("logits must be bfloat16 or float32")
    rs = V if row_stride is None else int(row_stride)
    S = B * N
    nsrc = (S - 1) * seq_step + 1 if S > 0 else 0
    tp = _dev(target, "target", target.dtype, nsrc * (K + 1) * rs - (rs - V) if S else 0)
    dp = _dev(draft, "draft", target.dtype, nsrc * K * rs - (rs - V) if S and K else 0) \
        if K > 0 and (draft is not None or logq_in is None) else None
    xp = _dev(draft_tokens, "draft_tokens", torch.int32, nsrc * K) if K > 0 else None
    lw = _dev(log_weights, "log_weights", torch.float32, S)
    rc = _L().smcsd_verify_static(
        tp, dp, _DT[target.dtype], rs, seq_step, xp, B, N, K, V, float(temperature), float(alpha),
        mode, int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
        _dev(lse_in, "lse_in", torch.float32, nsrc * (2 * K + 1)),
        _dev(logq_in, "logq_in", torch.float32, nsrc * K), lw,
        _dev(out_tokens, "out_tokens", torch.int32, S * (K + 1)),
        _dev(out_num_tokens, "out_num_tokens", torch.int32, S),
        _dev(out_logp, "out_logp", torch.float32, S * (K + 1)),
        _dev(out_logq, "out_logq", torch.float32, S * K),
        _dev(out_lse, "out_lse", torch.float32, S * (2 * K + 1)),
        _dev(status, "status", torch.int32, 1), _stream(stream))
    _check(rc, "smcsd_verify_static")


def draft_sample(draft: torch.Tensor, n: int, V: int, temperature: float, seed: int, step: int,
                 pos: int, out_tokens: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
                 out_logq: Optional[torch.Tensor] = None, row_stride: Optional[int] = None,
                 stream=None) -> None:
    """smcsd_draft_sample.  draft [n, row_stride] (bf16 or fp32) at one draft position."""
    if draft.dtype not in _DT:
        raise SmcsdError("logits must be bfloat16 or float32")
    rs = V if row_stride is None else int(row_stride)
    rc = _L().smcsd_draft_sample(
        _dev(draft, "draft", draft.dtype, n * rs - (rs - V) if n else 0), _DT[draft.dtype], rs, n,
        V, float(temperature), int(seed) & (2**64 - 1), int(step) & (2**64 - 1), int(pos),
        _dev(out_tokens, "out_tokens", torch.int32, n),
        _dev(out_logq, "out_logq", torch.float32, n), _dev(status, "status", torch.int32, 1),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(rc, "smcsd_draft_sample")


def resample(log_weights: torch.Tensor, B: int, N: int, tau: float, seed: int, step: int,
             ancestors: torch.Tensor, ess: torch.Tensor, resampled: torch.Tensor,
             status: torch.Tensor, stream=None) -> None:
    """smcsd_resample over log_weights [B, N]."""
    rc = _L().smcsd_resample(
        _dev(log_weights, "log_weights", torch.float32, B * N), B, N, float(tau),
        int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
        _dev(ancestors, "ancestors", torch.int32, B * N), _dev(ess, "ess", torch.float32, B),
        _dev(resampled, "resampled", torch.int32, B), _dev(status, "status", torch.int32, 1),
        _stream(stream))
    _check(rc, "smcsd_resample")


def kv_reassign(ancestors: torch.Tensor, resampled: torch.Tensor, B: int, N: int,
                block_tables: torch.Tensor, block_size: int, seq_len: int, reserve_tokens: int,
                refcounts: torch.Tensor, free_list: torch.Tensor, free_top: torch.Tensor,
                cow: torch.Tensor, cow_count: torch.Tensor, status: torch.Tensor,
                workspace: torch.Tensor, stream=None) -> None:
    """smcsd_kv_reassign.  block_tables [B*N, M_cap] int32; refcounts / free_list [P] int32."""
    if block_tables.dim() != 2 or block_tables.shape[0] != B * N:
        raise SmcsdError("block_tables must be [B*N, M_cap]")
    M_cap = block_tables.shape[1]
    P = refcounts.numel()
    rc = _L().smcsd_kv_reassign(
        _dev(ancestors, "ancestors", torch.int32, B * N), _dev(resampled, "resampled", torch.int32, B),
        B, N, _dev(block_tables, "block_tables", torch.int32), M_cap, block_size, int(seq_len),
        reserve_tokens, _dev(refcounts, "refcounts", torch.int32), _dev(free_list, "free_list",
                                                                       torch.int32, P),
        _dev(free_top, "free_top", torch.int32, 1), P, _dev(cow, "cow", torch.int32, 3 * B * N),
        _dev(cow_count, "cow_count", torch.int32, 1), _dev(status, "status", torch.int32, 1),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(rc, "smcsd_kv_reassign")
    _debug_kv_check(block_tables, block_size, seq_len, reserve_tokens, refcounts, free_list,
                    free_top, "smcsd_kv_reassign", stream)


def resample_kv_reassign(log_weights: torch.Tensor, B: int, N: int, tau: float, seed: int,
                         step: int, ancestors: torch.Tensor, ess: torch.Tensor,
                         resampled: torch.Tensor, block_tables: torch.Tensor, block_size: int,
                         seq_len: int, reserve_tokens: int, refcounts: torch.Tensor,
                         free_list: torch.Tensor, free_top: torch.Tensor, cow: torch.Tensor,
                         cow_count: torch.Tensor, status: torch.Tensor, workspace: torch.Tensor,
                         stream=None) -> None:
    """smcsd_resample_kv_reassign: resample then kv_reassign in one launch fewer."""
    if block_tables.dim() != 2 or block_tables.shape[0] != B * N:
        raise SmcsdError("block_tables must be [B*N, M_cap]")
    M_cap = block_tables.shape[1]
    P = refcounts.numel()
    rc = _L().smcsd_resample_kv_reassign(
        _dev(log_weights, "log_weights", torch.float32, B * N), B, N, float(tau),
        int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
        _dev(ancestors, "ancestors", torch.int32, B * N), _dev(ess, "ess", torch.float32, B),
        _dev(resampled, "resampled", torch.int32, B),
        _dev(block_tables, "block_tables", torch.int32), M_cap, block_size, int(seq_len),
        reserve_tokens, _dev(refcounts, "refcounts", torch.int32),
        _dev(free_list, "free_list", torch.int32, P), _dev(free_top, "free_top", torch.int32, 1), P,
        _dev(cow, "cow", torch.int32, 3 * B * N), _dev(cow_count, "cow_count", torch.int32, 1),
        _dev(status, "status", torch.int32, 1), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream))
    _check(rc, "smcsd_resample_kv_reassign")
    _debug_kv_check(block_tables, block_size, seq_len, reserve_tokens, refcounts, free_list,
                    free_top, "smcsd_resample_kv_reassign", stream)


def step(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
         B: int, N: int, K: int, V: int, temperature: float, alpha: float, mode: int, tau: float,
         seed: int, step: int, log_weights: torch.Tensor, out_tokens: torch.Tensor,
         ancestors: torch.Tensor, ess: torch.Tensor, resampled: torch.Tensor,
         block_tables: torch.Tensor, block_size: int, seq_len: int, reserve_tokens: int,
         refcounts: torch.Tensor, free_list: torch.Tensor, free_top: torch.Tensor,
         cow: torch.Tensor, cow_count: torch.Tensor, status: torch.Tensor,
         verify_workspace: torch.Tensor, kv_workspace: torch.Tensor, out_num_tokens=None,
         out_logp=None, out_logq=None, out_lse=None, logq_in=None,
         row_stride: Optional[int] = None, stream=None) -> None:
    """smcsd_step: smcsd_verify (MODE_SMC or MODE_SMC_RACE) then smcsd_resample_kv_reassign
    in one call (the same bits); seq_len is the length after this round's K+1 tokens."""
    if target.dtype not in _DT:
        raise SmcsdError("logits must be bfloat16 or float32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B * N:
        raise SmcsdError("block_tables must be [B*N, M_cap]")
    rs = V if row_stride is None else int(row_stride)
    S = B * N
    M_cap = block_tables.shape[1]
    P = refcounts.numel()
    tp = _dev(target, "target", target.dtype, S * (K + 1) * rs - (rs - V) if S else 0)
    dp = _dev(draft, "draft", target.dtype, S * K * rs - (rs - V) if S and K else 0) \
        if K > 0 and (draft is not None or logq_in is None) else None
    xp = _dev(draft_tokens, "draft_tokens", torch.int32, S * K) if K > 0 else None
    rc = _L().smcsd_step(
        tp, dp, _DT[target.dtype], rs, xp, B, N, K, V, float(temperature), float(alpha), mode,
        float(tau), int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
        _dev(logq_in, "logq_in", torch.float32, S * K),
        _dev(log_weights, "log_weights", torch.float32, S),
        _dev(out_tokens, "out_tokens", torch.int32, S * (K + 1)),
        _dev(out_num_tokens, "out_num_tokens", torch.int32, S),
        _dev(out_logp, "out_logp", torch.float32, S * (K + 1)),
        _dev(out_logq, "out_logq", torch.float32, S * K),
        _dev(out_lse, "out_lse", torch.float32, S * (2 * K + 1)),
        _dev(ancestors, "ancestors", torch.int32, S), _dev(ess, "ess", torch.float32, B),
        _dev(resampled, "resampled", torch.int32, B),
        _dev(block_tables, "block_tables", torch.int32), M_cap, block_size, int(seq_len),
        reserve_tokens, _dev(refcounts, "refcounts", torch.int32),
        _dev(free_list, "free_list", torch.int32, P), _dev(free_top, "free_top", torch.int32, 1), P,
        _dev(cow, "cow", torch.int32, 3 * S), _dev(cow_count, "cow_count", torch.int32, 1),
        _dev(status, "status", torch.int32, 1),
        _dev(verify_workspace, "verify_workspace", torch.uint8), verify_workspace.numel(),
        _dev(kv_workspace, "kv_workspace", torch.uint8), kv_workspace.numel(), _stream(stream))
    _check(rc, "smcsd_step")
    _debug_kv_check(block_tables, block_size, seq_len, reserve_tokens, refcounts, free_list,
                    free_top, "smcsd_step", stream)


def kv_check(block_tables: torch.Tensor, slots: int, refcounts: torch.Tensor,
             free_list: torch.Tensor, free_top: torch.Tensor, violations: torch.Tensor,
             status: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """smcsd_kv_check: violations [KV_CHECK_KINDS] int32 receives the counts (KV_CHECK_NAMES);
    workspace from alloc_workspace(OP_KV_CHECK, 0, 0, P=P)."""
    if block_tables.dim() != 2:
        raise SmcsdError("block_tables must be [S, M_cap]")
    S, M_cap = block_tables.shape
    P = refcounts.numel()
    rc = _L().smcsd_kv_check(
        _dev(block_tables, "block_tables", torch.int32), S, M_cap, int(slots),
        _dev(refcounts, "refcounts", torch.int32), _dev(free_list, "free_list", torch.int32, P),
        _dev(free_top, "free_top", torch.int32, 1), P,
        _dev(violations, "violations", torch.int32, KV_CHECK_KINDS),
        _dev(status, "status", torch.int32, 1), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream))
    _check(rc, "smcsd_kv_check")


def _debug_kv_check(block_tables, block_size, seq_len, reserve_tokens, refcounts, free_list,
                    free_top, what, stream):
    """With SMCSD_DEBUG_CHECK=1 in the environment: smcsd_kv_check after a KV call, waited
    for, raising SmcsdError on any violation (debug runs only: it synchronises the stream)."""
    if os.environ.get("SMCSD_DEBUG_CHECK") != "1":
        return
    dev = block_tables.device
    P = refcounts.numel()
    ws = alloc_workspace(OP_KV_CHECK, 0, 0, P=P, device=dev)
    viol = torch.zeros(KV_CHECK_KINDS, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    slots = -(-(int(seq_len) + int(reserve_tokens)) // int(block_size))
    kv_check(block_tables, slots, refcounts, free_list, free_top, viol, st, ws, stream)
    counts = viol.cpu().tolist()
    if any(counts):
        raise SmcsdError("%s left an inconsistent KV state: %s" % (what, ", ".join(
            "%s: %d" % (n, c) for n, c in zip(KV_CHECK_NAMES, counts) if c)))


def philox4x32_10(counters: torch.Tensor, keys: torch.Tensor, out: torch.Tensor, stream=None):
    """Device Philox4x32-10 blocks: counters [n, 4], keys [n, 2] -> out [n, 4] (int32 views)."""
    n = counters.shape[0]
    rc = _L().smcsd_philox4x32_10(_dev(counters, "counters", torch.int32, 4 * n),
                                  _dev(keys, "keys", torch.int32, 2 * n), n,
                                  _dev(out, "out", torch.int32, 4 * n), _stream(stream))
    _check(rc, "smcsd_philox4x32_10")


def stream_read(buf: torch.Tensor, tile_xor: torch.Tensor, stream=None):
    """Reads every byte of the contiguous device tensor `buf` once (16-byte aligned, a
    multiple of 16 bytes) and writes the XOR of each STREAM_READ_TILE_BYTES tile's 32-bit
    words to tile_xor (int32, one word per tile): the achievable HBM read rate that the LSE
    pass is compared with."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise SmcsdError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    ntiles = -(-nbytes // STREAM_READ_TILE_BYTES)
    rc = _L().smcsd_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                _dev(tile_xor, "tile_xor", torch.int32, ntiles), _stream(stream))
    _check(rc, "smcsd_stream_read")
