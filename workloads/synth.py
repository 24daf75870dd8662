"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the CPU oracle's tests.

What is generated (all from fixed seeds):
  * target logits  [S, K+1, V]  and draft logits [S, K, V]   (S = B*N sequences)
      - "normal": target ~ Normal(0, sigma_t); draft = target + Normal(0, sigma_d)
      - "zipf":   target[v] = -a*ln(rank(v)) + Normal(0, sigma_t) with one seeded
                  permutation rank(.) of the vocabulary per configuration, shared by
                  every row; draft = target + Normal(0, sigma_d)
    stored as fp32 or bf16 (round-to-nearest-even by torch).
  * draft tokens [S, K] int32 drawn from softmax(draft / T) - this stands in for the
    draft model's Extend step, which lies before the verify path.
  * the initial paged-KV bookkeeping: a block table per sequence, refcounts and a free
    stack holding block ids P-1 .. 0 (so pops hand out 0, 1, 2, ...), with the ctx0
    prompt tokens already allocated - once per prompt with refcount N when the prefix
    is shared, once per sequence otherwise.

Nothing here computes a step of the verify / resample / KV-exchange method itself.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np
import torch

from .configs import Config

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(cfg: Config) -> torch.dtype:
    return _TORCH_DTYPE[cfg.dtype]


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def zipf_base(cfg: Config, device) -> torch.Tensor:
    """-a*ln(rank) over one seeded permutation of the vocabulary (fp32, [V])."""
    g = _gen("cpu", cfg.data_seed * 7919 + 17)
    perm = torch.randperm(cfg.V, generator=g)
    rank = (perm + 1).to(torch.float64)
    return (-cfg.zipf_a * torch.log(rank)).to(torch.float32).to(device)


def make_logit_set(cfg: Config, set_index: int, device="cpu",
                   base: torch.Tensor | None = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One logit set: (target [S, K+1, V], draft [S, K, V]) in the configuration dtype."""
    S, K, V = cfg.S, cfg.K, cfg.V
    g = _gen(device, cfg.data_seed * 1_000_003 + set_index * 7_919 + 1)
    dt = torch_dtype(cfg)
    target = torch.empty((S, K + 1, V), dtype=dt, device=device)
    draft = torch.empty((S, K, V), dtype=dt, device=device) if K > 0 else \
        torch.empty((S, 0, V), dtype=dt, device=device)
    if cfg.target_kind == "zipf" and base is None:
        base = zipf_base(cfg, device)
    # generate sequence blocks to bound temporaries
    chunk = max(1, (1 << 26) // max(1, (K + 1) * V))
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        n = s1 - s0
        t = torch.randn((n, K + 1, V), generator=g, device=device, dtype=torch.float32)
        t.mul_(cfg.target_sigma)
        if cfg.target_kind == "zipf":
            t.add_(base)
        target[s0:s1] = t.to(dt)
        if K > 0:
            d = t[:, :K] + cfg.draft_sigma * torch.randn((n, K, V), generator=g, device=device,
                                                         dtype=torch.float32)
            draft[s0:s1] = d.to(dt)
        del t
    return target, draft


def sample_draft_tokens(cfg: Config, draft: torch.Tensor, set_index: int) -> torch.Tensor:
    """Draft tokens x[s, k] ~ softmax(draft[s, k] / T) (the Extend step's output), int32 [S, K]."""
    S, K, V = cfg.S, cfg.K, cfg.V
    out = torch.empty((S, K), dtype=torch.int32, device=draft.device)
    if K == 0:
        return out
    g = _gen(draft.device, cfg.data_seed * 104_729 + set_index * 31 + 5)
    flat = draft.reshape(S * K, V)
    rows = max(1, (1 << 26) // V)
    res = out.view(S * K)
    for r0 in range(0, S * K, rows):
        r1 = min(S * K, r0 + rows)
        pr = torch.softmax(flat[r0:r1].float() / cfg.temperature, dim=-1)
        res[r0:r1] = torch.multinomial(pr, 1, generator=g).view(-1).to(torch.int32)
    return out


def initial_kv(cfg: Config) -> Dict[str, object]:
    """Initial block tables / refcounts / free stack with ctx0 tokens allocated.

    The free stack is free_list[0..top) with the top at index top-1; it starts as
    P-1, ..., 1, 0 so that successive pops return ascending ids.  Prompt blocks are
    popped in ascending (sequence, slot) order; a shared prefix is popped once per
    prompt and referenced by all N particles (refcount N)."""
    B, N, M, bs, P = cfg.B, cfg.N, cfg.M_cap, cfg.block_size, cfg.pool
    S = B * N
    nb0 = math.ceil(cfg.ctx0 / bs)
    tables = np.full((S, M), -1, dtype=np.int32)
    rc = np.zeros(P, dtype=np.int32)
    free_list = np.arange(P - 1, -1, -1, dtype=np.int32)
    nxt = 0
    if cfg.shared_prefix:
        for b in range(B):
            ids = np.arange(nxt, nxt + nb0, dtype=np.int32)
            tables[b * N:(b + 1) * N, :nb0] = ids[None, :]
            rc[ids] = N
            nxt += nb0
    else:
        for s in range(S):
            ids = np.arange(nxt, nxt + nb0, dtype=np.int32)
            tables[s, :nb0] = ids
            rc[ids] = 1
            nxt += nb0
    return {
        "tables": tables,
        "refcounts": rc,
        "free_list": free_list,
        "free_top": np.array([P - nxt], dtype=np.int32),
        "seq_len": cfg.ctx0,
    }


def initial_log_weights(cfg: Config) -> np.ndarray:
    return np.zeros(cfg.S, dtype=np.float32)
