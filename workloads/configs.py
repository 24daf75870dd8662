"""Synthetic workload definitions for the SMC-SD verify / resample path.

Five configurations, each a synthetic stand-in for the logits that the target and
draft models of the SMC-SD explainers ("Faster LLM Inference via Sequential Monte
Carlo", §4 experimental results: Llama and Qwen families on GSM8K, MATH500,
AlpacaEval, DS1000) would produce.  No model weights or dataset items are used:
vocabulary sizes follow the public tokenizer sizes (32000, 128256, 152064) and the
Zipf generator mimics next-token statistics.

Every value that a configuration leaves unstated is filled with an explicit reading
(temperature 1.0, alpha 1, tau 0.5, block size 16, unshared blocks) and marked in
the field ``readings``.

This module holds only sizes, seeds and generator parameters; it does none of the
method's arithmetic.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int                 # prompts
    N: int                 # particles per prompt
    K: int                 # draft tokens per round
    V: int                 # vocabulary size
    dtype: str             # "f32" or "bf16" logits
    target_kind: str       # "normal" or "zipf"
    target_sigma: float    # Normal sigma (normal) or per-element noise sigma (zipf)
    draft_sigma: float     # draft = target + Normal(0, draft_sigma)
    temperature: float
    alpha: float           # target log-density = alpha * log_softmax(l / T)
    tau: float             # resample iff ESS < tau * N
    ctx0: int              # initial context length in tokens
    block_size: int        # tokens per KV block
    shared_prefix: bool    # initial ctx0 blocks shared by the N particles of a prompt
    iters: int             # SMC rounds
    n_sets: int            # distinct logit sets; round t uses set t mod n_sets
    sps: bool = False      # also run the SpS verify on particle 0 of every prompt
    data_seed: int = 0
    rng_seed: int = 0
    zipf_a: float = 1.1
    readings: Tuple[str, ...] = ()

    # ---- derived sizes -------------------------------------------------------
    @property
    def S(self) -> int:
        return self.B * self.N

    @property
    def rows_per_seq(self) -> int:
        return 2 * self.K + 1

    @property
    def M_cap(self) -> int:
        # ctx0 tokens, one reservation of K+1 before round 0, one per round after it
        return math.ceil((self.ctx0 + (self.iters + 1) * (self.K + 1)) / self.block_size)

    @property
    def pool(self) -> int:
        return self.B * self.N * self.M_cap

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def logit_bytes_per_step(self) -> int:
        return self.B * self.N * self.rows_per_seq * self.V * self.elt_bytes

    def scaled(self, **kw) -> "Config":
        """A copy with some sizes replaced (downsized parity cases)."""
        d = dataclasses.asdict(self)
        d.update(kw)
        d["readings"] = tuple(d["readings"])
        return Config(**d)


C1 = Config(
    name="c1_tiny", B=1, N=4, K=2, V=8, dtype="f32",
    target_kind="normal", target_sigma=1.0, draft_sigma=0.5,
    temperature=1.0, alpha=1.0, tau=0.5, ctx0=16, block_size=4, shared_prefix=False,
    iters=10, n_sets=10, data_seed=101, rng_seed=1001,
    readings=("temperature=1.0", "ctx0=16 (4 blocks of 4)", "unshared blocks"),
)

C2 = Config(
    name="c2_single_prompt", B=1, N=8, K=4, V=32000, dtype="bf16",
    target_kind="normal", target_sigma=2.0, draft_sigma=1.0,
    temperature=1.0, alpha=1.0, tau=0.5, ctx0=512, block_size=16, shared_prefix=False,
    iters=1000, n_sets=256, data_seed=202, rng_seed=2002,
    readings=("unshared blocks",),
)

C3 = Config(
    name="c3_batched", B=32, N=16, K=4, V=128256, dtype="bf16",
    target_kind="zipf", target_sigma=0.3, draft_sigma=0.8,
    temperature=0.8, alpha=1.0, tau=0.5, ctx0=2048, block_size=16, shared_prefix=True,
    iters=500, n_sets=4, data_seed=303, rng_seed=3003,
    readings=(),
)

C4 = Config(
    name="c4_wide_particle", B=16, N=64, K=8, V=128256, dtype="f32",
    target_kind="zipf", target_sigma=0.3, draft_sigma=1.2,
    temperature=1.0, alpha=1.0, tau=0.5, ctx0=4096, block_size=16, shared_prefix=False,
    iters=200, n_sets=2, sps=True, data_seed=404, rng_seed=4004,
    readings=("temperature=1.0", "tau=0.5", "block_size=16", "unshared blocks"),
)

C5 = Config(
    name="c5_power", B=8, N=128, K=5, V=152064, dtype="bf16",
    target_kind="zipf", target_sigma=0.3, draft_sigma=1.0,
    temperature=1.0, alpha=4.0, tau=0.3, ctx0=4096, block_size=16, shared_prefix=True,
    iters=200, n_sets=4, data_seed=505, rng_seed=5005,
    readings=("temperature=1.0",),
)

ALL = (C1, C2, C3, C4, C5)
BY_NAME = {c.name: c for c in ALL}


def get(name: str) -> Config:
    return BY_NAME[name]


def downsized(cfg: Config, B: Optional[int] = None, V: Optional[int] = None,
              iters: Optional[int] = None, n_sets: Optional[int] = None) -> Config:
    """Same generator, dtype, K, N, T, alpha, tau and block rules at a size the CPU
    oracle finishes in seconds."""
    return cfg.scaled(
        name=cfg.name + "_small",
        B=B if B is not None else min(cfg.B, 2),
        V=V if V is not None else cfg.V,
        iters=iters if iters is not None else min(cfg.iters, 12),
        n_sets=n_sets if n_sets is not None else min(cfg.n_sets, 3),
    )
