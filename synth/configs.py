"""Workload shapes of the decode step (pure data, no arithmetic).

Every workload is synthetic.  The shapes follow the model shapes the LowRAM
pages name (Llama-3-8B / Mistral-7B style GQA: 32 layers, 32 query heads,
8 KV heads, head dim 128) and the 262K-token peak-throughput point of the
LowRAM review (agihunt.info), results paragraph.  The remaining knobs (chunk
size, top-k, window, rank, MLP width, residual fraction, RoPE base) are the
synthetic instance this library is built and measured on.

Derived sizes:
  P  = ctx - window          prefix tokens (chunked, compressed)
  nC = P / chunk             chunks in the prefix
  nR = floor(resid_frac * P) stored residual rows per (sequence, layer, KV head)
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int            # selects the seed family
    batch: int             # NB
    ctx: int               # T
    window: int            # W, exact recent tokens
    n_layers: int          # L
    group_layers: int      # G, layers sharing one key basis
    n_heads_q: int         # Hq
    n_heads_kv: int        # Hkv
    rank: int              # r, coefficients per token per layer-group
    topk: int              # chunks selected per KV head per step
    resid_frac: float      # fraction of prefix tokens with a stored residual
    rope_theta: float
    head_dim: int = 128    # d
    chunk: int = 8         # S
    mlp_hidden: int = 256  # H
    latent_dim: int = 64   # dimension of the key latents
    key_noise_std: float = 0.05
    laplace_scale: float = 0.02
    spike_frac: float = 0.03
    needle: bool = False   # plant one high-affinity chunk per KV head in q
    int4: bool = False     # coefficients and residuals stored int4, group 32
    evict: bool = False    # per-head eviction of half of the non-sink chunks
    n_sinks: int = 4
    bias_std: float = 0.0  # MLP biases (zero in the named workloads)

    # ---- derived -------------------------------------------------------
    @property
    def prefix(self) -> int:
        return self.ctx - self.window

    @property
    def n_chunks(self) -> int:
        return self.prefix // self.chunk

    @property
    def n_groups(self) -> int:
        return self.n_layers // self.group_layers

    @property
    def n_resid(self) -> int:
        return int(self.resid_frac * self.prefix)

    @property
    def gqa(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def group_dim(self) -> int:
        """Width of the concatenated keys one basis spans (G * Hkv * d)."""
        return self.group_layers * self.n_heads_kv * self.head_dim

    @property
    def n_cand(self) -> int:
        """Candidate chunks per KV head (survivors when eviction is on)."""
        if not self.evict:
            return self.n_chunks
        return self.n_chunks - self.n_chunks // 2

    @property
    def sel_tokens(self) -> int:
        return min(self.topk, self.n_cand) * self.chunk

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# Tiny single step: one layer-group of two layers, 4K context.
C0 = Config(name="c0_tiny_4k", cfg_id=0, batch=1, ctx=4096, window=64,
            n_layers=2, group_layers=2, n_heads_q=8, n_heads_kv=2, rank=64,
            topk=32, resid_frac=0.125, rope_theta=1e4)

# Llama-3-8B-shaped full step at 32K.
C1 = Config(name="c1_llama8b_32k", cfg_id=1, batch=1, ctx=32768, window=128,
            n_layers=32, group_layers=4, n_heads_q=32, n_heads_kv=8,
            rank=512, topk=256, resid_frac=0.125, rope_theta=5e5)

# Mistral-7B-shaped 128K step with a planted needle chunk per head.
# The RoPE base is not given for this workload; 1e6 is the long-context
# convention of that model family.
C2 = Config(name="c2_mistral7b_128k_needle", cfg_id=2, batch=4, ctx=131072,
            window=128, n_layers=32, group_layers=4, n_heads_q=32,
            n_heads_kv=8, rank=512, topk=512, resid_frac=0.125,
            rope_theta=1e6, needle=True)

# Peak-throughput point: 262K context, batch 28 (swept 1, 4, 8, 16, 28).
C3 = Config(name="c3_llama8b_262k", cfg_id=3, batch=28, ctx=262144,
            window=256, n_layers=32, group_layers=4, n_heads_q=32,
            n_heads_kv=8, rank=512, topk=1024, resid_frac=0.125,
            rope_theta=5e5)
C3_BATCHES = (1, 4, 8, 16, 28)

# Composed quantisation + eviction at 262K, batch 16.
C4 = Config(name="c4_eq_int4_evict_262k", cfg_id=4, batch=16, ctx=262144,
            window=256, n_layers=32, group_layers=4, n_heads_q=32,
            n_heads_kv=8, rank=512, topk=512, resid_frac=0.25,
            rope_theta=5e5, int4=True, evict=True)

CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4)}
BY_ID = {c.cfg_id: c for c in (C0, C1, C2, C3, C4)}
