"""The five synthetic workloads, shaped like the models on the pages, plus
reduced variants of the same shapes for parity tests.

Stand-ins for the pages' LoCoMo runs: no dataset items are used; every input
is drawn from the seeded generator in this package.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

from . import (BF16, F32, block_tables, embeddings, len_lognormal, len_uniform,
               prefixes, queries, zipf_requests)


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_kv_heads: int
    head_dim: int
    dtype: int                      # F32 or BF16 (store and cache)
    n_facts: int
    len_dist: tuple                 # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    emb_dim: int                    # 0: no embedding index
    n_req: int
    k: int
    fact_choice: str                # "topk" | "zipf"
    prefix: tuple                   # (lo, hi), inclusive
    block_size: int
    n_blocks: int
    theta: float
    scaling: str = "none"           # "none" | "llama3"
    rope_factor: float = 8.0
    rope_low: float = 1.0
    rope_high: float = 4.0
    rope_orig: float = 8192.0
    zipf_s: float = 1.1
    host_fraction: float = 0.0      # fraction of facts (the highest ids) in host memory
    seed: int = 0

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def row_elems(self) -> int:
        """Elements of one token's K (or V) over all layers and heads."""
        return self.n_layers * self.n_kv_heads * self.head_dim

    @property
    def token_bytes(self) -> int:
        return self.row_elems * self.elem_size

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


LLAMA_STORE = dict(n_layers=32, n_kv_heads=8, head_dim=128, dtype=BF16,
                   n_facts=10_000, len_dist=("uniform", 12, 64), emb_dim=1024,
                   theta=500000.0, scaling="llama3")

WORKLOADS = {
    # Tiny: 1 layer, 2 KV heads, head_dim 64, fp32, 20 facts of 8-24 tokens,
    # 32-dim embeddings, 1 request, top-5, prefix 16, block 16, 16 blocks.
    "tiny": Workload("tiny", 1, 2, 64, F32, 20, ("uniform", 8, 24), 32, 1, 5, "topk",
                     (16, 16), 16, 16, 10000.0),
    # Llama-3.1-8B-shaped store, one request, k=5, prefix 32; it shares the
    # batch workload's cache geometry.
    "llama8b_single": Workload("llama8b_single", n_req=1, k=5, fact_choice="topk",
                               prefix=(32, 32), block_size=16, n_blocks=98_304,
                               **LLAMA_STORE),
    # Same store, 100 requests x 50 distinct Zipf(1.1) facts, prefixes 16-256.
    # 98,304 blocks x 16 slots: the 2M-slot cache of the description does not
    # fit next to the store in 288 GB.
    "llama8b_batch": Workload("llama8b_batch", n_req=100, k=50, fact_choice="zipf",
                              prefix=(16, 256), block_size=16, n_blocks=98_304,
                              **LLAMA_STORE),
    # Mistral-7B-shaped: lognormal lengths (median 32, sigma 0.5, clipped
    # 8-256), top-50 over 50,000 embeddings for 100 requests, block 32.
    "mistral7b_batch": Workload("mistral7b_batch", 32, 8, 128, BF16, 50_000,
                                ("lognormal", 32.0, 0.5, 8, 256), 1024, 100, 50,
                                "topk", (16, 256), 32, 7_168, 1e6),
    # Qwen2.5-7B-shaped: 1M facts, half of them (the upper ids) in pinned host
    # memory, exact top-50 over 1M embeddings for 100 queries, block 16.
    # Lengths 1-3 tokens (mean 2): the host half is then 57 GB, within the
    # 64 GiB of host memory an MI355X host here can pin (4-12 tokens would need
    # 229 GB pinned).
    "qwen7b_offload": Workload("qwen7b_offload", 28, 4, 128, BF16, 1_000_000,
                               ("uniform", 1, 3), 1024, 100, 50, "topk",
                               (16, 256), 16, 8_192, 1e6, host_fraction=0.5),
    # Qwen3-14B-shaped (shape from the public model card: 40 layers, 8 kv
    # heads, head_dim 128, RoPE theta 1e6): one request, top-50, half of the
    # 16,000 facts (lengths 12-64) in pinned host memory -- the single-request
    # latency of injecting from the host tier.  K+V: 163,840 B per token,
    # about 50 GB on each tier.
    "qwen3_14b_offload": Workload("qwen3_14b_offload", 40, 8, 128, BF16, 16_000,
                                  ("uniform", 12, 64), 1024, 1, 50, "topk",
                                  (32, 32), 16, 512, 1e6, host_fraction=0.5),
}


def fact_lengths(w: Workload) -> np.ndarray:
    d = w.len_dist
    if d[0] == "uniform":
        return len_uniform(w.seed, w.n_facts, d[1], d[2])
    if d[0] == "lognormal":
        return len_lognormal(w.seed, w.n_facts, d[1], d[2], d[3], d[4])
    raise ValueError(d)


def fact_embeddings(w: Workload) -> np.ndarray:
    return embeddings(w.seed, 0, w.n_facts, w.emb_dim)


def query_embeddings(w: Workload) -> np.ndarray:
    return queries(w.seed, w.n_req, w.emb_dim)


def zipf_fact_ids(w: Workload) -> np.ndarray:
    return zipf_requests(w.seed, w.n_req, w.k, w.n_facts, w.zipf_s)


def request_prefixes(w: Workload) -> np.ndarray:
    return prefixes(w.seed, w.n_req, w.prefix[0], w.prefix[1])


def request_block_tables(w: Workload, lens: np.ndarray, fact_ids: np.ndarray,
                         prefix: np.ndarray) -> np.ndarray:
    """Block tables sized for each request's prefix plus its facts (the
    allocation a serving engine makes once it knows the request's length)."""
    need = prefix.astype(np.int64) + lens[fact_ids].astype(np.int64).sum(axis=1)
    return block_tables(w.seed, need, w.block_size, w.n_blocks)
