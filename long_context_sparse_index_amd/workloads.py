"""The DSA workloads this library is measured and checked on (shapes and recipes only).

The shapes follow the page "SkyRL extends GLM-5.3-Flash training context to 1 million
tokens": one pooled key per 4 tokens and about 2048 selected keys per query (section "Model
and bottleneck"); query-chunked indexer scoring, an indexer sharded over tensor-parallel
ranks and DeepSeek-V3.2-shaped sparse-attention tensors, i.e. a 576-wide latent KV row whose
first 512 columns are the value (section "Four optimizations", item 1).  The pages train on
real books and a genome at 128k-1M tokens; seeded synthetic tensors of the same shapes
stand in for them (no dataset or weights are used).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    n_pools: int
    # indexer
    h_i: int
    d_i: int
    index_dtype: str  # "bf16" or "fp8" (OCP e4m3)
    int_range: int  # indexer q/k entries are integers drawn uniformly from [-r, r]
    w_period: int  # head weight w_j = 2^-(j mod w_period)
    topk: int
    # attention (heads == 0: indexer + top-k only)
    heads: int = 0
    d_qk: int = 0
    d_v: int = 0
    scale: float = 0.0
    chunk: int = 0
    attn_out: str = "fp32"  # dtype of the attention output O ("fp32" or "bf16")
    phases: tuple = field(default=("indexer", "topk", "attn_fwd"))
    description: str = ""

    @property
    def kv_aliased(self) -> bool:
        return True


def _s(d):
    return 1.0 / math.sqrt(d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_4k",
            n_tokens=4096, n_pools=1024, h_i=4, d_i=64, index_dtype="bf16", int_range=4,
            w_period=4, topk=256, heads=8, d_qk=128, d_v=128, scale=_s(128), chunk=4096,
            phases=("indexer", "topk", "attn_fwd", "attn_bwd"),
            description="Tiny DSA layer, 4096 tokens, 1024 pools, 4x64 indexer, top-256, "
                        "8 heads of 128"),
        Workload(
            name="fwd_128k",
            n_tokens=131072, n_pools=32768, h_i=32, d_i=128, index_dtype="bf16", int_range=4,
            w_period=4, topk=2048, heads=64, d_qk=576, d_v=512, scale=_s(576), chunk=8192,
            attn_out="bf16",
            description="DSA forward at 128k tokens: 32x128 bf16 indexer, top-2048, 64-head "
                        "sparse MQA over 576/512 latent rows, chunk 8192; O in bf16"),
        Workload(
            name="index_topk_256k_fp8",
            n_tokens=262144, n_pools=65536, h_i=32, d_i=128, index_dtype="fp8", int_range=8,
            w_period=4, topk=2048, chunk=16384, phases=("indexer", "topk"),
            description="Indexer + top-k at 256k tokens, 32x128 fp8-e4m3 indexer, top-2048, "
                        "chunk 16384"),
        Workload(
            name="fwd_bwd_64k",
            n_tokens=65536, n_pools=16384, h_i=32, d_i=128, index_dtype="bf16", int_range=4,
            w_period=4, topk=2048, heads=64, d_qk=576, d_v=512, scale=_s(576), chunk=8192,
            phases=("indexer", "topk", "attn_fwd", "attn_bwd"),
            description="Sparse attention forward + backward at 64k tokens, indices from the "
                        "128k-rule indexer, 64 heads over 576/512 latent rows"),
        Workload(
            name="nope_16k",
            n_tokens=16384, n_pools=4096, h_i=8, d_i=64, index_dtype="bf16", int_range=4,
            w_period=4, topk=2051, heads=16, d_qk=512, d_v=512, scale=_s(512), chunk=4096,
            phases=("indexer", "topk", "attn_fwd", "attn_bwd"),
            description="Flash-native shapes, small: top-2051 (not a multiple of the 32-key "
                        "tile), 16 heads over 512-wide NoPE latent rows (V = the whole row), "
                        "chunk 4096"),
        Workload(
            name="flash_nope_128k",
            n_tokens=131072, n_pools=32768, h_i=32, d_i=128, index_dtype="bf16", int_range=4,
            w_period=4, topk=2051, heads=64, d_qk=512, d_v=512, scale=_s(512), chunk=8192,
            attn_out="bf16",
            description="DSA forward at 128k with Flash-native shapes: top-2051 and 64-head "
                        "sparse MQA over 512-wide NoPE latent rows (no padding to 576/512); "
                        "O in bf16"),
        Workload(
            name="tp_share_1m",
            n_tokens=1048576, n_pools=262144, h_i=8, d_i=128, index_dtype="bf16", int_range=4,
            w_period=4, topk=2048, heads=64, d_qk=576, d_v=512, scale=_s(576), chunk=16384,
            attn_out="bf16",
            description="One tensor-parallel rank's share of a 1M-token DSA layer: 8 of 32 "
                        "indexer heads, top-2048, 64-head sparse MQA, chunk 16384; O in bf16 "
                        "(69 GB; fp32 would be 137 GB next to the 77 GB of queries)"),
    ]
}


def visible_count_total(n_tokens: int, n_pools: int) -> int:
    """Number of (query, visible pool) pairs, by a closed form when n_tokens == 4 * n_pools."""
    if n_tokens == 4 * n_pools:
        return 2 * n_pools * n_pools - n_pools
    return sum(min(n_pools, (t + 1) // 4) for t in range(n_tokens))


def valid_slot_total(n_tokens: int, n_pools: int, k: int) -> int:
    """Sum over queries of min(k, V(t)): the number of non-empty top-k slots."""
    full = max(0, n_tokens - (4 * k - 1))  # rows t >= 4k-1 see at least k pools (when P >= k)
    if n_pools >= k and n_tokens >= 4 * k - 1:
        # rows below 4k-1: V(t) = floor((t+1)/4) < k ; sum_{t<4k-1} floor((t+1)/4) = 2k(k-1)
        return 2 * k * (k - 1) + full * k
    return sum(min(k, n_pools, (t + 1) // 4) for t in range(n_tokens))
