"""Seeded synthetic inputs for the DSA workloads.

This module draws random tensors and picks sample rows; it holds none of the layer's
arithmetic.  The same tensors feed the HIP path and the CPU oracle.  Every tensor gets its
own torch.Generator seeded with seed * 1000 + tensor_id, on the device where it is made.
Recipes (the pages train on books and a genome; these stand in for them):
  * indexer q/k: integers drawn uniformly from [-r, r], stored exactly in bf16 or OCP e4m3;
  * indexer head weights: w_j = 2^-(j mod period), one vector shared by all queries;
  * attention q, latent kv and dO: bf16 draws from N(0, 1).
"""

from __future__ import annotations

import numpy as np
import torch

from .workloads import Workload

TENSOR_IDS = {"q_idx": 1, "k_idx": 2, "q": 3, "kv": 4, "v": 5, "d_o": 6, "rows": 7}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed * 1000 + TENSOR_IDS[name])
    return g


def int_tensor(shape, r: int, dtype: str, seed: int, name: str, device) -> torch.Tensor:
    """Integers uniform in [-r, r]; bf16 tensor, or uint8 tensor of OCP e4m3 bit patterns."""
    g = _gen(seed, name, device)
    x = torch.randint(-r, r + 1, shape, generator=g, device=device, dtype=torch.int8)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp8":
        return x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(dtype)


def normal_bf16(shape, seed: int, name: str, device) -> torch.Tensor:
    g = _gen(seed, name, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)


def head_weights(h_i: int, period: int, device="cpu") -> torch.Tensor:
    return torch.tensor([2.0 ** -(j % period) for j in range(h_i)], dtype=torch.float32,
                        device=device)


def index_inputs(wl: Workload, device, seed: int = 0, n_tokens: int | None = None):
    """(q_idx [N, h_i, d_i], k_idx [P, d_i], w [h_i])."""
    n = wl.n_tokens if n_tokens is None else n_tokens
    q = int_tensor((n, wl.h_i, wl.d_i), wl.int_range, wl.index_dtype, seed, "q_idx", device)
    k = int_tensor((wl.n_pools, wl.d_i), wl.int_range, wl.index_dtype, seed, "k_idx", device)
    return q, k, head_weights(wl.h_i, wl.w_period, device)


def attn_inputs(wl: Workload, device, seed: int = 0, separate_v: bool = False,
                n_tokens: int | None = None):
    """(q [N, H, d_qk], kv [P, d_qk], v [P, d_v] or None), bf16 N(0,1)."""
    n = wl.n_tokens if n_tokens is None else n_tokens
    q = normal_bf16((n, wl.heads, wl.d_qk), seed, "q", device)
    kv = normal_bf16((wl.n_pools, wl.d_qk), seed, "kv", device)
    v = normal_bf16((wl.n_pools, wl.d_v), seed, "v", device) if separate_v else None
    return q, kv, v


def grad_output(wl: Workload, device, seed: int = 0, n_tokens: int | None = None):
    n = wl.n_tokens if n_tokens is None else n_tokens
    return normal_bf16((n, wl.heads, wl.d_v), seed, "d_o", device)


def sample_rows(wl: Workload, n_uniform: int = 48, seed: int = 0) -> np.ndarray:
    """Query rows to check at sizes the oracle cannot finish in full: the empty and first
    visible rows, the rows around the top-k fill point 4k-1, three chunk boundaries, the
    last row, and seeded uniform rows.  Sorted, unique, int64."""
    n, k, c = wl.n_tokens, wl.topk, max(1, wl.chunk)
    fixed = [0, 1, 2, 3, 6, 7, 4 * k - 2, 4 * k - 1, 4 * k, n - 1]
    n_chunks = (n + c - 1) // c
    for ci in sorted({1, n_chunks // 2, n_chunks - 1}):
        t0 = ci * c
        fixed += [t0 - 1, t0, t0 + 1]
    g = np.random.default_rng(seed * 1000 + TENSOR_IDS["rows"])
    uni = g.integers(0, n, size=n_uniform).tolist()
    rows = sorted({int(t) for t in fixed + uni if 0 <= t < n})
    return np.asarray(rows, dtype=np.int64)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint8)


def index_bits(t: torch.Tensor) -> np.ndarray:
    return bits_u16(t) if t.dtype == torch.bfloat16 else bits_u8(t)
