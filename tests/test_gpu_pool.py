"""GPU parity of dsa_pool_keys (pooled key rows from per-token rows and gate scores) against
the CPU oracle, through the C ABI.  The GPU sums in fp32 and the oracle in double, each
rounding once to bf16, so a pooled value may land on the other side of a bf16 rounding
boundary when the exact value lies within the fp32 error of it: every value must be equal or
one bf16 step apart, and at least 99.9% of them bit-identical."""

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_index_amd import binding as B
from long_context_sparse_index_amd import inputs as I
from long_context_sparse_index_amd import workloads as W

from gpu_util import say

pytestmark = pytest.mark.gpu


def _compare(got_bits, ref_bits, what):
    g = got_bits.astype(np.int32)
    r = ref_bits.astype(np.int32)
    # bf16 patterns of one sign are ordered like their values: one step = one unit
    same_sign = (g >> 15) == (r >> 15)
    step = np.where(same_sign, np.abs(g - r), np.where((g & 0x7FFF) + (r & 0x7FFF) <= 1, 1, 99))
    exact = float(np.mean(step == 0)) if step.size else 1.0
    say("  %s: %d values, %.5f%% bit-identical, max %d step(s)" % (what, step.size, 100 * exact,
                                                                  step.max(initial=0)))
    assert step.max(initial=0) <= 1 and exact >= 0.999


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,d,pad_x,pad_out", [(4099, 128, 0, 0), (4096, 576, 64, 8),
                                               (1001, 64, 8, 0), (12, 8, 0, 8)])
def test_pool_keys_matches_oracle(gpu, n, d, pad_x, pad_out):
    say("case: pool_keys n=%d d=%d pad_x=%d pad_out=%d" % (n, d, pad_x, pad_out))
    g = torch.Generator(device=gpu).manual_seed(n + d)
    xw = torch.randn((n, d + pad_x), generator=g, device=gpu).to(torch.bfloat16)
    gate = (2.0 * torch.randn((n,), generator=g, device=gpu)).float().contiguous()
    x = xw[:, :d]
    p = n // 4
    outw = torch.full((p, d + pad_out), float("nan"), dtype=torch.bfloat16, device=gpu)
    out = outw[:, :d]
    B.pool_keys(x, gate, out)
    torch.cuda.synchronize()
    _, ref = oracle.pool_keys(_bits(x), gate.cpu().numpy())
    _compare(_bits(out), ref, "pooled keys")
    if pad_out:
        assert bool(torch.isnan(outw[:, d:].float()).all())  # columns past d untouched


def test_pool_keys_edge_cases(gpu):
    say("case: pool_keys with fewer than 4 tokens, and bad arguments")
    x = torch.randn((3, 64), device=gpu).to(torch.bfloat16)
    gate = torch.zeros((3,), device=gpu)
    out = torch.empty((0, 64), dtype=torch.bfloat16, device=gpu)
    B.pool_keys(x, gate, out)  # no pool: nothing to do
    x8 = torch.randn((8, 60), device=gpu).to(torch.bfloat16)
    with pytest.raises(B.DSAError) as e:
        B.pool_keys(x8, torch.zeros((8,), device=gpu),
                    torch.empty((2, 60), dtype=torch.bfloat16, device=gpu))
    assert e.value.status == 2  # d not a multiple of 8
    torch.cuda.synchronize()


def test_pool_keys_full_size_1m_sampled(gpu):
    """The 1M-token latent KV rows (1048576 x 576 bf16) pooled in one call; sampled pools
    (first, last, around chunk boundaries, seeded uniform) against the oracle."""
    wl = W.WORKLOADS["tp_share_1m"]
    n, d = wl.n_tokens, wl.d_qk
    say("case: pool_keys full size n=%d d=%d" % (n, d))
    x = I.normal_bf16((n, d), 5, "kv", gpu)
    gate = I.normal_bf16((n,), 6, "q", gpu).float().contiguous()
    out = torch.empty((n // 4, d), dtype=torch.bfloat16, device=gpu)
    B.pool_keys(x, gate, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    pools = np.unique(np.concatenate([[0, 1, n // 4 - 1, 4095, 4096, 65535, 65536],
                                      rng.integers(0, n // 4, size=200)]))
    tok = (4 * pools[:, None] + np.arange(4)[None, :]).reshape(-1)
    tok_t = torch.from_numpy(tok).to(gpu)
    _, ref = oracle.pool_keys(_bits(x[tok_t]), gate[tok_t].cpu().numpy())
    _compare(_bits(out[torch.from_numpy(pools).to(gpu)]), ref, "sampled pools")
