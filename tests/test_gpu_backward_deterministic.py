"""GPU tests of the deterministic backward (dsa_sparse_attn_bwd_deterministic): gradients
within the backward's tolerance of the CPU oracle, bit-identical across repeated calls (no
atomics: every pool's staged dK/dV rows are summed in row-major order after a stable sort by
pool), and within tolerance of the fp32-atomic backward."""

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_index_amd import binding as B
from long_context_sparse_index_amd import inputs as I
from long_context_sparse_index_amd import workloads as W

from gpu_util import assert_close, host_bits, say

pytestmark = pytest.mark.gpu
TINY = W.WORKLOADS["tiny_4k"]


def _bwd(det, q, kv, idx, o, lse, d_o, scale, d_v, v=None, separate_dv=False):
    n_pools, d_qk = kv.shape[0], q.shape[2]
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dkv = torch.zeros((n_pools, d_qk), dtype=torch.float32, device=q.device)
    dv = torch.zeros((n_pools, d_v), dtype=torch.float32, device=q.device) \
        if (v is not None or separate_dv) else None
    f = B.sparse_attn_bwd_deterministic if det else B.sparse_attn_bwd
    f(q, kv, idx, o, lse, d_o, dq, dkv, scale=scale, d_v=d_v, v=v, dv=dv)
    torch.cuda.synchronize()
    return dq, dkv, dv


def _same_bits(a, b):
    return a is None and b is None or torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("separate_v", [False, True])
def test_deterministic_backward_tiny(gpu, separate_v):
    say("case: deterministic backward tiny_4k separate_v=%s" % separate_v)
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    idx = B.topk_new(B.index_scores_new(q_i, k_i, w), q_start=0, n_pools=TINY.n_pools,
                     k=TINY.topk)
    q, kv, v = I.attn_inputs(TINY, gpu, separate_v=separate_v)
    d_o = I.grad_output(TINY, gpu)
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=TINY.scale, d_v=TINY.d_v, v=v)
    first = _bwd(True, q, kv, idx, o, lse, d_o, TINY.scale, TINY.d_v, v=v)
    for _ in range(2):
        again = _bwd(True, q, kv, idx, o, lse, d_o, TINY.scale, TINY.d_v, v=v)
        assert all(_same_bits(a, b) for a, b in zip(first, again)), "not reproducible"
    dq, dkv, dv = first
    rq, rk, rv = oracle.sparse_attn_bwd(host_bits(q), host_bits(kv), idx.cpu().numpy(),
                                        host_bits(d_o), TINY.scale,
                                        v_bits=None if v is None else host_bits(v),
                                        d_v=TINY.d_v)
    assert_close(dq.cpu().numpy(), rq, "dQ")
    assert_close(dkv.cpu().numpy(), rk, "dK" if separate_v else "dKV (aliased V folded)")
    if separate_v:
        assert_close(dv.cpu().numpy(), rv, "dV")


@pytest.mark.parametrize("d_qk,d_v,h", [(576, 512, 64), (512, 512, 24)])
def test_deterministic_backward_random_selection(gpu, d_qk, d_v, h):
    say("case: deterministic backward %d/%d h=%d random idx" % (d_qk, d_v, h))
    nq, p, k = 48, 3000, 2048
    g = torch.Generator(device=gpu).manual_seed(7 * h + d_qk)
    q = torch.randn((nq, h, d_qk), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, d_qk), generator=g, device=gpu, dtype=torch.bfloat16)
    d_o = torch.randn((nq, h, d_v), generator=g, device=gpu, dtype=torch.bfloat16)
    idx = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = idx.to(torch.int32).contiguous()
    idx[torch.rand((nq, k), generator=g, device=gpu) < 0.1] = -1
    idx[0] = -1
    scale = 1.0 / float(np.sqrt(d_qk))
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=d_v)
    sep = d_qk == d_v  # NoPE rows: dV into its own buffer
    a = _bwd(True, q, kv, idx, o, lse, d_o, scale, d_v, separate_dv=sep)
    b = _bwd(True, q, kv, idx, o, lse, d_o, scale, d_v, separate_dv=sep)
    assert all(_same_bits(x, y) for x, y in zip(a, b)), "not reproducible"
    at = _bwd(False, q, kv, idx, o, lse, d_o, scale, d_v, separate_dv=sep)
    assert_close(a[1].cpu().numpy(), at[1].cpu().numpy(), "dKV vs fp32 atomics")
    assert _same_bits(a[0], at[0])  # dQ does not go through the dK/dV accumulators
    kv_h = host_bits(kv)
    rq, rk, rv = oracle.sparse_attn_bwd(host_bits(q), kv_h, idx.cpu().numpy(), host_bits(d_o),
                                        scale, v_bits=kv_h[:, :d_v].copy() if sep else None,
                                        d_v=d_v)
    assert_close(a[1].cpu().numpy(), rk, "dK" if sep else "dKV")
    if sep:
        assert_close(a[2].cpu().numpy(), rv, "dV")


def test_deterministic_backward_accumulates_and_rejects(gpu):
    """dkv is accumulated (a running sum is kept); a short workspace is an error."""
    say("case: deterministic backward accumulation and workspace errors")
    nq, p, k, h, d = 16, 500, 256, 8, 128
    g = torch.Generator(device=gpu).manual_seed(3)
    q = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16)
    d_o = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    idx = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = idx.to(torch.int32).contiguous()
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=0.1, d_v=d)
    dq = torch.empty(q.shape, dtype=torch.float32, device=gpu)
    once = torch.zeros((p, d), dtype=torch.float32, device=gpu)
    B.sparse_attn_bwd_deterministic(q, kv, idx, o, lse, d_o, dq, once, scale=0.1, d_v=d)
    twice = once.clone()
    B.sparse_attn_bwd_deterministic(q, kv, idx, o, lse, d_o, dq, twice, scale=0.1, d_v=d)
    torch.cuda.synchronize()
    assert torch.equal(twice, once + once)  # x + x is exact in fp32
    small = torch.empty(256, dtype=torch.uint8, device=gpu)
    with pytest.raises(B.DSAError) as e:
        B.sparse_attn_bwd_deterministic(q, kv, idx, o, lse, d_o, dq, once, scale=0.1, d_v=d,
                                        ws=small)
    assert e.value.status == 3


def test_deterministic_backward_full_size_64k(gpu):
    """fwd_bwd_64k: reproducible to the bit over the whole sequence, within tolerance of the
    fp32-atomic backward, and the exact gradient-sum identity on dV."""
    wl = W.WORKLOADS["fwd_bwd_64k"]
    n, p, k = wl.n_tokens, wl.n_pools, wl.topk
    say("case: deterministic backward fwd_bwd_64k full size (N=%d, P=%d)" % (n, p))
    q_i, k_i, w = I.index_inputs(wl, gpu)
    q, kv, _ = I.attn_inputs(wl, gpu)
    d_o = I.grad_output(wl, gpu)
    o = torch.empty((n, wl.heads, wl.d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((n, wl.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, k), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=k, chunk=wl.chunk, scale=wl.scale,
                      d_v=wl.d_v, idx_out=idx)
    a = _bwd(True, q, kv, idx, o, lse, d_o, wl.scale, wl.d_v, separate_dv=True)
    b = _bwd(True, q, kv, idx, o, lse, d_o, wl.scale, wl.d_v, separate_dv=True)
    assert all(_same_bits(x, y) for x, y in zip(a, b)), "not reproducible"
    say("  two runs bit-identical")
    at = _bwd(False, q, kv, idx, o, lse, d_o, wl.scale, wl.d_v, separate_dv=True)
    assert_close(a[1].cpu().numpy(), at[1].cpu().numpy(), "dK vs fp32 atomics")
    assert_close(a[2].cpu().numpy(), at[2].cpu().numpy(), "dV vs fp32 atomics")
    has = (idx >= 0).any(dim=1)
    sum_do = d_o.float()[has].sum(dim=(0, 1)).double()
    scale_do = d_o.float()[has].abs().sum(dim=(0, 1)).double()
    assert float(((a[2].double().sum(0) - sum_do).abs() / scale_do).max()) < 1e-4


def test_deterministic_backward_two_chunks_repeats_and_junk(gpu):
    """5000 query rows (two chunks of the staged reduction: 4096 + 904), selections with
    repeated pools in a row, -1 anywhere and out-of-range values (skipped like -1): bit-identical
    across calls, dQ bit-identical to the atomic backward, and dK / dV within tolerance of the
    oracle (given the same selection with the out-of-range values as -1)."""
    say("case: deterministic backward two chunks, repeated pools and junk slots")
    nq, p, k, h, d = 5000, 700, 96, 8, 128
    g = torch.Generator(device=gpu).manual_seed(11)
    q = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16)
    v = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16)
    d_o = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    idx = torch.randint(0, p, (nq, k), generator=g, device=gpu, dtype=torch.int32)
    idx[:, 5] = idx[:, 2]  # a pool repeated in every row
    junk = torch.rand((nq, k), generator=g, device=gpu)
    idx[junk < 0.05] = -1
    idx[(junk >= 0.05) & (junk < 0.08)] = p + 3  # out of range: skipped like -1
    idx[(junk >= 0.08) & (junk < 0.09)] = -5
    idx[4100:4110] = -1  # rows without a valid slot in the second chunk
    idx = idx.contiguous()
    scale = 1.0 / float(np.sqrt(d))
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=d, v=v)
    a = _bwd(True, q, kv, idx, o, lse, d_o, scale, d, v=v)
    b = _bwd(True, q, kv, idx, o, lse, d_o, scale, d, v=v)
    assert all(_same_bits(x, y) for x, y in zip(a, b)), "not reproducible"
    at = _bwd(False, q, kv, idx, o, lse, d_o, scale, d, v=v)
    assert _same_bits(a[0], at[0])
    assert_close(a[1].cpu().numpy(), at[1].cpu().numpy(), "dK vs fp32 atomics")
    assert_close(a[2].cpu().numpy(), at[2].cpu().numpy(), "dV vs fp32 atomics")
    clean = idx.cpu().numpy().copy()
    clean[(clean < 0) | (clean >= p)] = -1
    rq, rk, rv = oracle.sparse_attn_bwd(host_bits(q), host_bits(kv), clean, host_bits(d_o),
                                        scale, v_bits=host_bits(v), d_v=d)
    assert_close(a[0].cpu().numpy(), rq, "dQ")
    assert_close(a[1].cpu().numpy(), rk, "dK")
    assert_close(a[2].cpu().numpy(), rv, "dV")
