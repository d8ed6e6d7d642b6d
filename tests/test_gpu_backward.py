"""GPU parity of the sparse-attention backward against the CPU oracle, through the C ABI.
Gradients must agree within max |err| <= 2e-2 RMS and mean |err| <= 2e-3 RMS per tensor."""

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


def _run_bwd(q, kv, idx, d_o, scale, d_v, v=None, separate_dv=False):
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=d_v, v=v)
    n_pools, d_qk = kv.shape[0], q.shape[2]
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dkv = torch.zeros((n_pools, d_qk), dtype=torch.float32, device=q.device)
    dv = torch.zeros((n_pools, d_v), dtype=torch.float32, device=q.device) \
        if (v is not None or separate_dv) else None
    B.sparse_attn_bwd(q, kv, idx, o, lse, d_o, dq, dkv, scale=scale, d_v=d_v, v=v, dv=dv)
    torch.cuda.synchronize()
    return dq, dkv, dv


@pytest.mark.parametrize("separate_v", [False, True])
def test_backward_tiny_full(gpu, separate_v):
    say("case: backward tiny_4k separate_v=%s" % separate_v)
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    idx = B.topk_new(B.index_scores_new(q_i, k_i, w), q_start=0, n_pools=TINY.n_pools,
                     k=TINY.topk)
    q, kv, v = I.attn_inputs(TINY, gpu, separate_v=separate_v)
    d_o = I.grad_output(TINY, gpu)
    dq, dkv, dv = _run_bwd(q, kv, idx, d_o, TINY.scale, TINY.d_v, v=v)
    rq, rk, rv = oracle.sparse_attn_bwd(host_bits(q), host_bits(kv), idx.cpu().numpy(),
                                        host_bits(d_o), TINY.scale,
                                        v_bits=None if v is None else host_bits(v),
                                        d_v=TINY.d_v)
    assert_close(dq.cpu().numpy(), rq, "dQ")
    assert_close(dkv.cpu().numpy(), rk, "dK" if separate_v else "dKV (aliased V folded)")
    if separate_v:
        assert_close(dv.cpu().numpy(), rv, "dV")
    assert np.all(dq[:3].cpu().numpy() == 0.0)  # rows without a visible pool


@pytest.mark.parametrize("h", [64, 24])
def test_backward_latent_576_random_selection(gpu, h):
    say("case: backward 576/512 random idx h=%d" % h)
    nq, p, k = 40, 3000, 2048
    g = torch.Generator(device=gpu).manual_seed(21 + h)
    q = torch.randn((nq, h, 576), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, 576), generator=g, device=gpu, dtype=torch.bfloat16)
    d_o = torch.randn((nq, h, 512), generator=g, device=gpu, dtype=torch.bfloat16)
    idx = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = idx.to(torch.int32).contiguous()
    idx[torch.rand((nq, k), generator=g, device=gpu) < 0.1] = -1
    idx[0] = -1
    idx[1, :] = -1
    idx[1, 7] = 11
    idx[2, 40:] = -1
    scale = 1.0 / 24.0
    dq, dkv, _ = _run_bwd(q, kv, idx, d_o, scale, 512)
    rq, rk, _ = oracle.sparse_attn_bwd(host_bits(q), host_bits(kv), idx.cpu().numpy(),
                                       host_bits(d_o), scale, d_v=512)
    assert_close(dq.cpu().numpy(), rq, "dQ")
    assert_close(dkv.cpu().numpy(), rk, "dKV")
    assert np.all(dq[0].cpu().numpy() == 0.0)  # no valid slot: nothing to differentiate
    # one valid slot: the softmax is constant, so dQ vanishes up to the fp32 rounding gap
    # between dP (MFMA summation order) and D = dO . O (|dP| ~ 20 here)
    assert np.abs(dq[1].cpu().numpy()).max() <= 1e-4 * float(np.sqrt(np.mean(rq * rq)))


@pytest.mark.parametrize("d", [256, 512])
def test_backward_nope_latent_rows(gpu, d):
    """NoPE latent rows (d_qk = d_v = d, V the whole row) with k = 2051."""
    say("case: backward NoPE %d/%d random idx" % (d, d))
    nq, p, k, h = 32, 3000, 2051, 64
    g = torch.Generator(device=gpu).manual_seed(41 + d)
    q = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16)
    d_o = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    idx = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = idx.to(torch.int32).contiguous()
    idx[torch.rand((nq, k), generator=g, device=gpu) < 0.1] = -1
    idx[0] = -1
    idx[2, 40:] = -1
    scale = 1.0 / float(np.sqrt(d))
    dq, dkv, dv = _run_bwd(q, kv, idx, d_o, scale, d, separate_dv=True)
    kv_h = host_bits(kv)
    rq, rk, rv = oracle.sparse_attn_bwd(host_bits(q), kv_h, idx.cpu().numpy(), host_bits(d_o),
                                        scale, v_bits=kv_h[:, :d].copy(), d_v=d)
    assert_close(dq.cpu().numpy(), rq, "dQ")
    assert_close(dkv.cpu().numpy(), rk, "dK")
    assert_close(dv.cpu().numpy(), rv, "dV")
    assert np.all(dq[0].cpu().numpy() == 0.0)


@pytest.mark.parametrize("name", ["fwd_bwd_64k", "nope_16k"])
def test_backward_full_size(gpu, name):
    wl = W.WORKLOADS[name]
    n, p, k = wl.n_tokens, wl.n_pools, wl.topk
    say("case: backward %s full size (N=%d, P=%d)" % (name, n, p))
    q_i, k_i, w = I.index_inputs(wl, gpu)
    q, kv, _ = I.attn_inputs(wl, gpu)
    d_o = I.grad_output(wl, gpu)
    o = torch.empty((n, wl.heads, wl.d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((n, wl.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, k), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=k, chunk=wl.chunk, scale=wl.scale,
                      d_v=wl.d_v, idx_out=idx)
    dq = torch.empty(q.shape, dtype=torch.float32, device=gpu)
    dk = torch.zeros((p, wl.d_qk), dtype=torch.float32, device=gpu)
    dv = torch.zeros((p, wl.d_v), dtype=torch.float32, device=gpu)
    B.sparse_attn_bwd(q, kv, idx, o, lse, d_o, dq, dk, scale=wl.scale, d_v=wl.d_v, dv=dv)
    torch.cuda.synchronize()
    say("  backward done")
    # exact identities over all rows: softmax weights sum to one, logit gradients to zero
    has = (idx >= 0).any(dim=1)
    sum_do = d_o.float()[has].sum(dim=(0, 1)).double()
    sum_dv = dv.double().sum(0)
    scale_do = d_o.float()[has].abs().sum(dim=(0, 1)).double()
    assert float(((sum_dv - sum_do).abs() / scale_do).max()) < 1e-4
    sum_dk = dk.double().sum(0)
    assert float((sum_dk.abs() / dk.double().abs().sum(0)).max()) < 1e-3
    say("  gradient-sum identities hold on all %d rows" % n)
    # sampled rows: dQ row by row
    rows = I.sample_rows(wl, n_uniform=12)
    rt = torch.from_numpy(rows).to(gpu)
    q_rows, do_rows, idx_rows = host_bits(q[rt]), host_bits(d_o[rt]), idx[rt].cpu().numpy()
    kv_h = host_bits(kv)
    rq, rk, rv = oracle.sparse_attn_bwd(q_rows, kv_h, idx_rows, do_rows, wl.scale,
                                        v_bits=kv_h[:, :wl.d_v].copy(), d_v=wl.d_v)
    assert_close(dq[rt].cpu().numpy(), rq, "dQ (sampled rows)")
    # dK / dV from the sampled rows alone: rerun with dO zero outside them
    d_o_m = torch.zeros_like(d_o)
    d_o_m[rt] = d_o[rt]
    dk.zero_()
    dv.zero_()
    B.sparse_attn_bwd(q, kv, idx, o, lse, d_o_m, dq, dk, scale=wl.scale, d_v=wl.d_v, dv=dv)
    torch.cuda.synchronize()
    assert_close(dk.cpu().numpy(), rk, "dK (masked dO)")
    assert_close(dv.cpu().numpy(), rv, "dV (masked dO)")
