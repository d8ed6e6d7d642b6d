"""The Python binding's own workspaces are safe when the kernels run on a side stream: a
workspace the caller did not pass is allocated on the current stream and freed when the call
returns, while the kernels may still be running on the given stream; the next allocation on
the current stream must not receive that memory before they finish."""

import pytest
import torch

from long_context_sparse_index_amd import binding as B
from long_context_sparse_index_amd import inputs as I
from long_context_sparse_index_amd import workloads as W

from gpu_util import say

pytestmark = pytest.mark.gpu
TINY = W.WORKLOADS["tiny_4k"]


def _forward(gpu, q_i, k_i, w, q, kv, stream=None, ws=None):
    n = TINY.n_tokens
    o = torch.empty((n, TINY.heads, TINY.d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((n, TINY.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, TINY.topk), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=TINY.topk, chunk=512, scale=TINY.scale,
                      d_v=TINY.d_v, idx_out=idx, ws=ws, stream=stream)
    return o, lse, idx


def test_side_stream_forward_and_backward_without_workspace(gpu):
    say("case: binding-allocated workspaces with kernels on a side stream (tiny_4k)")
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    q, kv, _ = I.attn_inputs(TINY, gpu)
    d_o = I.grad_output(TINY, gpu)
    ref_o, ref_lse, ref_idx = _forward(gpu, q_i, k_i, w, q, kv)
    ref_dq = torch.empty(q.shape, dtype=torch.float32, device=gpu)
    ref_dkv = torch.zeros((TINY.n_pools, TINY.d_qk), dtype=torch.float32, device=gpu)
    B.sparse_attn_bwd_deterministic(q, kv, ref_idx, ref_o, ref_lse, d_o, ref_dq, ref_dkv,
                                    scale=TINY.scale, d_v=TINY.d_v)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    for _ in range(3):
        dq = torch.empty_like(ref_dq)
        dkv = torch.zeros_like(ref_dkv)
        torch.cuda.synchronize()
        side.wait_stream(torch.cuda.current_stream())
        o, lse, idx = _forward(gpu, q_i, k_i, w, q, kv, stream=side)
        need = B.forward_chunked_workspace_bytes(TINY.n_pools, 512, TINY.topk)
        # same-size allocations on the current stream, written at once
        junk = [torch.full((need,), 0xFF, dtype=torch.uint8, device=gpu) for _ in range(2)]
        B.sparse_attn_bwd_deterministic(q, kv, idx, o, lse, d_o, dq, dkv, scale=TINY.scale,
                                        d_v=TINY.d_v, stream=side)
        need_b = B.sparse_attn_bwd_deterministic_workspace_bytes(
            TINY.n_tokens, TINY.heads, TINY.n_pools, TINY.topk, TINY.d_qk, TINY.d_v, False)
        junk += [torch.full((need_b,), 0x7F, dtype=torch.uint8, device=gpu) for _ in range(2)]
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(o.view(torch.int32), ref_o.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        assert torch.equal(dq.view(torch.int32), ref_dq.view(torch.int32))
        assert torch.equal(dkv.view(torch.int32), ref_dkv.view(torch.int32))
        del junk
