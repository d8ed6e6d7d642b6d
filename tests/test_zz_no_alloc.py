"""dsa_sparse_attn_bwd_noalloc (static scratch, allocates nothing) against dsa_sparse_attn_bwd
(workspace argument), through the C ABI, on consecutive calls that share the library's static
array: the largest size it accepts, then smaller calls of other shapes.  dQ does not depend on
the order of any atomic and must be bit-identical; dK/dV (fp32 atomics in both) within the
backward's tolerance."""

import pytest
import torch

from long_context_sparse_index_amd import binding as B

from gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def _case(gpu, nq, p, h, d_qk, d_v, k, seed, separate_v=False):
    g = torch.Generator(device=gpu).manual_seed(seed)
    q = torch.randn((nq, h, d_qk), generator=g, device=gpu).to(torch.bfloat16)
    kv = torch.randn((p, d_qk), generator=g, device=gpu).to(torch.bfloat16)
    v = torch.randn((p, d_v), generator=g, device=gpu).to(torch.bfloat16) if separate_v else None
    d_o = torch.randn((nq, h, d_v), generator=g, device=gpu).to(torch.bfloat16)
    # k distinct pools per row, some slots empty, a few rows with no valid slot
    idx = torch.rand((nq, p), generator=g, device=gpu).argsort(dim=1)[:, :k].to(torch.int32)
    drop = torch.rand((nq, k), generator=g, device=gpu) < 0.1
    idx = torch.where(drop, torch.full_like(idx, -1), idx).contiguous()
    idx[: min(3, nq)] = -1
    o = torch.empty((nq, h, d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((nq, h), dtype=torch.float32, device=gpu)
    scale = d_qk ** -0.5
    B.sparse_attn_fwd(q, kv, idx, o, lse, scale=scale, d_v=d_v, v=v)
    return q, kv, v, d_o, idx, o, lse, scale


@pytest.mark.parametrize("stream_kind", ["current", "side"])
def test_noalloc_backward_matches_workspace_backward(gpu, stream_kind):
    cases = [  # (nq, p, h, d_qk, d_v, k, separate_v): the first at the 2^22-delta limit
        (65536, 300, 64, 128, 128, 48, False),
        (4096, 1024, 8, 128, 128, 256, True),
        (777, 500, 64, 576, 512, 130, False),
    ]
    stream = torch.cuda.Stream() if stream_kind == "side" else None
    for i, (nq, p, h, d_qk, d_v, k, sep) in enumerate(cases):
        say("case: bwd_noalloc call %d (%s stream): nq=%d p=%d h=%d %d/%d k=%d separate_v=%s"
            % (i, stream_kind, nq, p, h, d_qk, d_v, k, sep))
        q, kv, v, d_o, idx, o, lse, scale = _case(gpu, nq, p, h, d_qk, d_v, k, seed=100 + i,
                                                  separate_v=sep)
        dq_ref = torch.empty(q.shape, dtype=torch.float32, device=gpu)
        dkv_ref = torch.zeros((p, d_qk), dtype=torch.float32, device=gpu)
        dv_ref = torch.zeros((p, d_v), dtype=torch.float32, device=gpu) if sep else None
        B.sparse_attn_bwd(q, kv, idx, o, lse, d_o, dq_ref, dkv_ref, scale=scale, d_v=d_v, v=v,
                          dv=dv_ref)
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=gpu)
        dkv = torch.zeros((p, d_qk), dtype=torch.float32, device=gpu)
        dv = torch.zeros((p, d_v), dtype=torch.float32, device=gpu) if sep else None
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        B.sparse_attn_bwd_noalloc(q, kv, idx, o, lse, d_o, dq, dkv, scale=scale, d_v=d_v, v=v,
                                  dv=dv, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(dq.view(torch.int32), dq_ref.view(torch.int32)), "dq differs"
        assert_close(dkv.cpu().numpy(), dkv_ref.cpu().numpy(), "dKV")
        if sep:
            assert_close(dv.cpu().numpy(), dv_ref.cpu().numpy(), "dV")
    # one row past the limit is refused, nothing launched
    big = 65537
    with pytest.raises(B.DSAError):
        q = torch.empty((big, 64, 128), dtype=torch.bfloat16, device=gpu)
        idx = torch.full((big, 8), -1, dtype=torch.int32, device=gpu)
        o = torch.empty((big, 64, 128), dtype=torch.float32, device=gpu)
        lse = torch.empty((big, 64), dtype=torch.float32, device=gpu)
        kv = torch.empty((16, 128), dtype=torch.bfloat16, device=gpu)
        B.sparse_attn_bwd_noalloc(q, kv, idx, o, lse, q, o, torch.empty_like(kv, dtype=torch.float32),
                                  scale=0.1, d_v=128)
