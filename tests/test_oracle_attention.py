"""Pins of the CPU oracle's sparse MQA attention, forward and backward (CPU only).

Attention reads only the selected pooled KV rows of each query (page "SkyRL extends
GLM-5.3-Flash training context to 1 million tokens", section "Model and bottleneck"), on
DeepSeek-V3.2-shaped tensors where all query heads share one latent KV row (section "Four
optimizations", item 1).  The pins: dense causal attention written with library softmax /
logsumexp, torch autograd, central finite differences, and exact identities.
"""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle


def _bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16_round(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _dense_causal(q, kv, v, rows, scale, d_v):
    """Dense attention of each listed row over all its visible pools (library softmax)."""
    n, h, d = q.shape
    p = kv.shape[0]
    vals = v if v is not None else kv[:, :d_v]
    o = np.zeros((n, h, d_v))
    lse = np.full((n, h), -np.inf)
    for r, t in enumerate(rows):
        vis = min(p, (t + 1) // 4)
        if vis == 0:
            continue
        logits = scale * q[r] @ kv[:vis, :d].T  # [h, vis]
        o[r] = softmax(logits, axis=1) @ vals[:vis]
        lse[r] = logsumexp(logits, axis=1)
    return o, lse


@pytest.mark.parametrize("separate_v", [False, True])
def test_full_selection_equals_dense_causal_attention(separate_v):
    rng = np.random.default_rng(20)
    p, h, d, d_v, k = 24, 3, 16, 12, 32  # k >= every V(t)
    rows = np.array([0, 2, 3, 5, 9, 40, 95, 96, 200])
    q = _bf16_round(rng.normal(size=(len(rows), h, d)))
    kv = _bf16_round(rng.normal(size=(p, d)))
    v = _bf16_round(rng.normal(size=(p, d_v))) if separate_v else None
    scores = rng.normal(size=(len(rows), p)).astype(np.float32)
    idx = oracle.topk(scores, rows, p, k)  # every visible pool, in some order
    o, lse = oracle.sparse_attn_fwd(_bits(q), _bits(kv), idx, 0.3,
                                    v_bits=None if v is None else _bits(v), d_v=d_v)
    ro, rl = _dense_causal(q, kv, v, rows, 0.3, d_v)
    assert np.allclose(o, ro, rtol=0, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], rl[fin], rtol=0, atol=1e-12)
    assert np.all(o[~fin] == 0.0) and np.all(np.isneginf(lse[~fin]))


def test_single_visible_pool_rows():
    rng = np.random.default_rng(21)
    p, h, d = 8, 4, 32
    rows = np.array([3, 4, 5, 6])
    q = _bf16_round(rng.normal(size=(4, h, d)))
    kv = _bf16_round(rng.normal(size=(p, d)))
    idx = np.full((4, 5), -1, np.int32)
    idx[:, 2] = 0
    o, lse = oracle.sparse_attn_fwd(_bits(q), _bits(kv), idx, 0.125)
    assert np.array_equal(o, np.broadcast_to(kv[0], o.shape))
    assert np.allclose(lse, 0.125 * q @ kv[0], rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_selected_values():
    rng = np.random.default_rng(22)
    p, h, d, k = 30, 2, 8, 6
    kv = _bf16_round(rng.normal(size=(p, d)))
    idx = np.array([[4, 9, -1, 0, 29, -1], [-1, -1, -1, -1, -1, 3]], np.int32)
    q = np.zeros((2, h, d))
    o, lse = oracle.sparse_attn_fwd(_bits(q), _bits(kv), idx, 1.0)
    assert np.allclose(o[0], kv[[4, 9, 0, 29]].mean(0), atol=1e-14)
    assert np.allclose(o[1], kv[3], atol=0)
    assert np.allclose(lse[0], np.log(4)) and np.allclose(lse[1], 0.0)


def test_slot_order_and_empty_slot_positions_do_not_matter():
    rng = np.random.default_rng(23)
    p, h, d, k = 50, 3, 16, 10
    q = _bits(rng.normal(size=(2, h, d)))
    kv = _bits(rng.normal(size=(p, d)))
    idx = np.array([[3, 7, 11, 20, 49, 0, -1, -1, -1, -1]] * 2, np.int32)
    o1, l1 = oracle.sparse_attn_fwd(q, kv, idx, 0.2)
    idx2 = idx.copy()
    idx2[0] = [-1, 49, 11, -1, 0, 3, -1, 7, 20, -1]
    idx2[1] = [20, -1, -1, -1, -1, 0, 49, 11, 7, 3]
    o2, l2 = oracle.sparse_attn_fwd(q, kv, idx2, 0.2)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_out_of_range_index_is_rejected():
    q = _bits(np.zeros((1, 1, 4)))
    kv = _bits(np.zeros((3, 4)))
    with pytest.raises(ValueError):
        oracle.sparse_attn_fwd(q, kv, np.array([[0, 3]], np.int32), 1.0)


# ----------------------------------------------------------------------------- backward


def _case(seed, separate_v, n=4, h=3, d=10, d_v=6, p=9, k=5):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(n, h, d))
    kv = rng.normal(size=(p, d))
    v = rng.normal(size=(p, d_v)) if separate_v else None
    idx = np.array([rng.permutation(p)[:k] for _ in range(n)], np.int32)
    idx[0, 1] = -1
    idx[1, :] = -1
    idx[1, 3] = 2  # a row with one valid slot
    idx[2, 0] = idx[2, 4] = -1
    do = rng.normal(size=(n, h, d_v))
    return q, kv, v, idx, do, d_v


def _loss(q, kv, v, idx, do, d_v, scale):
    o, _ = oracle.sparse_attn_fwd(q, kv, idx, scale, v_bits=v, d_v=d_v)
    return float((o * do).sum())


@pytest.mark.parametrize("separate_v", [False, True])
def test_backward_matches_central_differences(separate_v):
    q, kv, v, idx, do, d_v = _case(30, separate_v)
    scale = 0.37
    dq, dk, dv = oracle.sparse_attn_bwd(q, kv, idx, do, scale, v_bits=v, d_v=d_v)
    eps = 1e-5

    def fd(arr, pos):
        a0 = arr[pos]
        arr[pos] = a0 + eps
        up = _loss(q, kv, v, idx, do, d_v, scale)
        arr[pos] = a0 - eps
        dn = _loss(q, kv, v, idx, do, d_v, scale)
        arr[pos] = a0
        return (up - dn) / (2 * eps)

    rng = np.random.default_rng(31)
    for _ in range(25):
        pos = tuple(int(rng.integers(0, s)) for s in q.shape)
        assert abs(fd(q, pos) - dq[pos]) < 1e-7 * max(1.0, abs(dq[pos]))
        pos = tuple(int(rng.integers(0, s)) for s in kv.shape)
        assert abs(fd(kv, pos) - dk[pos]) < 1e-7 * max(1.0, abs(dk[pos]))
        if v is not None:
            pos = tuple(int(rng.integers(0, s)) for s in v.shape)
            assert abs(fd(v, pos) - dv[pos]) < 1e-7 * max(1.0, abs(dv[pos]))


def _torch_masked_attention(q, kv, v, idx, scale, d_v):
    """Independent formulation: gather + masked torch.softmax, differentiated by autograd."""
    qt = torch.tensor(q, requires_grad=True)
    kvt = torch.tensor(kv, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True) if v is not None else None
    it = torch.tensor(idx.astype(np.int64))
    valid = it >= 0
    g = it.clamp(min=0)
    keys = kvt[g]  # [n, k, d]
    vals = (vt if vt is not None else kvt[:, :d_v])[g]
    logits = scale * torch.einsum("nhd,nkd->nhk", qt, keys)
    logits = logits.masked_fill(~valid[:, None, :], float("-inf"))
    has = valid.any(dim=1)
    prob = torch.softmax(torch.where(has[:, None, None], logits, torch.zeros_like(logits)), -1)
    prob = prob * has[:, None, None]
    out = torch.einsum("nhk,nke->nhe", prob, vals)
    return qt, kvt, vt, out


@pytest.mark.parametrize("separate_v", [False, True])
def test_backward_matches_torch_autograd(separate_v):
    q, kv, v, idx, do, d_v = _case(32, separate_v, n=6, h=4, d=24, d_v=16, p=40, k=12)
    scale = 0.2
    dq, dk, dv = oracle.sparse_attn_bwd(q, kv, idx, do, scale, v_bits=v, d_v=d_v)
    o, _ = oracle.sparse_attn_fwd(q, kv, idx, scale, v_bits=v, d_v=d_v)
    qt, kvt, vt, out = _torch_masked_attention(q, kv, v, idx, scale, d_v)
    assert np.allclose(out.detach().numpy(), o, atol=1e-12)
    (out * torch.tensor(do)).sum().backward()
    assert np.allclose(qt.grad.numpy(), dq, atol=1e-12)
    assert np.allclose(kvt.grad.numpy(), dk, atol=1e-12)
    if v is not None:
        assert np.allclose(vt.grad.numpy(), dv, atol=1e-12)


def test_backward_identities():
    q, kv, v, idx, do, d_v = _case(33, True, n=8, h=5, d=12, d_v=7, p=30, k=9)
    dq, dk, dv = oracle.sparse_attn_bwd(q, kv, idx, do, 0.5, v_bits=v, d_v=d_v)
    has = (idx >= 0).any(axis=1)
    # softmax weights sum to one: the V gradient sums to the summed dO of non-empty rows
    assert np.allclose(dv.sum(0), do[has].sum(axis=(0, 1)), atol=1e-12)
    # the logit gradients of a row sum to zero: so do the key gradients
    assert np.allclose(dk.sum(0), 0.0, atol=1e-12)
    # a row with one valid slot has a constant softmax: no query gradient
    assert np.allclose(dq[1], 0.0, atol=0)


def test_aliased_value_gradient_folds_into_key_gradient():
    q, kv, _, idx, do, d_v = _case(34, False, d=10, d_v=6)
    dq_a, dk_a, dv_a = oracle.sparse_attn_bwd(q, kv, idx, do, 0.3, d_v=d_v)
    dq_s, dk_s, dv_s = oracle.sparse_attn_bwd(q, kv, idx, do, 0.3, v_bits=kv[:, :d_v].copy(),
                                              d_v=d_v)
    assert dv_a is None
    assert np.allclose(dq_a, dq_s, atol=1e-13)
    assert np.allclose(dk_a[:, :d_v], dk_s[:, :d_v] + dv_s, atol=1e-13)
    assert np.allclose(dk_a[:, d_v:], dk_s[:, d_v:], atol=1e-13)


def test_only_listed_rows_contribute():
    q, kv, v, idx, do, d_v = _case(35, True, n=6)
    _, dk, dv = oracle.sparse_attn_bwd(q, kv, idx, do, 0.3, v_bits=v, d_v=d_v)
    a, b = [0, 2, 5], [1, 3, 4]
    _, dk_a, dv_a = oracle.sparse_attn_bwd(q[a], kv, idx[a], do[a], 0.3, v_bits=v, d_v=d_v)
    _, dk_b, dv_b = oracle.sparse_attn_bwd(q[b], kv, idx[b], do[b], 0.3, v_bits=v, d_v=d_v)
    assert np.allclose(dk, dk_a + dk_b, atol=1e-13)
    assert np.allclose(dv, dv_a + dv_b, atol=1e-13)


def test_bf16_entry_point_decodes_like_the_double_one():
    q, kv, v, idx, do, d_v = _case(36, True)
    qb, kvb, vb, dob = (_bits(x) for x in (q, kv, v, do))
    o1, l1 = oracle.sparse_attn_fwd(qb, kvb, idx, 0.3, v_bits=vb, d_v=d_v)
    o2, l2 = oracle.sparse_attn_fwd(*(_bf16_round(x) for x in (q, kv)), idx, 0.3,
                                    v_bits=_bf16_round(v), d_v=d_v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    g1 = oracle.sparse_attn_bwd(qb, kvb, idx, dob, 0.3, v_bits=vb, d_v=d_v)
    g2 = oracle.sparse_attn_bwd(*(_bf16_round(x) for x in (q, kv)), idx, _bf16_round(do), 0.3,
                                v_bits=_bf16_round(v), d_v=d_v)
    for x, y in zip(g1, g2):
        assert np.array_equal(x, y)
