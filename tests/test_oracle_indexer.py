"""Pins of the CPU oracle's indexer scores and its number decoders (CPU only).

Each check ties the oracle to something other than itself: a library conversion or matmul,
a hand-worked example, or an exact identity of the score's definition
(page "SkyRL extends GLM-5.3-Flash training context to 1 million tokens", section "Model and
bottleneck": every query scores every visible pooled key, one pool per 4 tokens).
"""

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_index_amd import workloads as W


def _bf16_bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _e4m3_bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _rand_int(rng, shape, r):
    return rng.integers(-r, r + 1, size=shape).astype(np.float32)


def test_decode_bf16_matches_torch_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])


def test_decode_e4m3_matches_torch_on_every_pattern():
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ours = oracle.decode_e4m3(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_visibility_closed_forms():
    p = 1024
    assert [oracle.visible(t, p) for t in range(8)] == [0, 0, 0, 1, 1, 1, 1, 2]
    for s in (0, 1, 17, 1023):  # pool s first becomes visible at t = 4s + 3
        assert oracle.visible(4 * s + 2, p) == s and oracle.visible(4 * s + 3, p) == s + 1
    assert oracle.visible(10 ** 9, p) == p
    total = sum(oracle.visible(t, p) for t in range(4 * p))
    assert total == 2 * p * p - p == W.visible_count_total(4 * p, p)


def test_hand_worked_example():
    # Two heads of width 2.  q_t = [[1, 2], [3, -1]], keys k0 = [1, 1], k1 = [-2, 1],
    # w = [0.5, 2].  Pool 0: dots 3 and 2 -> 0.5*3 + 2*2 = 5.5.  Pool 1: dots 0 and -7, both
    # cut by the ReLU -> 0.  Row t = 7 sees both pools, t = 3 only pool 0, t = 2 none.
    q = np.array([[1, 2], [3, -1]], dtype=np.float32)
    k = np.array([[1, 1], [-2, 1]], dtype=np.float32)
    w = np.array([0.5, 2.0], dtype=np.float32)
    qb = np.stack([_bf16_bits(q)] * 3)
    out = oracle.index_scores(qb, _bf16_bits(k), w, [7, 3, 2], 2)
    inf = np.float32(np.inf)
    assert out[0].tolist() == [5.5, 0.0]
    assert out[1].tolist() == [5.5, -inf]
    assert out[2].tolist() == [-inf, -inf]
    assert not np.signbit(out[0, 1])  # zero is +0


def test_single_head_unit_weight_is_relu_of_matmul():
    rng = np.random.default_rng(1)
    n, p, d = 96, 24, 64
    q = _rand_int(rng, (n, 1, d), 4)
    k = _rand_int(rng, (p, d), 4)
    rows = np.arange(n)
    out = oracle.index_scores(_bf16_bits(q), _bf16_bits(k), np.ones(1, np.float32), rows, p)
    ref = np.maximum(q[:, 0, :].astype(np.float64) @ k.T.astype(np.float64), 0.0)
    for t in range(n):
        v = min(p, (t + 1) // 4)
        assert np.array_equal(out[t, :v], ref[t, :v].astype(np.float32))
        assert np.all(np.isneginf(out[t, v:]))


def _scores(q, k, w, rows, p, dtype="bf16"):
    enc = _bf16_bits if dtype == "bf16" else _e4m3_bits
    return oracle.index_scores(enc(q), enc(k), w, rows, p)


def test_zero_weight_heads_change_nothing():
    rng = np.random.default_rng(2)
    n, p, h, d = 64, 16, 4, 32
    q = _rand_int(rng, (n, h, d), 4)
    k = _rand_int(rng, (p, d), 4)
    w = np.array([1.0, 0.5, 0.25, 0.125], np.float32)
    base = _scores(q, k, w, np.arange(n), p)
    extra = rng.normal(size=(n, 3, d)).astype(np.float32) * 7.0
    q2 = np.concatenate([q[:, :2], extra[:, :1], q[:, 2:], extra[:, 1:]], axis=1)
    w2 = np.array([1.0, 0.5, 0.0, 0.25, 0.125, 0.0, 0.0], np.float32)
    assert np.array_equal(base, _scores(q2, k, w2, np.arange(n), p))


def test_head_additivity_and_weight_doubling_are_exact():
    rng = np.random.default_rng(3)
    n, p, h, d = 80, 20, 8, 64
    q = _rand_int(rng, (n, h, d), 4)
    k = _rand_int(rng, (p, d), 4)
    w = np.array([2.0 ** -(j % 4) for j in range(h)], np.float32)
    rows = np.arange(n)
    full = _scores(q, k, w, rows, p)
    a = _scores(q[:, :3], k, w[:3], rows, p)
    b = _scores(q[:, 3:], k, w[3:], rows, p)
    fin = np.isfinite(full)
    assert np.array_equal(full[fin], (a + b)[fin])
    assert np.array_equal(np.isfinite(a), fin)
    twice = _scores(q, k, 2 * w, rows, p)
    assert np.array_equal(twice[fin], 2 * full[fin])


def test_fp8_and_bf16_agree_on_values_both_hold_exactly():
    rng = np.random.default_rng(4)
    n, p, h, d = 64, 16, 3, 128
    q = _rand_int(rng, (n, h, d), 8)
    k = _rand_int(rng, (p, d), 8)
    w = np.array([1.0, 0.5, 0.25], np.float32)
    rows = np.arange(n)
    assert np.array_equal(_scores(q, k, w, rows, p, "bf16"), _scores(q, k, w, rows, p, "fp8"))


def test_per_row_weights_and_row_subsets():
    rng = np.random.default_rng(5)
    n, p, h, d = 40, 10, 2, 32
    q = _rand_int(rng, (n, h, d), 4)
    k = _rand_int(rng, (p, d), 4)
    wrow = rng.choice([0.25, 0.5, 1.0, 2.0], size=(n, h)).astype(np.float32)
    rows = np.arange(n)
    full = oracle.index_scores(_bf16_bits(q), _bf16_bits(k), wrow, rows, p)
    for t in (3, 17, 39):
        one = oracle.index_scores(_bf16_bits(q[t:t + 1]), _bf16_bits(k), wrow[t], [t], p)
        assert np.array_equal(one[0], full[t])
    sub = [5, 30, 11]
    part = oracle.index_scores(_bf16_bits(q[sub]), _bf16_bits(k), wrow[sub], sub, p)
    assert np.array_equal(part, full[sub])


def test_scores_of_integer_inputs_are_exact_in_fp32():
    # The indexer's fp32 result is exact for the workloads' integer inputs, which is what
    # makes bit-exact comparison with any summation order possible: check the bound.
    for wl in W.WORKLOADS.values():
        r = wl.int_range
        max_dot = wl.d_i * r * r
        max_score = max_dot * sum(2.0 ** -(j % wl.w_period) for j in range(wl.h_i))
        granularity_bits = wl.w_period - 1  # weights are multiples of 2^-(period-1)
        assert max_score * 2 ** granularity_bits < 2 ** 24, wl.name
    rng = np.random.default_rng(6)
    q = np.full((8, 32, 128), 4.0, np.float32)
    k = np.full((4, 128), 4.0, np.float32)
    w = np.array([2.0 ** -(j % 4) for j in range(32)], np.float32)
    out = _scores(q, k, w, np.arange(8) + 16, 4)
    assert out[0, 0] == 2048.0 * w.sum()
    del rng


def test_hand_worked_example_with_negative_weights():
    # The head weight multiplies the ReLU'd dot product; it is not inside the ReLU.  Two heads
    # of width 3, q_t = [[2, 0, -1], [1, 1, 1]], keys k0 = [1, 2, 3], k1 = [-1, 0, 2],
    # w = [-1, 2].
    #   pool 0: dots 2*1 + 0*2 - 1*3 = -1 and 1 + 2 + 3 = 6 -> -1*0 + 2*6 = 12
    #   pool 1: dots -2 + 0 - 2 = -4 and -1 + 0 + 2 = 1 -> -1*0 + 2*1 = 2
    # with w = [-2, -1] instead: pool 0 -> -2*0 - 1*6 = -6, pool 1 -> -2*0 - 1*1 = -1.
    # Had the weight sat inside the ReLU (max(0, w*dot)) these would read 1*... = 13, 6, 2, 8.
    q = np.array([[2, 0, -1], [1, 1, 1]], dtype=np.float32)
    k = np.array([[1, 2, 3], [-1, 0, 2]], dtype=np.float32)
    q = np.pad(q, ((0, 0), (0, 29)))  # d_i = 32 (zero columns change no dot product)
    k = np.pad(k, ((0, 0), (0, 29)))
    qb = _bf16_bits(q)[None]
    kb = _bf16_bits(k)
    pos = oracle.index_scores(qb, kb, np.array([-1.0, 2.0], np.float32), [7], 2)
    neg = oracle.index_scores(qb, kb, np.array([-2.0, -1.0], np.float32), [7], 2)
    assert pos[0].tolist() == [12.0, 2.0]
    assert neg[0].tolist() == [-6.0, -1.0]


def test_signed_per_row_weights_match_numpy_relu_sum():
    # Per-token signed weights: I[t, s] = sum_j w[t, j] * max(0, q[t, j] . k[s]), written with
    # numpy matmuls in float64 (every value is an exact integer multiple of 1/8, so the one
    # fp32 rounding of the oracle is exact too).
    rng = np.random.default_rng(7)
    n, p, h, d = 72, 18, 5, 64
    q = _rand_int(rng, (n, h, d), 4)
    k = _rand_int(rng, (p, d), 4)
    w = (rng.choice([-2.0, -1.0, -0.5, -0.125, 0.25, 1.0, 2.0], size=(n, h))).astype(np.float32)
    rows = np.arange(n)
    out = oracle.index_scores(_bf16_bits(q), _bf16_bits(k), w, rows, p)
    dots = np.einsum("thd,sd->ths", q.astype(np.float64), k.astype(np.float64))
    ref = np.einsum("th,ths->ts", w.astype(np.float64), np.maximum(dots, 0.0))
    assert np.any(ref < 0) and np.any(ref > 0)
    for t in range(n):
        v = min(p, (t + 1) // 4)
        assert np.array_equal(out[t, :v], ref[t, :v].astype(np.float32)), t
        assert np.all(np.isneginf(out[t, v:]))
    # a negated weight vector negates every score exactly (the ReLU does not see w)
    neg = oracle.index_scores(_bf16_bits(q), _bf16_bits(k), -w, rows, p)
    fin = np.isfinite(out)
    assert np.array_equal(neg[fin], -out[fin] + 0.0)
