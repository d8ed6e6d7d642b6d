"""Pins of the CPU oracle's pooled keys and of its bf16 rounding (CPU only).

Reading (the pages name "one pool per 4 tokens" and "k-pool gate scores" on the page "SkyRL
extends GLM-5.3-Flash training context to 1 million tokens", sections "Model and
bottleneck" and "Four optimizations" item 3, but print no formula): pool s is the average of
the rows of tokens 4s .. 4s+3 weighted by the softmax of their gate scores, rounded once to
bf16.  The checks below tie the oracle to closed forms of that reading and to an exact
nearest-even search, not to the oracle itself.
"""

import math

import numpy as np
import torch

import oracle


def _bf16_bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _decode(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _nearest_even_bf16(v):
    """Brute force: among all finite bf16 values, the nearest to v (ties: even mantissa)."""
    allbits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):  # the NaN patterns
        vals = (allbits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    out = []
    for x in np.atleast_1d(v):
        if x == 0:  # signed zero keeps its sign
            out.append(0x8000 if math.copysign(1.0, x) < 0 else 0)
            continue
        with np.errstate(over="ignore", invalid="ignore"):
            dist = np.where(ok, np.abs(vals - x), np.inf)
        best = dist.min()
        cands = allbits[dist == best]
        # prefer the sign of x for zero, then an even last bit
        cands = [c for c in cands if not (x != 0 and (c >> 15) != (1 if x < 0 else 0))] or list(cands)
        even = [c for c in cands if c % 2 == 0]
        out.append((even or cands)[0])
    return np.array(out, dtype=np.uint16)


def test_round_bf16_is_nearest_even_including_exact_ties():
    rng = np.random.default_rng(11)
    vals = list(rng.normal(size=300) * np.exp2(rng.integers(-20, 20, size=300)))
    # exact midpoints between neighbouring bf16 values (ties) and their neighbours
    base = _decode(_bf16_bits(rng.normal(size=40)))
    for b in base:
        bits = int(_bf16_bits([b])[0])
        nxt = _decode([bits + 1])[0]
        mid = (b + nxt) / 2.0
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    vals += [0.0, -0.0, 1.0, -2.5, 2.0 ** -130, -3.0 * 2.0 ** -133, 1.7e38]
    vals = np.array(vals, dtype=np.float64)
    got = oracle.round_bf16(vals)
    ref = _nearest_even_bf16(vals)
    assert np.array_equal(got, ref)


def test_equal_gates_give_the_mean_of_the_four_rows():
    rng = np.random.default_rng(12)
    x = rng.integers(-8, 9, size=(20, 24)).astype(np.float32)  # 5 pools
    f64, bits = oracle.pool_keys(_bf16_bits(x), np.full(20, 0.75, np.float32))
    ref = x.astype(np.float64).reshape(5, 4, 24).mean(axis=1)  # exact: multiples of 1/4
    assert np.array_equal(f64, ref)
    assert np.array_equal(bits, _bf16_bits(ref))


def test_hand_worked_gates():
    # gates [0, ln 3, 0, 0] -> weights [1, 3, 1, 1] / 6; rows 6, 0, 12, -6 -> 12 / 6 = 2
    x = np.array([[6.0, 1.0], [0.0, 1.0], [12.0, 1.0], [-6.0, 1.0]], np.float32)
    g = np.array([0.0, math.log(3.0), 0.0, 0.0], np.float32)
    f64, bits = oracle.pool_keys(_bf16_bits(x), g)
    w = np.exp(g.astype(np.float64))
    w /= w.sum()
    assert abs(f64[0, 0] - float(w @ x[:, 0].astype(np.float64))) < 1e-15
    assert abs(f64[0, 0] - 2.0) < 1e-6 and abs(f64[0, 1] - 1.0) < 1e-15
    assert bits[0].tolist() == [0x4000, 0x3F80]  # 2.0 and 1.0


def test_dominant_gate_selects_its_row_and_shift_invariance():
    rng = np.random.default_rng(13)
    x = rng.normal(size=(16, 64)).astype(np.float32)
    xb = _bf16_bits(x)
    # gates on a 1/1024 grid, so that adding 4 to them is exact in fp32
    g = (np.round(rng.normal(size=16) * 1024) / 1024).astype(np.float32)
    g_dom = g.copy()
    g_dom[1::4] = 800.0  # the second token of every pool dominates
    _, bits = oracle.pool_keys(xb, g_dom)
    assert np.array_equal(bits, xb[1::4])
    f1, _ = oracle.pool_keys(xb, g)
    f2, _ = oracle.pool_keys(xb, g + np.float32(4.0))  # softmax is shift-invariant
    assert np.max(np.abs(f1 - f2)) <= 1e-12 * np.max(np.abs(f1))


def test_pool_reads_only_its_four_tokens_and_drops_the_partial_tail():
    rng = np.random.default_rng(14)
    x = rng.normal(size=(23, 32)).astype(np.float32)  # 5 pools, 3 tail tokens
    g = rng.normal(size=23).astype(np.float32)
    f64, _ = oracle.pool_keys(_bf16_bits(x), g)
    assert f64.shape == (5, 32)
    x2, g2 = x.copy(), g.copy()
    x2[8:12] += 3.0  # pool 2's tokens only
    g2[20:] = -7.0  # tail tokens: no pool
    f2, _ = oracle.pool_keys(_bf16_bits(x2), g2)
    changed = np.any(f64 != f2, axis=1)
    assert changed.tolist() == [False, False, True, False, False]
    # weights from numpy softmax, row by row
    xd = _decode(_bf16_bits(x))
    for s in range(5):
        w = np.exp(g[4 * s:4 * s + 4].astype(np.float64) - g[4 * s:4 * s + 4].max())
        w /= w.sum()
        assert np.allclose(f64[s], w @ xd[4 * s:4 * s + 4], rtol=1e-13, atol=1e-15)
    assert oracle.pool_keys(_bf16_bits(x[:3]), g[:3])[1].shape == (0, 32)


def test_pooled_value_is_rounded_once_from_the_exact_sum():
    # Equal gates, rows 1 + 2^-7, 1, 2^-30, 0: the mean is 0.5 + 2^-9 + 2^-32, just above the
    # midpoint 0.5 + 2^-9 between the bf16 neighbours 0.5 and 0.5 + 2^-8, so it rounds up.
    # Rounding to fp32 first would land on the midpoint and then tie to the even 0.5.
    col = np.array([1.0 + 2.0 ** -7, 1.0, 2.0 ** -30, 0.0], np.float64)
    x = np.stack([col, -col], axis=1).astype(np.float32)
    f64, bits = oracle.pool_keys(_bf16_bits(x), np.zeros(4, np.float32))
    assert f64[0, 0] == 0.5 + 2.0 ** -9 + 2.0 ** -32
    assert _decode(bits[0]).tolist() == [0.5 + 2.0 ** -8, -(0.5 + 2.0 ** -8)]
