"""GPU parity of the forward path (indexer scores, top-k, sparse attention, chunked driver)
against the CPU oracle, through the C ABI.  Scores and indices must match bit-exactly;
attention outputs within max |err| <= 2e-2 RMS and mean |err| <= 2e-3 RMS."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_index_amd import binding as B
from long_context_sparse_index_amd import inputs as I
from long_context_sparse_index_amd import workloads as W

from gpu_util import MAX_REL, MEAN_REL, assert_close, f32_bits_equal, host_bits, say

pytestmark = pytest.mark.gpu
TINY = W.WORKLOADS["tiny_4k"]


def _visible(t, p):
    return min(p, (t + 1) // 4)


def _check_scores(gpu_scores, ref, rows, p, sentinel_untouched=True):
    g = gpu_scores.cpu().numpy()
    for r, t in enumerate(rows):
        v = _visible(int(t), p)
        assert f32_bits_equal(g[r, :v], ref[r, :v]), "row %d (t=%d) differs" % (r, t)
        if sentinel_untouched:
            assert np.all(np.isnan(g[r, v:p])), "row %d wrote beyond its visible prefix" % r


def test_indexer_tiny_full_bit_exact(gpu):
    say("case: indexer tiny_4k full")
    q, k, w = I.index_inputs(TINY, gpu)
    scores = B.index_scores_new(q, k, w)
    torch.cuda.synchronize()
    rows = np.arange(TINY.n_tokens)
    ref = oracle.index_scores(host_bits(q), host_bits(k), w.cpu().numpy(), rows, TINY.n_pools)
    _check_scores(scores, ref, rows, TINY.n_pools)


@pytest.mark.parametrize("d_i", [32, 64, 128, 256])
def test_indexer_ragged_offsets_negative_weights_accumulate(gpu, d_i):
    say("case: indexer ragged d_i=%d" % d_i)
    # 12 heads, written as 3 then accumulated as 9: calls with at most 8 heads and with
    # more take the two query-tile sizes of the kernel
    nq, q_start, p, h_i, ld = 777, 1234, 301, 12, 304
    g = torch.Generator(device=gpu).manual_seed(7 + d_i)
    q = torch.randint(-4, 5, (nq, h_i, d_i), generator=g, device=gpu, dtype=torch.int8).to(
        torch.bfloat16)
    k = torch.randint(-4, 5, (p, d_i), generator=g, device=gpu, dtype=torch.int8).to(
        torch.bfloat16)
    choices = torch.tensor([1.0, 0.5, -0.25, 2.0, 0.0], device=gpu)
    w = choices[torch.randint(0, 5, (nq, h_i), generator=g, device=gpu)].float().contiguous()
    scores = torch.full((nq, ld), float("nan"), device=gpu)
    # heads 0..2 written, heads 3..11 accumulated on top (a head-share partial sum)
    B.index_scores(q[:, :3], k, w[:, :3], scores, q_start=q_start)
    B.index_scores(q[:, 3:], k, w[:, 3:], scores, q_start=q_start, accumulate=True)
    torch.cuda.synchronize()
    rows = np.arange(q_start, q_start + nq)
    ref = oracle.index_scores(host_bits(q), host_bits(k), w.cpu().numpy(), rows, p)
    _check_scores(scores, ref, rows, p)


@pytest.mark.parametrize("h_i", [6, 12])
def test_indexer_fp8_bit_exact(gpu, h_i):
    say("case: indexer fp8 e4m3, d_i=128, %d heads" % h_i)
    wl = W.Workload(name="fp8_small", n_tokens=3000, n_pools=750, h_i=h_i, d_i=128,
                    index_dtype="fp8", int_range=8, w_period=4, topk=64)
    q, k, w = I.index_inputs(wl, gpu, seed=3)
    scores = B.index_scores_new(q, k, w)
    torch.cuda.synchronize()
    rows = np.arange(wl.n_tokens)
    ref = oracle.index_scores(host_bits(q), host_bits(k), w.cpu().numpy(), rows, wl.n_pools)
    _check_scores(scores, ref, rows, wl.n_pools)


@pytest.mark.parametrize("d_i,h_i", [(128, 8), (256, 8), (128, 12), (256, 12)])
def test_indexer_fp8_mixed_weights(gpu, d_i, h_i):
    """e4m3 indexer with head weights of every kind in one call: tiles whose weights are
    all positive powers of two and tiles with a 3.0 weight, a zero weight or negative
    weights must all be bit-exact against the oracle on every row, the ragged last tile
    included.  At d_i = 128 eight heads take the 64-row tiles of few-head launches; the
    other cases take 32-row tiles, whose MFMAs issue as one group per head."""
    say("case: indexer fp8 mixed weights, d_i=%d, %d heads" % (d_i, h_i))
    rng = np.random.default_rng(17 + d_i + h_i)
    nq, p, q_start = 200, 900, 3000
    x = rng.integers(-8, 9, size=(nq, h_i, d_i)).astype(np.float32)
    y = rng.integers(-8, 9, size=(p, d_i)).astype(np.float32)
    q = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).to(gpu)
    k = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).to(gpu)
    wh = np.tile(np.array([2.0 ** -(j % 4) for j in range(h_i)], np.float32), (nq, 1))
    wh[70, 3] = 3.0      # tile 2: not a power of two
    wh[100, 0] = 0.0     # tile 3: zero weight
    wh[130:140, 5] = -0.5  # tile 4: negative weights
    wh[199, 7] = 0.375   # the ragged last tile
    w = torch.from_numpy(wh).to(gpu)
    scores = B.index_scores_new(q, k, w, q_start=q_start)
    torch.cuda.synchronize()
    rows = np.arange(q_start, q_start + nq)
    ref = oracle.index_scores(host_bits(q), host_bits(k), wh, rows, p)
    _check_scores(scores, ref, rows, p)


@pytest.mark.parametrize("h_i,d_i,dtype", [(1, 128, "bf16"), (3, 64, "bf16"), (4, 128, "bf16"),
                                          (8, 128, "bf16"), (12, 128, "bf16"), (16, 128, "bf16"),
                                          (8, 64, "bf16"), (8, 128, "fp8"), (5, 32, "bf16")])
def test_indexer_large_launch_few_heads(gpu, h_i, d_i, dtype):
    """Few heads over 131k pools in one launch of 1000 rows (thousands of blocks, both query
    tile sizes): every visible score bit-identical to 32-row calls, nothing written past a
    row's visible prefix, and the oracle's scores on rows at each position of 32- and 64-row
    tiles, at the causal edge (pool count still growing) and at the ragged end.  Written in
    one call and as a head split (write, then accumulate)."""
    p, nq = 131072 + 77, 1000
    q_start = 4 * p - 600  # local rows below 599 see fewer than p pools
    say("case: indexer large launch h_i=%d d_i=%d %s (P=%d, nq=%d)" % (h_i, d_i, dtype, p,
                                                                           nq))
    rng = np.random.default_rng(1000 * h_i + d_i + (1 if dtype == "fp8" else 0))
    r = 8 if dtype == "fp8" else 4

    def ints(shape):
        x = torch.from_numpy(rng.integers(-r, r + 1, size=shape).astype(np.float32))
        x = x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float8_e4m3fn).view(
            torch.uint8)
        return x.to(gpu)

    q, k = ints((nq, h_i, d_i)), ints((p, d_i))
    # per-row weights in eighths, zero and negative ones included: every score stays exact
    w = torch.from_numpy((rng.integers(-8, 17, size=(nq, h_i)) / 8.0).astype(np.float32)).to(gpu)
    ld = ((p + 3) // 4) * 4
    one = torch.full((nq, ld), float("nan"), device=gpu)
    B.index_scores(q, k, w, one, q_start=q_start)
    split = torch.full((nq, ld), float("nan"), device=gpu)
    h0 = max(1, h_i // 2)
    B.index_scores(q[:, :h0], k, w[:, :h0], split, q_start=q_start)
    if h0 < h_i:
        B.index_scores(q[:, h0:], k, w[:, h0:], split, q_start=q_start, accumulate=True)
    ref = torch.full((nq, ld), float("nan"), device=gpu)
    for r0 in range(0, nq, 32):
        r1 = min(nq, r0 + 32)
        B.index_scores(q[r0:r1], k, w[r0:r1], ref[r0:r1], q_start=q_start + r0)
    torch.cuda.synchronize()
    t = torch.arange(q_start, q_start + nq, device=gpu, dtype=torch.int64)
    vis = torch.clamp((t + 1) // 4, max=p)
    inside = torch.arange(ld, device=gpu)[None, :] < vis[:, None]
    assert bool(torch.isnan(ref[~inside]).all())
    for name, got in (("one call", one), ("head split", split)):
        assert torch.equal(got[inside].view(torch.int32), ref[inside].view(torch.int32)), name
        assert bool(torch.isnan(got[~inside]).all()), name + " wrote past a visible prefix"
    rows = np.array([0, 31, 32, 63, 64, 95, 96, 127, 128, 598, 599, 600, 960, 999])
    want = oracle.index_scores(host_bits(q[torch.from_numpy(rows).to(gpu)]), host_bits(k),
                               w.cpu().numpy()[rows], q_start + rows, p)
    _check_scores(one[torch.from_numpy(rows).to(gpu)], want, q_start + rows, p)


def test_topk_tiny_bit_exact(gpu):
    say("case: topk tiny_4k")
    q, k, w = I.index_inputs(TINY, gpu)
    scores = B.index_scores_new(q, k, w)
    idx = B.topk_new(scores, q_start=0, n_pools=TINY.n_pools, k=TINY.topk)
    torch.cuda.synchronize()
    rows = np.arange(TINY.n_tokens)
    ref = oracle.topk(scores.cpu().numpy(), rows, TINY.n_pools, TINY.topk)
    assert np.array_equal(idx.cpu().numpy(), ref)
    assert int((idx == -1).sum()) == 131328


def _edge_scores(kind, nq, ld, rng):
    if kind == "ties":
        return np.zeros((nq, ld), np.float32)
    if kind == "few_values":
        return (rng.integers(0, 6, size=(nq, ld)) / 8.0).astype(np.float32)
    if kind == "signed_zero_neg":
        s = rng.choice(np.array([0.0, -0.0, -1.5, 2.0, -3e-38, 1e30], np.float32), size=(nq, ld))
        return s.astype(np.float32)
    if kind == "normal":
        return rng.normal(size=(nq, ld)).astype(np.float32)
    if kind == "clustered_ints":
        return (rng.normal(450, 130, size=(nq, ld)).round() / 8.0).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["ties", "few_values", "signed_zero_neg", "normal",
                                  "clustered_ints"])
@pytest.mark.parametrize("k", [1, 100, 1030, 2048, 2051, 2056, 4096])
def test_topk_edge_cases(gpu, kind, k):
    say("case: topk edge kind=%s k=%d" % (kind, k))
    rng = np.random.default_rng(zlib.crc32(("%s/%d" % (kind, k)).encode()))
    p = 20000
    ld = 20000
    rows = np.array([0, 1, 2, 3, 7, 4 * k - 2, 4 * k - 1, 4 * k, 4 * k + 5, 30011, 79999,
                     4 * p + 9], dtype=np.int64)
    host = _edge_scores(kind, len(rows), ld, rng)
    scores = torch.from_numpy(host).to(gpu)
    idx = torch.empty((len(rows), k), dtype=torch.int32, device=gpu)
    # rows are not consecutive: run one call per row with its own q_start
    for r, t in enumerate(rows):
        B.topk(scores[r:r + 1], idx[r:r + 1], q_start=int(t), n_pools=p)
    torch.cuda.synchronize()
    ref = oracle.topk(host, rows, p, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("p", [40000, 70000])
@pytest.mark.parametrize("kind", ["ties", "clustered_ints", "normal"])
@pytest.mark.parametrize("k", [2048, 4096])
def test_topk_pool_counts(gpu, p, kind, k):
    """Row lengths past 32768 and 65536 visible pools (the 64-key-per-thread and the
    streaming selection paths)."""
    say("case: topk pools=%d kind=%s k=%d" % (p, kind, k))
    rng = np.random.default_rng(zlib.crc32(("%d/%s/%d" % (p, kind, k)).encode()))
    rows = np.array([5, 4 * k - 1, 4 * k + 3, 2 * p + 1, 4 * p - 5, 4 * p + 100],
                    dtype=np.int64)
    host = _edge_scores(kind, len(rows), p, rng)
    scores = torch.from_numpy(host).to(gpu)
    idx = torch.empty((len(rows), k), dtype=torch.int32, device=gpu)
    for r, t in enumerate(rows):
        B.topk(scores[r:r + 1], idx[r:r + 1], q_start=int(t), n_pools=p)
    torch.cuda.synchronize()
    ref = oracle.topk(host, rows, p, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("kind", ["sampled_high", "sampled_low"])
def test_topk_long_rows_sample_fallbacks(gpu, kind):
    """Long rows estimate their threshold from 256-byte pieces every 4 KB of the row (score
    positions i with i % 1024 < 64).  Scores that make those pieces unrepresentative push
    the candidate count below k (sampled_high) or past the candidate list (sampled_low);
    either way the result must stay exact."""
    say("case: topk long rows, %s" % kind)
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    p, k = 70000, 2048
    rows = np.array([4 * 32768 - 1, 4 * 40000 + 3, 4 * p + 7], dtype=np.int64)
    pos = np.arange(p)
    in_sample = (pos % 1024) < 64
    shift = 10.0 if kind == "sampled_high" else -10.0
    host = np.stack([(rng.normal(size=p) + np.where(in_sample, shift, 0.0)).astype(np.float32)
                     for _ in rows])
    scores = torch.from_numpy(host).to(gpu)
    idx = torch.empty((len(rows), k), dtype=torch.int32, device=gpu)
    for r, t in enumerate(rows):
        B.topk(scores[r:r + 1], idx[r:r + 1], q_start=int(t), n_pools=p)
    torch.cuda.synchronize()
    ref = oracle.topk(host, rows, p, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_many_marked_rows(gpu):
    """Rows the list paths cannot finish are selected by a pass over marked rows with one
    block per compute unit, each taking every G-th row in batches of 1024.  263144 rows of
    4200 visible pools (more than 256 x 1024, so blocks run several batches and several rows
    per batch): every third row all zero (the sampled list overflows: marked; ties go to the
    lowest pools), the others distinct values (sampled list in range).  Both expected
    results are closed forms: pools 0 .. k-1, and the pools of the k largest values."""
    nq, p, k = 263144, 4200, 2048
    say("case: topk %d rows, every third one marked" % nq)
    pos = torch.arange(p, device=gpu, dtype=torch.int64)
    distinct = ((pos * 7919) % p).to(torch.float32)
    scores = distinct.repeat(nq, 1)
    scores[0::3] = 0.0
    idx = B.topk_new(scores, q_start=4 * p, n_pools=p, k=k)
    torch.cuda.synchronize()
    want_ties = torch.arange(k, device=gpu, dtype=torch.int32)
    want_distinct = torch.argsort(distinct, descending=True)[:k].to(torch.int32)
    assert bool((idx[0::3] == want_ties).all())
    other = torch.ones(nq, dtype=torch.bool, device=gpu)
    other[0::3] = False
    assert bool((idx[other] == want_distinct).all())


def test_topk_chunk_of_consecutive_rows(gpu):
    say("case: topk consecutive rows, clustered ints, q_start=100000")
    rng = np.random.default_rng(5)
    p, nq, k, q_start = 32768, 256, 2048, 100000
    host = _edge_scores("clustered_ints", nq, p, rng)
    scores = torch.from_numpy(host).to(gpu)
    idx = B.topk_new(scores, q_start=q_start, n_pools=p, k=k)
    torch.cuda.synchronize()
    ref = oracle.topk(host, np.arange(q_start, q_start + nq), p, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def _attn_ref(q, kv, idx, scale, d_v, v=None):
    return oracle.sparse_attn_fwd(host_bits(q), host_bits(kv), idx.cpu().numpy(), scale,
                                  v_bits=None if v is None else host_bits(v), d_v=d_v)


@pytest.mark.parametrize("separate_v", [False, True])
def test_attention_tiny(gpu, separate_v):
    say("case: attention tiny_4k separate_v=%s" % separate_v)
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    idx = B.topk_new(B.index_scores_new(q_i, k_i, w), q_start=0, n_pools=TINY.n_pools,
                     k=TINY.topk)
    q, kv, v = I.attn_inputs(TINY, gpu, separate_v=separate_v)
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=TINY.scale, d_v=TINY.d_v, v=v)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, kv, idx, TINY.scale, TINY.d_v, v)
    assert_close(o.cpu().numpy(), ro, "O")
    lse_h = lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse_h), fin)
    assert np.all(o.cpu().numpy()[:3] == 0.0)
    assert np.max(np.abs(lse_h[fin] - rl[fin])) < 1e-4


def test_attention_bf16_output_is_correctly_rounded(gpu):
    say("case: attention tiny_4k, bf16 output")
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    idx = B.topk_new(B.index_scores_new(q_i, k_i, w), q_start=0, n_pools=TINY.n_pools,
                     k=TINY.topk)
    q, kv, _ = I.attn_inputs(TINY, gpu)
    o, _ = B.sparse_attn_fwd_new(q, kv, idx, scale=TINY.scale, d_v=TINY.d_v,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, _ = _attn_ref(q, kv, idx, TINY.scale, TINY.d_v)
    got = o.float().cpu().numpy()
    # bf16 round-to-nearest-even moves a value by at most 2^-8 of its magnitude; allow that
    # plus a small absolute term for the fp32 path before the rounding.
    rms = float(np.sqrt(np.mean(ro * ro)))
    excess = np.abs(got - ro) - (2.0 ** -8 * np.abs(ro) + 1e-4 * rms)
    say("  worst excess over the bf16 rounding bound: %.3g (rms %.3g)" % (excess.max(), rms))
    assert excess.max() <= 0.0


@pytest.mark.parametrize("h", [64, 40, 16, 5])
def test_attention_latent_576_random_selection(gpu, h):
    say("case: attention 576/512 random idx h=%d" % h)
    nq, p, k = 48, 4096, 2048
    g = torch.Generator(device=gpu).manual_seed(11 + h)
    q = torch.randn((nq, h, 576), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, 576), generator=g, device=gpu, dtype=torch.bfloat16)
    perm = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = perm.to(torch.int32).contiguous()
    drop = torch.rand((nq, k), generator=g, device=gpu) < 0.1
    idx[drop] = -1
    idx[0] = -1  # a row with no valid slot
    idx[1, :] = -1
    idx[1, 5] = 17  # a row with one valid slot
    idx[2, 33:] = -1  # a partial last tile
    # Rows whose gathers run past the last tile (the tile two ahead is reloaded from a valid
    # row into the free stage): exactly 2 and 3 tiles, 3 and 4 tiles with one key in the
    # last; and the two sides of the probability-precision boundary (512 valid slots).
    for r, n_keep in [(3, 64), (4, 65), (5, 96), (6, 97), (7, 511), (8, 512)]:
        keep = perm[r, :n_keep].to(torch.int32)
        idx[r, :] = -1
        idx[r, k - n_keep:] = keep  # valid slots at the end of the row: compaction matters
    scale = 1.0 / 24.0
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=512)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, kv, idx, scale, 512)
    assert_close(o.cpu().numpy(), ro, "O")
    lse_h = lse.cpu().numpy()
    assert np.all(np.isneginf(lse_h[0])) and np.all(o[0].cpu().numpy() == 0)
    assert np.array_equal(o[1].cpu().numpy(), np.broadcast_to(
        kv[17, :512].float().cpu().numpy(), (h, 512)))  # one slot: O is that value row
    fin = np.isfinite(rl)
    assert np.max(np.abs(lse_h[fin] - rl[fin])) < 1e-4


@pytest.mark.parametrize("separate_v", [False, True])
@pytest.mark.parametrize("h", [64, 24])
@pytest.mark.parametrize("d", [256, 512])
def test_attention_nope_latent_rows(gpu, d, h, separate_v):
    """Latent rows without their rotary columns (NoPE): d_qk = d_v = d, V the whole row (or
    a separate table), k = 2051, not a multiple of the 32-key tile."""
    say("case: attention NoPE %d/%d random idx h=%d separate_v=%s" % (d, d, h, separate_v))
    nq, p, k = 40, 4096, 2051
    g = torch.Generator(device=gpu).manual_seed(31 + d + h + int(separate_v))
    q = torch.randn((nq, h, d), generator=g, device=gpu, dtype=torch.bfloat16)
    kv = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16)
    v = torch.randn((p, d), generator=g, device=gpu, dtype=torch.bfloat16) if separate_v \
        else None
    perm = torch.argsort(torch.rand((nq, p), generator=g, device=gpu), dim=1)[:, :k]
    idx = perm.to(torch.int32).contiguous()
    idx[torch.rand((nq, k), generator=g, device=gpu) < 0.1] = -1
    idx[0] = -1  # a row with no valid slot
    idx[1, :] = -1
    idx[1, 2050] = 9  # one valid slot, in the partial last tile
    idx[2, 33:] = -1
    scale = 1.0 / float(np.sqrt(d))
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=d, v=v)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, kv, idx, scale, d, v=v)
    assert_close(o.cpu().numpy(), ro, "O")
    assert np.all(o[0].cpu().numpy() == 0) and np.all(np.isneginf(lse[0].cpu().numpy()))
    vt = v if separate_v else kv
    assert np.array_equal(o[1].cpu().numpy(), np.broadcast_to(
        vt[9, :d].float().cpu().numpy(), (h, d)))  # one slot: O is that value row
    fin = np.isfinite(rl)
    assert np.max(np.abs(lse.cpu().numpy()[fin] - rl[fin])) < 1e-4


def test_attention_logit_far_above_first_tile(gpu):
    """The forward takes each head's softmax reference from the first gathered tile; a
    later logit more than 2^64 above it must trigger the exact-maximum redo of the token."""
    say("case: attention 576/512, huge logit in a later tile")
    nq, h, p, k = 4, 64, 512, 256
    g = torch.Generator(device=gpu).manual_seed(5)
    q = torch.zeros((nq, h, 576), dtype=torch.bfloat16, device=gpu)
    q[:, :, 0] = 64.0
    q[:, :, 1:] = (0.01 * torch.randn((nq, h, 575), generator=g, device=gpu)).to(torch.bfloat16)
    kv = (0.01 * torch.randn((p, 576), generator=g, device=gpu)).to(torch.bfloat16)
    kv[300, 0] = 64.0    # logit ~ 4096/24: far above the first tile's (~0)
    kv[301, 0] = -64.0
    idx = torch.arange(k, dtype=torch.int32, device=gpu).repeat(nq, 1).contiguous()
    idx[0, 100] = 300    # row 0: the huge key sits in tile 3
    idx[1, 5] = 300      # row 1: the huge key is in the first tile (no redo)
    idx[3, 200] = 301    # row 3: a huge negative logit only
    scale = 1.0 / 24.0
    o, lse = B.sparse_attn_fwd_new(q, kv, idx, scale=scale, d_v=512)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(q, kv, idx, scale, 512)
    assert_close(o.cpu().numpy(), ro, "O")
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3 * np.max(np.abs(rl))
    assert np.allclose(o[0].cpu().numpy(), kv[300, :512].float().cpu().numpy(), atol=1e-6)


def test_chunked_matches_separate_calls_and_is_chunk_invariant(gpu):
    say("case: forward_chunked tiny_4k, chunks 4096/1000/7")
    q_i, k_i, w = I.index_inputs(TINY, gpu)
    q, kv, _ = I.attn_inputs(TINY, gpu)
    n = TINY.n_tokens
    outs = []
    for chunk in (4096, 1000, 7):
        o = torch.empty((n, TINY.heads, TINY.d_v), dtype=torch.float32, device=gpu)
        lse = torch.empty((n, TINY.heads), dtype=torch.float32, device=gpu)
        idx = torch.empty((n, TINY.topk), dtype=torch.int32, device=gpu)
        B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=TINY.topk, chunk=chunk,
                          scale=TINY.scale, d_v=TINY.d_v, idx_out=idx)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu(), idx.cpu()))
    for o, lse, idx in outs[1:]:
        assert torch.equal(idx, outs[0][2])
        assert torch.equal(o.view(torch.int32), outs[0][0].view(torch.int32))
        assert torch.equal(lse, outs[0][1])
    rows = np.arange(n)
    ref_idx = oracle.topk(oracle.index_scores(host_bits(q_i), host_bits(k_i), w.cpu().numpy(),
                                              rows, TINY.n_pools), rows, TINY.n_pools, TINY.topk)
    assert np.array_equal(outs[0][2].numpy(), ref_idx)
    ro, _ = oracle.sparse_attn_fwd(host_bits(q), host_bits(kv), ref_idx, TINY.scale)
    assert_close(outs[0][0].numpy(), ro, "O")


def _check_selection_order_all_rows(gpu, wl, q_i, k_i, w, idx, sub=1024):
    """On every row, against that row's indexer scores (dsa_index_scores of its chunk, which
    the sampled rows pin to the oracle bit for bit): the valid slots are in the order of a
    full sort (score non-increasing, lower pool first on equal scores), and no visible pool
    left out beats the last selected one (an equal score only with a higher pool index)."""
    n, p, k = wl.n_tokens, wl.n_pools, wl.topk
    ld = ((p + 3) // 4) * 4
    scores = torch.empty((wl.chunk, ld), dtype=torch.float32, device=gpu)
    cols = torch.arange(ld, device=gpu)
    ninf = float("-inf")
    for t0 in range(0, n, wl.chunk):
        nq = min(wl.chunk, n - t0)
        B.index_scores(q_i[t0:t0 + nq], k_i, w, scores[:nq], q_start=t0)
        for r0 in range(0, nq, sub):
            m = min(sub, nq - r0)
            sc = scores[r0:r0 + m]
            blk = idx[t0 + r0:t0 + r0 + m]
            t = torch.arange(t0 + r0, t0 + r0 + m, device=gpu, dtype=torch.int64)
            vis = torch.clamp((t + 1) // 4, max=p)
            valid = blk >= 0
            pos = blk.clamp(min=0).long()
            g = torch.where(valid, torch.gather(sc, 1, pos),
                            torch.full((m, k), ninf, device=gpu))
            both = valid[:, 1:]
            assert not bool(((g[:, 1:] > g[:, :-1]) & both).any()), "t0=%d: order" % t0
            tie = (g[:, 1:] == g[:, :-1]) & both
            assert not bool((tie & (blk[:, 1:] <= blk[:, :-1])).any()), "t0=%d: tie order" % t0
            # the best visible pool that was not selected
            picked = torch.zeros((m, ld + 1), dtype=torch.bool, device=gpu)
            picked.scatter_(1, torch.where(valid, pos, torch.full_like(pos, ld)),
                            torch.ones_like(valid))
            left = (cols[None, :] < vis[:, None]) & ~picked[:, :ld]
            rest = torch.where(left, sc, torch.full_like(sc, ninf))
            del picked, left
            c = valid.sum(1)
            has_rest = c < vis
            if not bool(has_rest.any()):
                continue
            last = torch.gather(g, 1, (c - 1).clamp(min=0)[:, None])[:, 0]
            last_pool = torch.gather(blk, 1, (c - 1).clamp(min=0)[:, None])[:, 0]
            best = rest.max(1).values
            assert not bool((has_rest & (best > last)).any()), "t0=%d: a better pool left out" % t0
            eq = (rest == last[:, None]) & has_rest[:, None]
            first_eq = torch.where(eq, cols[None, :], torch.full_like(cols[None, :], ld)).min(1).values
            assert not bool((first_eq <= last_pool.long()).any()), "t0=%d: tie left out" % t0
    del scores


def _full_size_forward(gpu, wl, check_rows):
    q_i, k_i, w = I.index_inputs(wl, gpu)
    q, kv, _ = I.attn_inputs(wl, gpu)
    n = wl.n_tokens
    o_dtype = torch.bfloat16 if wl.attn_out == "bf16" else torch.float32
    o = torch.empty((n, wl.heads, wl.d_v), dtype=o_dtype, device=gpu)
    lse = torch.empty((n, wl.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, wl.topk), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=wl.topk, chunk=wl.chunk, scale=wl.scale,
                      d_v=wl.d_v, idx_out=idx)
    torch.cuda.synchronize()
    say("  forward done")
    # structural invariants on every row (in blocks of rows to bound temporaries)
    slot = torch.arange(wl.topk, device=gpu)
    for r0 in range(0, n, 65536):
        blk = idx[r0:r0 + 65536]
        t = torch.arange(r0, r0 + blk.shape[0], device=gpu, dtype=torch.int64)
        vis = torch.clamp((t + 1) // 4, max=wl.n_pools)
        c = torch.clamp(vis, max=wl.topk)
        valid = blk >= 0
        assert torch.equal(valid.sum(1), c)
        assert torch.equal(valid, slot[None, :] < c[:, None])  # valid slots first
        assert bool((blk.long() < vis[:, None]).all())
        srt = torch.sort(blk, dim=1).values
        dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
        assert not bool(dup.any())
    say("  structure ok on all %d rows" % n)
    _check_selection_order_all_rows(gpu, wl, q_i, k_i, w, idx)
    say("  selection order and threshold ok on all %d rows" % n)
    # sampled rows against the oracle
    rows = check_rows
    q_rows = host_bits(q_i[torch.from_numpy(rows).to(gpu)])
    ref_scores = oracle.index_scores(q_rows, host_bits(k_i), w.cpu().numpy(), rows, wl.n_pools)
    ref_idx = oracle.topk(ref_scores, rows, wl.n_pools, wl.topk)
    got_idx = idx[torch.from_numpy(rows).to(gpu)].cpu().numpy()
    assert np.array_equal(got_idx, ref_idx)
    say("  idx bit-exact on %d sampled rows" % len(rows))
    ro, rl = oracle.sparse_attn_fwd(host_bits(q[torch.from_numpy(rows).to(gpu)]),
                                    host_bits(kv), ref_idx, wl.scale, d_v=wl.d_v)
    got_o = o[torch.from_numpy(rows).to(gpu)].float().cpu().numpy()
    if o_dtype == torch.float32:
        assert_close(got_o, ro, "O (sampled rows)")
    else:
        # A bf16 output also carries the rounding to bf16 (at most 2^-8 of |O|, round to
        # nearest even): the max-abs tolerance applies on top of that bound, the mean-abs
        # tolerance as it stands.
        rms = float(np.sqrt(np.mean(ro * ro)))
        err = np.abs(got_o - ro)
        excess = err - (2.0 ** -8 * np.abs(ro) + MAX_REL * rms)
        say("  O bf16 (sampled rows): worst excess over rounding + tolerance %.3g, "
            "mean/rms %.3g (rms %.3g)" % (excess.max(), err.mean() / rms, rms))
        assert excess.max() <= 0.0 and err.mean() <= MEAN_REL * rms
    got_l = lse[torch.from_numpy(rows).to(gpu)].cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.max(np.abs(got_l[fin] - rl[fin])) < 1e-4


def test_fwd_128k_full_size_sampled(gpu):
    wl = W.WORKLOADS["fwd_128k"]
    say("case: fwd_128k full size (N=%d), chunk %d" % (wl.n_tokens, wl.chunk))
    _full_size_forward(gpu, wl, I.sample_rows(wl, n_uniform=24))


@pytest.mark.parametrize("name", ["nope_16k", "flash_nope_128k"])
def test_flash_native_full_size_sampled(gpu, name):
    """Flash-native shapes end to end: top-2051 indices bit-exact and NoPE 512/512 attention
    within tolerance on sampled rows, all rows structurally checked."""
    wl = W.WORKLOADS[name]
    say("case: %s full size (N=%d), chunk %d" % (name, wl.n_tokens, wl.chunk))
    _full_size_forward(gpu, wl, I.sample_rows(wl, n_uniform=24))


def test_tp_share_1m_full_size_sampled(gpu):
    """One GPU's share of the 1M-token layer: indices bit-exact and attention within tolerance
    on sampled rows (O in bf16 at this size)."""
    wl = W.WORKLOADS["tp_share_1m"]
    say("case: tp_share_1m full size (N=%d, P=%d), chunk %d" % (wl.n_tokens, wl.n_pools,
                                                              wl.chunk))
    _full_size_forward(gpu, wl, I.sample_rows(wl, n_uniform=16))
    torch.cuda.empty_cache()
