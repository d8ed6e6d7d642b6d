"""GPU parity of the fused select (dsa_index_topk): the indices must be bit-identical to
dsa_index_scores followed by dsa_topk, and to the CPU oracle, on every path of the fused
select: rows taking every visible pool, sampled thresholds, and rows redone exactly because
their candidate list fell outside [k, 4096] (heavy ties, score layouts that fool the
every-16th-pool sample)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_index_amd import binding as B
from long_context_sparse_index_amd import inputs as I

from gpu_util import host_bits, say

pytestmark = pytest.mark.gpu


def _ints(shape, lo, hi, rng, dtype):
    x = torch.from_numpy(rng.integers(lo, hi + 1, size=shape).astype(np.float32))
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def _two_calls(q_i, k_i, w, q_start, p, k):
    nq = q_i.shape[0]
    ld = ((max(p, 1) + 3) // 4) * 4
    scores = torch.empty((nq, ld), dtype=torch.float32, device=q_i.device)
    B.index_scores(q_i, k_i, w, scores, q_start=q_start, n_pools=p)
    idx = torch.empty((nq, k), dtype=torch.int32, device=q_i.device)
    B.topk(scores, idx, q_start=q_start, n_pools=p)
    return idx


def _fused(q_i, k_i, w, q_start, p, k):
    idx = torch.full((q_i.shape[0], k), -7, dtype=torch.int32, device=q_i.device)
    B.index_topk(q_i, k_i, w, idx, q_start=q_start, n_pools=p)
    return idx


def _oracle_rows(q_i, k_i, w, q_start, p, k, rows):
    """Oracle top-k of the given local rows (scores recomputed on the CPU)."""
    qb = host_bits(q_i.cpu())[rows]
    kb = host_bits(k_i.cpu())
    wh = w.cpu().numpy()
    if wh.ndim == 2:
        wh = wh[rows]
    t = q_start + np.asarray(rows, dtype=np.int64)
    sc = oracle.index_scores(qb, kb, wh, t, p)
    return oracle.topk(sc, t, p, k)


CASES = [
    # name, p, h_i, d_i, dtype, k, q_start, nq
    ("tiny_all_visible", 1024, 4, 64, "bf16", 256, 0, 4096),
    ("sampled_40k", 40000, 8, 128, "bf16", 2048, 100000, 700),
    ("sampled_70k_32h", 70000, 32, 128, "bf16", 2048, 4 * 70000 - 300, 600),
    ("fp8_k2051", 40000, 6, 128, "fp8", 2051, 60000, 333),
    ("d256_k1000", 20000, 3, 256, "bf16", 1000, 70000, 130),
    ("d32_k1", 9000, 12, 32, "bf16", 1, 30000, 77),
    ("k2730", 30000, 5, 64, "bf16", 2730, 4 * 30000 - 50, 100),
    ("boundary_4096", 8192, 4, 64, "bf16", 2048, 4 * 4096 - 40, 80),
    # 8 heads over 131k pools: a candidate pass of thousands of blocks
    ("large_131k_8h", 131149, 8, 128, "bf16", 2048, 4 * 131149 - 600, 1000),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_select_matches_two_calls_and_oracle(gpu, case):
    name, p, h_i, d_i, dtype, k, q_start, nq = case
    say("case: fused select %s (P=%d, h_i=%d, d_i=%d, %s, k=%d, q_start=%d, nq=%d)" % case)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    r = 8 if dtype == "fp8" else 4
    q_i = _ints((nq, h_i, d_i), -r, r, rng, dtype).to(gpu)
    k_i = _ints((p, d_i), -r, r, rng, dtype).to(gpu)
    # per-row weights, negative ones included: multiples of 1/8 keep every score exact
    w = torch.from_numpy((rng.integers(-8, 17, size=(nq, h_i)) / 8.0).astype(np.float32)).to(gpu)
    ref = _two_calls(q_i, k_i, w, q_start, p, k)
    got = _fused(q_i, k_i, w, q_start, p, k)
    torch.cuda.synchronize()
    g, rf = got.cpu().numpy(), ref.cpu().numpy()
    bad = np.nonzero(np.any(g != rf, axis=1))[0]
    assert bad.size == 0, "rows %s differ from the two-call path" % bad[:10]
    rows = np.unique(np.concatenate([[0, nq // 2, nq - 1], rng.integers(0, nq, size=5)]))
    assert np.array_equal(g[rows], _oracle_rows(q_i, k_i, w, q_start, p, k, rows))


@pytest.mark.parametrize("kind", ["all_ties", "few_values", "sample_high", "sample_low",
                                  "mixed"])
def test_fused_select_redo_rows(gpu, kind):
    """Candidate lists outside [k, 4096] send rows to the exact redo."""
    say("case: fused select redo, %s" % kind)
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    p, k, d_i = 20000, 2048, 64
    q_start, nq = 4 * p - 150, 150  # every row sees all 20000 pools
    if kind == "all_ties":
        q_i = torch.zeros((nq, 1, d_i), dtype=torch.bfloat16)
        k_i = _ints((p, d_i), -4, 4, rng, "bf16")
    elif kind == "mixed":
        # rows 40..69 and 130..149 tie everywhere (redone), the others select normally:
        # only the query tiles holding redone rows are recomputed
        q_i = _ints((nq, 1, d_i), -4, 4, rng, "bf16")
        q_i[40:70] = 0
        q_i[130:150] = 0
        k_i = _ints((p, d_i), -4, 4, rng, "bf16")
    elif kind == "few_values":
        q_i = _ints((nq, 1, d_i), 0, 1, rng, "bf16")
        k_i = _ints((p, d_i), 0, 1, rng, "bf16")
    else:
        # q = 1: the score is the key row's sum; pools that are multiples of 16 (the
        # threshold sample) get much larger (sample_high: too few candidates) or smaller
        # (sample_low: far too many) sums than the rest
        q_i = torch.ones((nq, 1, d_i), dtype=torch.bfloat16)
        kh = rng.integers(0, 3, size=(p, d_i)).astype(np.float32)
        kh[::16] += 3.0 if kind == "sample_high" else -3.0
        k_i = torch.from_numpy(kh).to(torch.bfloat16)
    q_i, k_i = q_i.to(gpu), k_i.to(gpu)
    w = torch.ones(1, dtype=torch.float32, device=gpu)
    ref = _two_calls(q_i, k_i, w, q_start, p, k)
    got = _fused(q_i, k_i, w, q_start, p, k)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(g, ref.cpu().numpy())
    if kind == "all_ties":  # closed form: the k lowest pools, in order
        assert np.array_equal(g, np.tile(np.arange(k, dtype=np.int32), (nq, 1)))
    rows = np.array([0, 45, 100, nq - 1])
    assert np.array_equal(g[rows], _oracle_rows(q_i, k_i, w, q_start, p, k, rows))


def test_fused_select_chunks_and_reuse(gpu):
    """One workspace reused across chunks of different sizes, as the chunked driver does."""
    say("case: fused select over chunks with one workspace")
    rng = np.random.default_rng(11)
    p, h_i, d_i, k = 12000, 4, 128, 2048
    n = 4 * p
    q_i = _ints((n, h_i, d_i), -4, 4, rng, "bf16").to(gpu)
    k_i = _ints((p, d_i), -4, 4, rng, "bf16").to(gpu)
    w = I.head_weights(h_i, 4, gpu)
    chunk = 9000
    ws = torch.empty(B.index_topk_workspace_bytes(chunk, p, k), dtype=torch.uint8, device=gpu)
    got = torch.empty((n, k), dtype=torch.int32, device=gpu)
    for t0 in range(0, n, chunk):
        nq = min(chunk, n - t0)
        B.index_topk(q_i[t0:t0 + nq], k_i, w, got[t0:t0 + nq], q_start=t0, n_pools=p, ws=ws)
    ref = _two_calls(q_i, k_i, w, 0, p, k)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_fused_select_rejects(gpu):
    say("case: fused select argument errors")
    q_i = torch.zeros((8, 2, 64), dtype=torch.bfloat16, device=gpu)
    k_i = torch.zeros((100, 64), dtype=torch.bfloat16, device=gpu)
    w = torch.ones(2, dtype=torch.float32, device=gpu)
    idx = torch.empty((8, 2731), dtype=torch.int32, device=gpu)
    with pytest.raises(B.DSAError) as e:
        B.index_topk(q_i, k_i, w, idx, q_start=0)
    assert e.value.status == 2  # unsupported: use the two calls
    idx = torch.empty((8, 16), dtype=torch.int32, device=gpu)
    small = torch.empty(256, dtype=torch.uint8, device=gpu)
    with pytest.raises(B.DSAError) as e:
        B.index_topk(q_i, k_i, w, idx, q_start=0, ws=small)
    assert e.value.status == 3


def test_chunked_forward_mixes_fused_and_two_call_chunks(gpu):
    """dsa_forward_chunked takes the fused select only with more than 16 indexer heads and on
    chunks whose first row sees at least 49152 pools: with 24 heads, P = 52000 and chunks of
    50000 queries only the last chunk does.
    Indices of every row must equal the two-call path, and the attention output is then the
    same kernel on the same indices (bit-identical)."""
    from long_context_sparse_index_amd import workloads as W

    say("case: chunked forward, P=52000, chunk 50000 (last chunk fused)")
    base = W.WORKLOADS["tiny_4k"]
    p = 52000
    wl = W.Workload(name="mixed", n_tokens=4 * p, n_pools=p, h_i=24, d_i=64,
                    index_dtype="bf16", int_range=4, w_period=4, topk=2048, heads=8,
                    d_qk=128, d_v=128, scale=base.scale, chunk=50000)
    q_i, k_i, w = I.index_inputs(wl, gpu)
    q, kv, _ = I.attn_inputs(wl, gpu)
    n, k = wl.n_tokens, wl.topk
    o = torch.empty((n, wl.heads, wl.d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((n, wl.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, k), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=k, chunk=wl.chunk, scale=wl.scale,
                      d_v=wl.d_v, idx_out=idx)
    ref_idx = torch.empty_like(idx)
    for t0 in range(0, n, wl.chunk):
        nq = min(wl.chunk, n - t0)
        ref_idx[t0:t0 + nq] = _two_calls(q_i[t0:t0 + nq], k_i, w, t0, p, k)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    o_ref = torch.empty_like(o)
    lse_ref = torch.empty_like(lse)
    B.sparse_attn_fwd(q, kv, ref_idx, o_ref, lse_ref, scale=wl.scale, d_v=wl.d_v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32))
    rows = np.array([4 * p - 1, 200001, 150000, 49999])
    qb = host_bits(q_i[torch.from_numpy(rows).to(gpu)].cpu())
    sc = oracle.index_scores(qb, host_bits(k_i.cpu()), w.cpu().numpy(), rows, p)
    assert np.array_equal(idx[torch.from_numpy(rows).to(gpu)].cpu().numpy(),
                          oracle.topk(sc, rows, p, k))


def test_chunked_forward_large_k_takes_two_call_select(gpu):
    """k above 2730 has no fused select: dsa_forward_chunked selects with dsa_index_scores +
    dsa_topk inside the same workspace layout; its indices and outputs must equal the
    separate calls."""
    from long_context_sparse_index_amd import workloads as W

    say("case: chunked forward, k=3000 (two-call select), P=6000, chunk 7000")
    base = W.WORKLOADS["tiny_4k"]
    p = 6000
    wl = W.Workload(name="large_k", n_tokens=4 * p, n_pools=p, h_i=4, d_i=64,
                    index_dtype="bf16", int_range=4, w_period=4, topk=3000, heads=8,
                    d_qk=128, d_v=128, scale=base.scale, chunk=7000)
    q_i, k_i, w = I.index_inputs(wl, gpu)
    q, kv, _ = I.attn_inputs(wl, gpu)
    n, k = wl.n_tokens, wl.topk
    o = torch.empty((n, wl.heads, wl.d_v), dtype=torch.float32, device=gpu)
    lse = torch.empty((n, wl.heads), dtype=torch.float32, device=gpu)
    idx = torch.empty((n, k), dtype=torch.int32, device=gpu)
    B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=k, chunk=wl.chunk, scale=wl.scale,
                      d_v=wl.d_v, idx_out=idx)
    ref_idx = _two_calls(q_i, k_i, w, 0, p, k)
    o_ref = torch.empty_like(o)
    lse_ref = torch.empty_like(lse)
    B.sparse_attn_fwd(q, kv, ref_idx, o_ref, lse_ref, scale=wl.scale, d_v=wl.d_v)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32))
    rows = np.array([3, 4 * 3000 + 1, n - 1])
    qb = host_bits(q_i[torch.from_numpy(rows).to(gpu)].cpu())
    sc = oracle.index_scores(qb, host_bits(k_i.cpu()), w.cpu().numpy(), rows, p)
    assert np.array_equal(idx[torch.from_numpy(rows).to(gpu)].cpu().numpy(),
                          oracle.topk(sc, rows, p, k))


def test_index_topk_256k_fp8_full_size_sampled(gpu):
    """The fp8 indexer + top-k workload at full size (N = 262144, P = 65536, 32 x 128 e4m3
    indexer, k = 2048, chunks of 16384), selected as the chunked driver does: the fused
    select on chunks whose rows see >= 49152 pools, the two calls elsewhere.  Structure on
    every row; sampled rows bit-exact against the oracle; the fused chunks also against the
    two-call path on all their rows."""
    from long_context_sparse_index_amd import workloads as W

    wl = W.WORKLOADS["index_topk_256k_fp8"]
    n, p, k, chunk = wl.n_tokens, wl.n_pools, wl.topk, wl.chunk
    say("case: index_topk_256k_fp8 full size (N=%d, P=%d), chunk %d" % (n, p, chunk))
    q_i, k_i, w = I.index_inputs(wl, gpu)
    idx = torch.empty((n, k), dtype=torch.int32, device=gpu)
    ws = torch.empty(B.index_topk_workspace_bytes(chunk, p, k), dtype=torch.uint8, device=gpu)
    n_fused = 0
    for t0 in range(0, n, chunk):
        nq = min(chunk, n - t0)
        if min(p, (t0 + 1) // 4) >= 49152:
            B.index_topk(q_i[t0:t0 + nq], k_i, w, idx[t0:t0 + nq], q_start=t0, n_pools=p, ws=ws)
            ref = _two_calls(q_i[t0:t0 + nq], k_i, w, t0, p, k)
            assert torch.equal(idx[t0:t0 + nq], ref), "fused chunk at %d differs" % t0
            n_fused += 1
        else:
            idx[t0:t0 + nq] = _two_calls(q_i[t0:t0 + nq], k_i, w, t0, p, k)
    torch.cuda.synchronize()
    say("  select done (%d fused chunks, equal to the two calls)" % n_fused)
    assert n_fused == 4
    slot = torch.arange(k, device=gpu)
    for r0 in range(0, n, 65536):
        blk = idx[r0:r0 + 65536]
        t = torch.arange(r0, r0 + blk.shape[0], device=gpu, dtype=torch.int64)
        vis = torch.clamp((t + 1) // 4, max=p)
        c = torch.clamp(vis, max=k)
        valid = blk >= 0
        assert torch.equal(valid.sum(1), c)
        assert torch.equal(valid, slot[None, :] < c[:, None])
        assert bool((blk.long() < vis[:, None]).all())
        srt = torch.sort(blk, dim=1).values
        assert not bool(((srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)).any())
    say("  structure ok on all %d rows" % n)
    rows = I.sample_rows(wl, n_uniform=16)
    rt = torch.from_numpy(rows).to(gpu)
    sc = oracle.index_scores(host_bits(q_i[rt].cpu()), host_bits(k_i.cpu()), w.cpu().numpy(),
                             rows, p)
    assert np.array_equal(idx[rt].cpu().numpy(), oracle.topk(sc, rows, p, k))
    say("  idx bit-exact on %d sampled rows" % len(rows))
