"""The C ABI library loads and exports every function include/dsa.h declares; host-side
argument checks reject bad calls before anything is launched (CPU only, no GPU calls)."""

import ctypes
import os
import re

import pytest

from long_context_sparse_index_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from long_context_sparse_index_amd import build
        build.build()
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert {"dsa_index_scores", "dsa_topk", "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd",
            "dsa_forward_chunked"} <= declared
    raw = ctypes.CDLL(binding.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(raw, name), name
    assert declared == set(binding.exported_symbols())


def test_status_strings_and_version(lib):
    assert lib.dsa_abi_version() == 2
    assert lib.dsa_status_string(0) == b"DSA_OK"
    assert lib.dsa_status_string(2) == b"DSA_ERR_UNSUPPORTED"


def test_workspace_sizes(lib):
    need = lib.dsa_forward_chunked_workspace_bytes(32768, 8192, 2048)
    assert need >= 8192 * 32768 * 4 + 8192 * 2048 * 4
    assert lib.dsa_sparse_attn_bwd_workspace_bytes(100, 64) >= 100 * 64 * 4


P = ctypes.c_void_p
FAKE = P(0x10000)  # never dereferenced: every call below fails validation


def _idx_call(lib, **kw):
    a = dict(q=FAKE, qs=4 * 64, k=FAKE, ks=64, w=FAKE, ws=0, sc=FAKE, ld=1024, q0=0, nq=16,
             P=1024, h=4, d=64, dt=0, acc=0)
    a.update(kw)
    return lib.dsa_index_scores(a["q"], a["qs"], a["k"], a["ks"], a["w"], a["ws"], a["sc"],
                                a["ld"], a["q0"], a["nq"], a["P"], a["h"], a["d"], a["dt"],
                                a["acc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(d=48), 2), (dict(d=64, dt=1), 2), (dict(h=65), 2),
    (dict(ld=1022), 1), (dict(ld=1000), 1), (dict(qs=100), 1), (dict(acc=2), 1),
    (dict(dt=7), 1), (dict(nq=-1), 1), (dict(sc=P(0x10004)), 1), (dict(ws=2), 1),
])
def test_indexer_rejects_bad_arguments(lib, kw, status):
    assert _idx_call(lib, **kw) == status
    assert lib.dsa_last_error() != b""


def test_topk_and_attention_reject_bad_arguments(lib):
    assert lib.dsa_topk(FAKE, 1024, 0, 4, 1024, 0, FAKE, None, 0, None) == 1
    assert lib.dsa_topk(FAKE, 1024, 0, 4, 1024, 4097, FAKE, None, 0, None) == 2
    assert lib.dsa_topk(FAKE, 1026, 0, 4, 1024, 16, FAKE, None, 0, None) == 1
    fwd = lib.dsa_sparse_attn_fwd
    F32 = 2
    # (d_qk, d_v) without a kernel, h > 64, bad ld_kv, missing output, k too large, bad o dtype
    assert fwd(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, 4, 100, 64, 576, 256, 0.1,
               None) == 2
    assert fwd(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, 4, 100, 65, 576, 512, 0.1,
               None) == 2
    assert fwd(FAKE, FAKE, 570, None, 0, FAKE, 2048, FAKE, F32, FAKE, 4, 100, 64, 576, 512, 0.1,
               None) == 1
    assert fwd(FAKE, FAKE, 576, None, 0, FAKE, 2048, None, F32, FAKE, 4, 100, 64, 576, 512, 0.1,
               None) == 1
    assert fwd(FAKE, FAKE, 576, None, 0, FAKE, 5000, FAKE, F32, FAKE, 4, 100, 64, 576, 512, 0.1,
               None) == 2
    assert fwd(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, 1, FAKE, 4, 100, 64, 576, 512, 0.1,
               None) == 1
    bwd = lib.dsa_sparse_attn_bwd
    # separate v without dv; too small workspace
    assert bwd(FAKE, FAKE, 576, FAKE, 512, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
               4, 100, 64, 576, 512, 0.1, FAKE, 1 << 20, None) == 1
    assert bwd(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None, 4,
               100, 64, 576, 512, 0.1, FAKE, 8, None) == 3


def test_chunked_rejects_small_workspace(lib):
    need = lib.dsa_forward_chunked_workspace_bytes(1024, 512, 256)
    st = lib.dsa_forward_chunked(FAKE, 256, FAKE, 64, FAKE, 0, 4, 64, 0, FAKE, FAKE, 128, None,
                                 0, 8, 128, 128, 0.1, 256, 4096, 1024, 512, FAKE, 2, FAKE, None,
                                 P(0x100000), need - 1, None)
    assert st == 3


def test_fused_select_and_deterministic_workspaces(lib):
    # the fused select keeps a full score buffer for its exact redo, plus 32 KB of candidate
    # list per row, a 1/16 sample of the scores and per-row flags
    need = lib.dsa_index_topk_workspace_bytes(8192, 32768, 2048)
    assert need >= 8192 * 32768 * 4 + 8192 * 4096 * 8 + 8192 * 2048 * 4
    assert lib.dsa_index_topk_workspace_bytes(0, 32768, 2048) == 0
    assert (lib.dsa_index_topk_workspace_bytes(100, 32768, 2048)
            < lib.dsa_index_topk_workspace_bytes(200, 32768, 2048))
    # the chunked forward holds the fused select's workspace and the index chunk
    assert (lib.dsa_forward_chunked_workspace_bytes(32768, 8192, 2048)
            >= lib.dsa_index_topk_workspace_bytes(8192, 32768, 2048) + 8192 * 2048 * 4)
    # k above the fused select's limit: score chunk, index chunk and top-k workspace only
    assert (lib.dsa_forward_chunked_workspace_bytes(32768, 8192, 3000)
            < lib.dsa_index_topk_workspace_bytes(8192, 32768, 2048))
    # deterministic backward: the per-row deltas, one staged fp32 dK (and dV) row per
    # (row, slot) of a chunk of at most 4096 rows, and the sort buffers (4 arrays of one int32
    # per pair, digit histograms, pool bounds)
    base = lib.dsa_sparse_attn_bwd_workspace_bytes(100, 64)
    det = lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(100, 64, 5000, 2048, 576, 512, 0)
    det_v = lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(100, 64, 5000, 2048, 576, 512,
                                                                  1)
    pairs = 100 * 2048
    assert det >= base + pairs * 576 * 4 + 4 * pairs * 4 + 5001 * 4
    # (one more staging row takes the stores of invalid slots)
    assert det_v - det == ((pairs + 1) * 512 * 4 + 255) // 256 * 256
    # chunks of 4096 rows: the staging does not grow past them
    big = lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(65536, 64, 16384, 2048, 576,
                                                                512, 0)
    mid = lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(4096, 64, 16384, 2048, 576,
                                                                512, 0)
    assert big - mid == (lib.dsa_sparse_attn_bwd_workspace_bytes(65536, 64)
                         - lib.dsa_sparse_attn_bwd_workspace_bytes(4096, 64))
    assert mid >= 4096 * 2048 * 576 * 4
    assert lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(0, 64, 100, 2048, 576, 512,
                                                                 0) == 0


def test_fused_select_and_deterministic_backward_reject_bad_arguments(lib):
    it = lib.dsa_index_topk
    # k beyond the fused select (2730), null idx, bad d_i, short or misaligned workspace
    assert it(FAKE, 256, FAKE, 64, FAKE, 0, 0, 16, 1024, 4, 64, 0, 2731, FAKE, FAKE, 1 << 30,
              None) == 2
    assert it(FAKE, 256, FAKE, 64, FAKE, 0, 0, 16, 1024, 4, 64, 0, 256, None, FAKE, 1 << 30,
              None) == 1
    assert it(FAKE, 256, FAKE, 64, FAKE, 0, 0, 16, 1024, 4, 48, 0, 256, FAKE, FAKE, 1 << 30,
              None) == 2
    need = lib.dsa_index_topk_workspace_bytes(16, 1024, 256)
    assert it(FAKE, 256, FAKE, 64, FAKE, 0, 0, 16, 1024, 4, 64, 0, 256, FAKE, P(0x100000),
              need - 1, None) == 3
    assert it(FAKE, 256, FAKE, 64, FAKE, 0, 0, 16, 1024, 4, 64, 0, 256, FAKE, P(0x100010),
              need, None) == 3
    det = lib.dsa_sparse_attn_bwd_deterministic
    F32 = 2
    # separate v without dv; (d_qk, d_v) without a kernel; short workspace
    assert det(FAKE, FAKE, 576, FAKE, 512, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
               4, 100, 64, 576, 512, 0.1, FAKE, 1 << 30, None) == 1
    assert det(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None, 4,
               100, 64, 576, 256, 0.1, FAKE, 1 << 30, None) == 2
    need = lib.dsa_sparse_attn_bwd_deterministic_workspace_bytes(4, 64, 100, 2048, 576, 512, 0)
    assert det(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None, 4,
               100, 64, 576, 512, 0.1, P(0x100000), need - 1, None) == 3


def test_noalloc_backward_rejects_sizes_past_its_static_scratch(lib):
    # nq * h above 2^22 per-row deltas is refused before any device call (this runs without
    # a GPU); so are the argument errors of dsa_sparse_attn_bwd
    nb = lib.dsa_sparse_attn_bwd_noalloc
    F32 = 2
    assert nb(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
              65537, 100, 64, 576, 512, 0.1, None) == 2
    assert b"static scratch" in lib.dsa_last_error()
    assert nb(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
              (1 << 22) + 1, 100, 1, 576, 512, 0.1, None) == 2
    assert nb(FAKE, FAKE, 576, FAKE, 512, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
              4, 100, 64, 576, 512, 0.1, None) == 1
    assert nb(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, None, FAKE, None,
              4, 100, 64, 576, 512, 0.1, None) == 1
    assert nb(FAKE, FAKE, 576, None, 0, FAKE, 2048, FAKE, F32, FAKE, FAKE, FAKE, FAKE, None,
              -1, 100, 64, 576, 512, 0.1, None) == 1


def test_pool_keys_rejects_bad_arguments(lib):
    pk = lib.dsa_pool_keys
    assert pk(None, 64, FAKE, 16, 64, FAKE, 64, None) == 1
    assert pk(None, 64, None, 3, 64, None, 64, None) == 0  # no pool: nothing accessed
    assert pk(FAKE, 64, FAKE, 16, 60, FAKE, 64, None) == 2  # d not a multiple of 8
    assert pk(FAKE, 56, FAKE, 16, 64, FAKE, 64, None) == 1  # ld_x < d
    assert pk(FAKE, 64, FAKE, -1, 64, FAKE, 64, None) == 1
    assert pk(P(0x10008), 64, FAKE, 16, 64, FAKE, 64, None) == 1  # misaligned x
