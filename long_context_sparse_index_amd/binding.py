"""Thin ctypes binding of libdsa (include/dsa.h) for torch device tensors.

Argument marshalling only: every step of the layer runs in the HIP kernels of libdsa.so.
torch supplies device memory and the current stream.  The functions with an ``out``-style
signature write into caller tensors; the ``*_new`` helpers allocate outputs with torch first.
A missing library raises ``DSALibraryMissing``; a non-OK status raises ``DSAError``.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK = 0
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}
DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
DTYPE_F32 = 2


class DSALibraryMissing(RuntimeError):
    pass


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "dsa_status_string": ([_I32], ctypes.c_char_p),
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_abi_version": ([], ctypes.c_int),
    "dsa_index_scores": ([_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32, _I32,
                          _I32, _I32, _P], ctypes.c_int),
    "dsa_topk": ([_P, _I64, _I64, _I64, _I64, _I32, _P, _P, _SZ, _P], ctypes.c_int),
    "dsa_topk_workspace_bytes": ([_I64, _I64, _I32], _SZ),
    "dsa_sparse_attn_fwd": ([_P, _P, _I64, _P, _I64, _P, _I32, _P, _I32, _P, _I64, _I64, _I32,
                             _I32, _I32, _F32, _P], ctypes.c_int),
    "dsa_sparse_attn_bwd": ([_P, _P, _I64, _P, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P, _P,
                             _I64, _I64, _I32, _I32, _I32, _F32, _P, _SZ, _P], ctypes.c_int),
    "dsa_sparse_attn_bwd_workspace_bytes": ([_I64, _I32], _SZ),
    "dsa_sparse_attn_bwd_noalloc": ([_P, _P, _I64, _P, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P,
                                     _P, _I64, _I64, _I32, _I32, _I32, _F32, _P], ctypes.c_int),
    "dsa_sparse_attn_bwd_deterministic": ([_P, _P, _I64, _P, _I64, _P, _I32, _P, _I32, _P, _P,
                                           _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _F32, _P,
                                           _SZ, _P], ctypes.c_int),
    "dsa_sparse_attn_bwd_deterministic_workspace_bytes": ([_I64, _I32, _I64, _I32, _I32, _I32,
                                                           _I32], _SZ),
    "dsa_forward_chunked": ([_P, _I64, _P, _I64, _P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P,
                             _I64, _I32, _I32, _I32, _F32, _I32, _I64, _I64, _I64, _P, _I32, _P,
                             _P, _P, _SZ, _P], ctypes.c_int),
    "dsa_forward_chunked_workspace_bytes": ([_I64, _I64, _I32], _SZ),
    "dsa_index_topk": ([_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                        _P, _P, _SZ, _P], ctypes.c_int),
    "dsa_index_topk_workspace_bytes": ([_I64, _I64, _I32], _SZ),
    "dsa_pool_keys": ([_P, _I64, _P, _I64, _I32, _P, _I64, _P], ctypes.c_int),
}

_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libdsa.so once (raises DSALibraryMissing if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise DSALibraryMissing(
                    "%s is not built: run `python -m long_context_sparse_index_amd.build` "
                    "(there is no fallback path)" % path)
            lib = ctypes.CDLL(path)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
    return _lib


def exported_symbols():
    return sorted(_SIGNATURES)


def _check(status: int):
    if status != DSA_OK:
        msg = load_library().dsa_last_error().decode(errors="replace")
        raise DSAError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace the caller did not pass: allocated from torch's caching allocator on the
    current stream.  When the kernels go to another stream, the block is marked as used by
    that stream, so that the allocator does not hand it out again before they finish."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DTYPE_FP8_E4M3
    raise TypeError("indexer operands must be bfloat16 or e4m3 bytes, got %s" % t.dtype)


def _out_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("attention output must be float32 or bfloat16, got %s" % t.dtype)


def _row_stride(t: torch.Tensor) -> int:
    return t.stride(0)


def index_scores(q_idx, k_idx, w, scores, *, q_start: int = 0, n_pools: int | None = None,
                 accumulate: bool = False, stream=None):
    """scores[r, s] (+)= I[q_start + r, s] for s < V(q_start + r).

    q_idx [nq, h_i, d_i] (row stride may exceed h_i * d_i), k_idx [n_pools, d_i],
    w [h_i] (shared) or [nq, h_i] fp32, scores [nq, ld] fp32.
    """
    nq, h_i, d_i = q_idx.shape
    n_pools = k_idx.shape[0] if n_pools is None else n_pools
    assert q_idx.stride(2) == 1 and q_idx.stride(1) == d_i and k_idx.stride(1) == 1
    assert scores.stride(1) == 1 and scores.dtype == torch.float32 and w.dtype == torch.float32
    w_stride = 0 if w.dim() == 1 else w.stride(0)
    lib = load_library()
    _check(lib.dsa_index_scores(_ptr(q_idx), _row_stride(q_idx), _ptr(k_idx), k_idx.stride(0),
                                _ptr(w), w_stride, _ptr(scores), scores.stride(0), q_start, nq,
                                n_pools, h_i, d_i, _dtype_code(q_idx), int(accumulate),
                                _stream(stream)))
    return scores


def topk_workspace_bytes(nq: int, n_pools: int, k: int) -> int:
    return int(load_library().dsa_topk_workspace_bytes(nq, n_pools, k))


def topk(scores, idx, *, q_start: int, n_pools: int, ws=None, stream=None):
    """idx[r, :] = top-k visible pools of row r of scores (k = idx.shape[1]), -1 padded."""
    nq, k = idx.shape
    assert scores.shape[0] == nq and idx.dtype == torch.int32 and idx.is_contiguous()
    need = topk_workspace_bytes(nq, n_pools, k)
    if need and ws is None:
        ws = _workspace(need, scores.device, stream)
    lib = load_library()
    _check(lib.dsa_topk(_ptr(scores), scores.stride(0), q_start, nq, n_pools, k, _ptr(idx),
                        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                        _stream(stream)))
    return idx


def index_topk_workspace_bytes(nq: int, n_pools: int, k: int) -> int:
    return int(load_library().dsa_index_topk_workspace_bytes(nq, n_pools, k))


def index_topk(q_idx, k_idx, w, idx, *, q_start: int = 0, n_pools: int | None = None, ws=None,
               stream=None):
    """idx[r, :] = top-k of the indexer scores of query q_start + r (fused select; the same
    result as index_scores followed by topk)."""
    nq, h_i, d_i = q_idx.shape
    k = idx.shape[1]
    n_pools = k_idx.shape[0] if n_pools is None else n_pools
    assert q_idx.stride(2) == 1 and q_idx.stride(1) == d_i and k_idx.stride(1) == 1
    assert idx.dtype == torch.int32 and idx.is_contiguous() and idx.shape[0] == nq
    assert w.dtype == torch.float32
    w_stride = 0 if w.dim() == 1 else w.stride(0)
    if ws is None:
        ws = _workspace(index_topk_workspace_bytes(nq, n_pools, k), q_idx.device, stream)
    lib = load_library()
    _check(lib.dsa_index_topk(_ptr(q_idx), _row_stride(q_idx), _ptr(k_idx), k_idx.stride(0),
                              _ptr(w), w_stride, q_start, nq, n_pools, h_i, d_i,
                              _dtype_code(q_idx), k, _ptr(idx), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))
    return idx


def sparse_attn_fwd(q, kv, idx, o, lse, *, scale: float, d_v: int, v=None,
                    n_pools: int | None = None, stream=None):
    """o [nq, h, d_v] (fp32 or bf16), lse [nq, h] fp32 = sparse MQA attention over kv[idx]."""
    nq, h, d_qk = q.shape
    n_pools = kv.shape[0] if n_pools is None else n_pools
    assert q.is_contiguous() and idx.is_contiguous() and o.is_contiguous() and lse.is_contiguous()
    assert kv.stride(1) == 1 and (v is None or v.stride(1) == 1)
    lib = load_library()
    _check(lib.dsa_sparse_attn_fwd(_ptr(q), _ptr(kv), kv.stride(0), _ptr(v),
                                   0 if v is None else v.stride(0), _ptr(idx), idx.shape[1],
                                   _ptr(o), _out_code(o), _ptr(lse), nq, n_pools, h, d_qk, d_v,
                                   float(scale), _stream(stream)))
    return o, lse


def sparse_attn_bwd_workspace_bytes(nq: int, h: int) -> int:
    return int(load_library().dsa_sparse_attn_bwd_workspace_bytes(nq, h))


def sparse_attn_bwd(q, kv, idx, o, lse, d_o, dq, dkv, *, scale: float, d_v: int, v=None,
                    dv=None, n_pools: int | None = None, ws=None, stream=None):
    """dq (overwritten), dkv and dv (accumulated) of the sparse attention."""
    nq, h, d_qk = q.shape
    n_pools = kv.shape[0] if n_pools is None else n_pools
    for t in (q, idx, o, lse, d_o, dq, dkv):
        assert t.is_contiguous()
    need = sparse_attn_bwd_workspace_bytes(nq, h)
    if need and ws is None:
        ws = _workspace(need, q.device, stream)
    lib = load_library()
    _check(lib.dsa_sparse_attn_bwd(_ptr(q), _ptr(kv), kv.stride(0), _ptr(v),
                                   0 if v is None else v.stride(0), _ptr(idx), idx.shape[1],
                                   _ptr(o), _out_code(o), _ptr(lse), _ptr(d_o), _ptr(dq),
                                   _ptr(dkv), _ptr(dv),
                                   nq, n_pools, h, d_qk, d_v, float(scale), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)))
    return dq, dkv, dv


def sparse_attn_bwd_noalloc(q, kv, idx, o, lse, d_o, dq, dkv, *, scale: float, d_v: int,
                            v=None, dv=None, n_pools: int | None = None, stream=None):
    """As sparse_attn_bwd, with the library's static scratch instead of a workspace (the call
    allocates nothing; nq * h <= 2^22; overlapping calls on one GPU race)."""
    nq, h, d_qk = q.shape
    n_pools = kv.shape[0] if n_pools is None else n_pools
    for t in (q, idx, o, lse, d_o, dq, dkv):
        assert t.is_contiguous()
    lib = load_library()
    _check(lib.dsa_sparse_attn_bwd_noalloc(_ptr(q), _ptr(kv), kv.stride(0), _ptr(v),
                                           0 if v is None else v.stride(0), _ptr(idx),
                                           idx.shape[1], _ptr(o), _out_code(o), _ptr(lse),
                                           _ptr(d_o), _ptr(dq), _ptr(dkv), _ptr(dv), nq, n_pools,
                                           h, d_qk, d_v, float(scale), _stream(stream)))
    return dq, dkv, dv


def sparse_attn_bwd_deterministic_workspace_bytes(nq: int, h: int, n_pools: int, k: int,
                                                  d_qk: int, d_v: int, separate_dv: bool) -> int:
    return int(load_library().dsa_sparse_attn_bwd_deterministic_workspace_bytes(
        nq, h, n_pools, k, d_qk, d_v, int(separate_dv)))


def sparse_attn_bwd_deterministic(q, kv, idx, o, lse, d_o, dq, dkv, *, scale: float, d_v: int,
                                  v=None, dv=None, n_pools: int | None = None, ws=None,
                                  stream=None):
    """As sparse_attn_bwd, with run-to-run identical dq, dkv and dv (no atomics: staged dK/dV
    rows summed per pool in a fixed order)."""
    nq, h, d_qk = q.shape
    n_pools = kv.shape[0] if n_pools is None else n_pools
    for t in (q, idx, o, lse, d_o, dq, dkv):
        assert t.is_contiguous()
    if ws is None:
        need = sparse_attn_bwd_deterministic_workspace_bytes(nq, h, n_pools, idx.shape[1], d_qk,
                                                             d_v, dv is not None)
        ws = _workspace(need, q.device, stream)
    lib = load_library()
    _check(lib.dsa_sparse_attn_bwd_deterministic(
        _ptr(q), _ptr(kv), kv.stride(0), _ptr(v), 0 if v is None else v.stride(0), _ptr(idx),
        idx.shape[1], _ptr(o), _out_code(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dkv),
        _ptr(dv), nq, n_pools, h, d_qk, d_v, float(scale), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return dq, dkv, dv


def forward_chunked_workspace_bytes(n_pools: int, chunk: int, k: int) -> int:
    return int(load_library().dsa_forward_chunked_workspace_bytes(n_pools, chunk, k))


def forward_chunked(q_idx, k_idx, w, q, kv, o, lse, *, k: int, chunk: int, scale: float,
                    d_v: int, v=None, idx_out=None, ws=None, stream=None):
    """Whole DSA forward, one query chunk at a time (indexer -> top-k -> attention)."""
    n_tokens, h_i, d_i = q_idx.shape
    _, h, d_qk = q.shape
    n_pools = k_idx.shape[0]
    assert q.shape[0] == n_tokens and q.is_contiguous() and o.is_contiguous()
    w_stride = 0 if w.dim() == 1 else w.stride(0)
    need = forward_chunked_workspace_bytes(n_pools, chunk, k)
    if ws is None:
        ws = _workspace(need, q.device, stream)
    lib = load_library()
    _check(lib.dsa_forward_chunked(
        _ptr(q_idx), _row_stride(q_idx), _ptr(k_idx), k_idx.stride(0), _ptr(w), w_stride, h_i,
        d_i, _dtype_code(q_idx), _ptr(q), _ptr(kv), kv.stride(0), _ptr(v),
        0 if v is None else v.stride(0), h, d_qk, d_v, float(scale), k, n_tokens, n_pools,
        chunk, _ptr(o), _out_code(o), _ptr(lse), _ptr(idx_out), _ptr(ws),
        ws.numel() * ws.element_size(),
        _stream(stream)))
    return o, lse, idx_out


def pool_keys(x, gate, out, *, stream=None):
    """out[s] = softmax(gate[4s:4s+4]) . x[4s:4s+4] in bf16, for s < x.shape[0] // 4.

    x [n_tokens, d] bf16 (row stride may exceed d), gate [n_tokens] fp32,
    out [n_tokens // 4, d] bf16."""
    n, d = x.shape
    assert x.dtype == torch.bfloat16 and out.dtype == torch.bfloat16
    assert gate.dtype == torch.float32 and gate.is_contiguous() and gate.shape == (n,)
    assert x.stride(1) == 1 and out.stride(1) == 1 and out.shape == (n // 4, d)
    lib = load_library()
    _check(lib.dsa_pool_keys(_ptr(x), x.stride(0), _ptr(gate), n, d, _ptr(out), out.stride(0),
                             _stream(stream)))
    return out


# ----------------------------------------------------------------- allocating conveniences


def index_scores_new(q_idx, k_idx, w, *, q_start: int = 0, ld: int | None = None):
    nq = q_idx.shape[0]
    n_pools = k_idx.shape[0]
    ld = ((max(n_pools, 1) + 3) // 4) * 4 if ld is None else ld
    scores = torch.full((nq, ld), float("nan"), dtype=torch.float32, device=q_idx.device)
    return index_scores(q_idx, k_idx, w, scores, q_start=q_start, n_pools=n_pools)


def topk_new(scores, *, q_start: int, n_pools: int, k: int):
    idx = torch.empty((scores.shape[0], k), dtype=torch.int32, device=scores.device)
    return topk(scores, idx, q_start=q_start, n_pools=n_pools)


def sparse_attn_fwd_new(q, kv, idx, *, scale: float, d_v: int, v=None,
                        out_dtype=torch.float32):
    nq, h, _ = q.shape
    o = torch.empty((nq, h, d_v), dtype=out_dtype, device=q.device)
    lse = torch.empty((nq, h), dtype=torch.float32, device=q.device)
    return sparse_attn_fwd(q, kv, idx, o, lse, scale=scale, d_v=d_v, v=v)
