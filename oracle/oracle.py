"""ctypes wrapper over the CPU oracle ``libdsa_oracle.so`` (test infrastructure only).

Arguments are numpy arrays: bf16 data travels as ``uint16`` bit patterns and OCP e4m3 data
as ``uint8`` bit patterns, so the oracle decodes every value itself.  The library is built
with g++ from ``dsa_oracle.cpp`` on first use (or by ``build()``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.cpp")
_LIB = os.path.join(_HERE, "libdsa_oracle.so")
_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_DBL = ctypes.c_double


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            lib.dsa_oracle_visible.restype = _I64
            lib.dsa_oracle_visible.argtypes = [_I64, _I64]
            lib.dsa_oracle_decode_bf16.argtypes = [_P, _P, _I64]
            lib.dsa_oracle_decode_e4m3.argtypes = [_P, _P, _I64]
            lib.dsa_oracle_index_scores.argtypes = [
                _P, _I64, _P, _I64, _P, _I64, _INT, _P, _I64, _I64, _INT, _INT, _P, _I64, _INT]
            lib.dsa_oracle_topk.argtypes = [_P, _I64, _P, _I64, _I64, _INT, _P, _INT]
            lib.dsa_oracle_sparse_attn_fwd.argtypes = [
                _P, _P, _I64, _P, _I64, _P, _INT, _I64, _I64, _INT, _INT, _INT, _DBL, _P, _P,
                _INT]
            lib.dsa_oracle_sparse_attn_bwd.argtypes = [
                _P, _P, _I64, _P, _I64, _P, _INT, _P, _I64, _I64, _INT, _INT, _INT, _DBL, _P,
                _P, _P, _INT]
            lib.dsa_oracle_round_bf16.argtypes = [_P, _P, _I64]
            lib.dsa_oracle_pool_keys.argtypes = [_P, _I64, _P, _I64, _INT, _P, _P, _INT]
            lib.dsa_oracle_sparse_attn_fwd_f64.argtypes = lib.dsa_oracle_sparse_attn_fwd.argtypes
            lib.dsa_oracle_sparse_attn_bwd_f64.argtypes = lib.dsa_oracle_sparse_attn_bwd.argtypes
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def visible(t: int, n_pools: int) -> int:
    return int(_load().dsa_oracle_visible(int(t), int(n_pools)))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().dsa_oracle_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def decode_e4m3(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().dsa_oracle_decode_e4m3(_ptr(bits), _ptr(out), bits.size)
    return out


def index_scores(q_bits, k_bits, w, rows, n_pools, *, threads: int = 0) -> np.ndarray:
    """Indexer scores of the listed rows.

    q_bits [nrows, h_i, d_i] uint16 (bf16) or uint8 (e4m3); k_bits [n_pools, d_i] same dtype;
    w float32 [h_i] (shared) or [nrows, h_i]; rows int64 absolute positions.
    Returns float32 [nrows, n_pools] with -inf beyond each row's visible prefix.
    """
    q_bits = np.ascontiguousarray(q_bits)
    k_bits = np.ascontiguousarray(k_bits)
    assert q_bits.dtype == k_bits.dtype and q_bits.dtype in (np.uint16, np.uint8)
    dtype = 0 if q_bits.dtype == np.uint16 else 1
    nrows, h_i, d_i = q_bits.shape
    assert k_bits.shape[1] == d_i and k_bits.shape[0] >= n_pools
    w = np.ascontiguousarray(w, dtype=np.float32)
    w_stride = 0 if w.ndim == 1 else w.shape[1]
    assert w.shape[-1] == h_i and (w.ndim == 1 or w.shape[0] == nrows)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.shape == (nrows,)
    out = np.empty((nrows, n_pools), dtype=np.float32)
    rc = _load().dsa_oracle_index_scores(
        _ptr(q_bits), h_i * d_i, _ptr(k_bits), d_i, _ptr(w), w_stride, dtype, _ptr(rows),
        nrows, n_pools, h_i, d_i, _ptr(out), n_pools, threads)
    _check(rc, "index_scores")
    return out


def topk(scores, rows, n_pools, k, *, threads: int = 0) -> np.ndarray:
    """Top-k pool indices (int32 [nrows, k], -1 padded) of each listed row of ``scores``."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    nrows, ld = scores.shape
    idx = np.empty((nrows, k), dtype=np.int32)
    rc = _load().dsa_oracle_topk(_ptr(scores), ld, _ptr(rows), nrows, n_pools, k, _ptr(idx),
                                 threads)
    _check(rc, "topk")
    return idx


def _attn_common(q_bits, kv_bits, v_bits, idx, d_v):
    # bf16 bit patterns travel as uint16; float64 arrays select the double entry points.
    dt = np.float64 if np.asarray(q_bits).dtype == np.float64 else np.uint16
    q_bits = np.ascontiguousarray(q_bits, dtype=dt)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=dt)
    v_bits = None if v_bits is None else np.ascontiguousarray(v_bits, dtype=dt)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nrows, h, d_qk = q_bits.shape
    if d_v is None:
        d_v = v_bits.shape[1] if v_bits is not None else d_qk
    return q_bits, kv_bits, v_bits, idx, nrows, h, d_qk, d_v


def sparse_attn_fwd(q_bits, kv_bits, idx, scale, *, v_bits=None, d_v=None, threads: int = 0):
    """Sparse MQA attention of the listed rows; returns (O float64 [nrows,h,d_v], LSE [nrows,h]).

    q_bits [nrows, h, d_qk] bf16 bits (or float64 values for the double entry point); kv_bits [n_pools, ld_kv] bf16 bits (keys are the first
    d_qk columns; V is the first d_v columns unless v_bits [n_pools, d_v] is given).
    """
    q_bits, kv_bits, v_bits, idx, nrows, h, d_qk, d_v = _attn_common(q_bits, kv_bits, v_bits,
                                                                    idx, d_v)
    n_pools, ld_kv = kv_bits.shape
    o = np.empty((nrows, h, d_v), dtype=np.float64)
    lse = np.empty((nrows, h), dtype=np.float64)
    lib = _load()
    fn = lib.dsa_oracle_sparse_attn_fwd_f64 if q_bits.dtype == np.float64 else \
        lib.dsa_oracle_sparse_attn_fwd
    rc = fn(
        _ptr(q_bits), _ptr(kv_bits), ld_kv, _ptr(v_bits),
        0 if v_bits is None else v_bits.shape[1], _ptr(idx), idx.shape[1], nrows, n_pools, h,
        d_qk, d_v, float(scale), _ptr(o), _ptr(lse), threads)
    _check(rc, "sparse_attn_fwd")
    return o, lse


def sparse_attn_bwd(q_bits, kv_bits, idx, do_bits, scale, *, v_bits=None, d_v=None,
                    threads: int = 0):
    """Gradients (dq [nrows,h,d_qk], dk [n_pools,d_qk], dv [n_pools,d_v] or None), float64.

    With v_bits None, V aliases kv[:, :d_v] and the V gradient is folded into dk[:, :d_v]
    (dv is returned as None).  Only the listed rows contribute to dk / dv.
    """
    q_bits, kv_bits, v_bits, idx, nrows, h, d_qk, d_v = _attn_common(q_bits, kv_bits, v_bits,
                                                                    idx, d_v)
    do_bits = np.ascontiguousarray(do_bits, dtype=q_bits.dtype)
    assert do_bits.shape == (nrows, h, d_v)
    n_pools, ld_kv = kv_bits.shape
    dq = np.empty((nrows, h, d_qk), dtype=np.float64)
    dk = np.empty((n_pools, d_qk), dtype=np.float64)
    dv = None if v_bits is None else np.empty((n_pools, d_v), dtype=np.float64)
    lib = _load()
    fn = lib.dsa_oracle_sparse_attn_bwd_f64 if q_bits.dtype == np.float64 else \
        lib.dsa_oracle_sparse_attn_bwd
    rc = fn(
        _ptr(q_bits), _ptr(kv_bits), ld_kv, _ptr(v_bits),
        0 if v_bits is None else v_bits.shape[1], _ptr(idx), idx.shape[1], _ptr(do_bits),
        nrows, n_pools, h, d_qk, d_v, float(scale), _ptr(dq), _ptr(dk), _ptr(dv), threads)
    _check(rc, "sparse_attn_bwd")
    return dq, dk, dv


def round_bf16(values) -> np.ndarray:
    """Nearest bf16 (ties to even) of each float64 value, as uint16 bit patterns."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint16)
    _load().dsa_oracle_round_bf16(_ptr(values), _ptr(out), values.size)
    return out


def pool_keys(x_bits, gate, *, threads: int = 0):
    """Pooled keys of floor(n / 4) pools: (float64 values before rounding, bf16 bits).

    x_bits [n, ld] uint16 bf16 bits (all ld columns pooled), gate float32 [n]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    n, d = x_bits.shape
    assert gate.shape == (n,)
    p = n // 4
    f64 = np.empty((p, d), dtype=np.float64)
    bits = np.empty((p, d), dtype=np.uint16)
    rc = _load().dsa_oracle_pool_keys(_ptr(x_bits), d, _ptr(gate), n, d, _ptr(f64), _ptr(bits),
                                      threads)
    _check(rc, "pool_keys")
    return f64, bits
