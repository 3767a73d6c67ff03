"""CPU oracle for the Lightning Indexer (score + top-k), loaded through ctypes.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library; the two meet only in the seeded inputs of ``workloads``.

The arithmetic lives in ``ds4idx_oracle.c`` (plain C, fp64, OpenMP over rows
and key blocks), ``ds4idx_kcache_oracle.c`` (the key-cache writer's E4M3
quantisation) and ``ds4idx_attn_oracle.c`` (sparse attention over the
selected positions); this wrapper only builds them with gcc and marshals
arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "ds4idx_oracle.c"), os.path.join(_HERE, "ds4idx_kcache_oracle.c"),
         os.path.join(_HERE, "ds4idx_attn_oracle.c")]
_LIB = os.path.join(_HERE, "libds4idx_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP)."""
    stale = not os.path.exists(_LIB) or \
        os.path.getmtime(_LIB) < max(os.path.getmtime(s) for s in _SRCS)
    if force or stale:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-Wall", "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        p, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.ds4o_e4m3_decode.argtypes = [i]
        lib.ds4o_e4m3_decode.restype = ctypes.c_double
        lib.ds4o_select.argtypes = [p, i, p, i, p, p, i, i, i, i, i, i64, i,
                                    p, i, p, p, p, p, i]
        lib.ds4o_select.restype = i
        lib.ds4o_score_pairs.argtypes = [p, i, p, i, p, p, i, i, i, i, i, i64,
                                         p, p, i64, p, i]
        lib.ds4o_score_pairs.restype = i
        lib.ds4o_e4m3_encode.argtypes = [ctypes.c_double]
        lib.ds4o_e4m3_encode.restype = i
        lib.ds4o_quantize_k.argtypes = [p, i, i64, i, p, p]
        lib.ds4o_quantize_k.restype = i
        lib.ds4o_sparse_attention.argtypes = [p, p, p, i, i, i, i, i, i, i, ctypes.c_double,
                                              p, i, p, p, i]
        lib.ds4o_sparse_attention.restype = i
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def e4m3_decode(code: int) -> float:
    return _load().ds4o_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    """Nearest OCP E4M3FN code to x (saturating at +-448, ties to the even code)."""
    return _load().ds4o_e4m3_encode(float(x))


def quantize_k(k: np.ndarray, dtype: int):
    """Per-token E4M3 quantisation of key vectors.

    k: [n, D] float32 values (dtype 0) or uint16 bf16 bit patterns (dtype 1).
    Returns (codes uint8 [n, D], scale float32 [n]).
    """
    k = np.ascontiguousarray(k, dtype=np.float32 if dtype == 0 else np.uint16)
    if k.ndim != 2:
        raise ValueError("k must be [n, D]")
    n, D = k.shape
    codes = np.empty((n, D), dtype=np.uint8)
    scale = np.empty(n, dtype=np.float32)
    if _load().ds4o_quantize_k(_ptr(k), int(dtype), n, D, _ptr(codes), _ptr(scale)) != 0:
        raise ValueError("oracle rejected the quantisation arguments")
    return codes, scale


def sparse_attention(q_bits, c_bits, idx, softmax_scale: float, d_v: int, rows=None,
                     nthreads: int = 0):
    """Sparse attention of the selected positions.

    q_bits [B,T,H,d_qk] and c_bits [B,S,d_qk] uint16 bf16 patterns, idx
    [B,T,k] int32 (entries outside [0,S) skipped). Returns (out float64
    [n,H,d_v], lse float64 [n,H]) for the flat rows b*T + t listed in rows
    (all rows by default)."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    c = np.ascontiguousarray(c_bits, dtype=np.uint16)
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    B, T, H, dqk = q.shape
    S = c.shape[1]
    k = ix.shape[2]
    rows = np.arange(B * T, dtype=np.int64) if rows is None else \
        np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), H, d_v), dtype=np.float64)
    lse = np.empty((len(rows), H), dtype=np.float64)
    used = _load().ds4o_sparse_attention(_ptr(q), _ptr(c), _ptr(ix), B, T, S, H, k, dqk, d_v,
                                         float(softmax_scale), _ptr(rows), len(rows), _ptr(out),
                                         _ptr(lse), nthreads)
    if used < 0:
        raise ValueError("oracle rejected the attention shape")
    return out, lse


def _problem_args(wl):
    q = np.ascontiguousarray(wl.q)
    k = np.ascontiguousarray(wl.k)
    ks = None if wl.k_scale is None else np.ascontiguousarray(wl.k_scale, dtype=np.float32)
    w = np.ascontiguousarray(wl.w, dtype=np.float32)
    keep = (q, k, ks, w)
    args = [_ptr(q), wl.q_dtype, _ptr(k), wl.k_dtype, _ptr(ks), _ptr(w),
            wl.B, wl.T, wl.S, wl.H, wl.D, wl.offset]
    return keep, args


def select(wl, rows=None, topk=None, nthreads: int = 0):
    """Oracle top-k for flat rows (b*T + t) of a workload.

    Returns (idx int32 [n, k] ascending/-1 padded, val float64 [n, k],
    kth float64 [n], rms float64 [n], threads_used).
    """
    lib = _load()
    topk = wl.topk if topk is None else topk
    rows = np.arange(wl.B * wl.T, dtype=np.int64) if rows is None else \
        np.ascontiguousarray(rows, dtype=np.int64)
    n = len(rows)
    idx = np.empty((n, topk), dtype=np.int32)
    val = np.empty((n, topk), dtype=np.float64)
    kth = np.empty(n, dtype=np.float64)
    rms = np.empty(n, dtype=np.float64)
    keep, args = _problem_args(wl)
    used = lib.ds4o_select(*args, topk, _ptr(rows), n, _ptr(idx), _ptr(val), _ptr(kth),
                           _ptr(rms), nthreads)
    if used < 0:
        raise ValueError("oracle rejected the problem shape")
    del keep
    return idx, val, kth, rms, used


def score_pairs(wl, rows, keys, nthreads: int = 0) -> np.ndarray:
    """Oracle scores at (row, key) pairs; NaN where the key is not visible."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    out = np.empty(len(rows), dtype=np.float64)
    keep, args = _problem_args(wl)
    if lib.ds4o_score_pairs(*args, _ptr(rows), _ptr(keys), len(rows), _ptr(out), nthreads) < 0:
        raise ValueError("oracle rejected the problem shape")
    del keep
    return out
