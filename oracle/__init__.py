"""fp64 CPU oracle for exact causal grouped-query attention (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.

The arithmetic lives in ``oracle_attn.c`` (plain C, fp64, OpenMP over rows);
this module only loads it with ctypes and marshals numpy arrays. Inputs are
fp32 arrays; bf16 inputs must be widened to fp32 first (exact).

Sources, cited by page title and section:
  * kev pull request 202, "Why fp32 fell to the L x L kernel": the math path
    materialises a 16 x L x L fp32 score matrix per attention layer; "The change":
    the memory-efficient kernel gives the same attention with memory linear in L,
    and K/V repetition per query head stands in for grouped-query attention.
  * system1-omni issue 27, "The closest planned or implemented model": 16 query
    heads share 4 key/value heads, head_dim 256; "Three differences from Cua-S1
    that matter", item 3: one state, then a branch per question whose positions
    restart at the state length.
  * maxtext pull request 4929 (problem statement and review): separate query and
    key/value segment ids; constant ids make the segmented and non-segmented
    kernels agree.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_attn.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def compile_source(src: str, out: str, werror: bool = True) -> str:
    """Compile an oracle source file with gcc (-O2, no fast-math, OpenMP)."""
    tmp = out + ".tmp%d" % os.getpid()
    warn = ["-Wall", "-Werror"] if werror else ["-w"]
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99"] + warn +
                          [src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile the oracle library next to its source if it is missing or stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_attn.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p,
                                ctypes.c_int, p, i64, p, p, ctypes.c_int]
    lib.oracle_attn.restype = ctypes.c_int
    lib.oracle_attn_weights.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p,
                                        ctypes.c_int, i64, i64, i64, p]
    lib.oracle_attn_weights.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [p, p, p, p, i64, i64, p, p]
    lib.oracle_merge.restype = None
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_attn_bwd_dq.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p,
                                       ctypes.c_int, p, i64, p, ctypes.c_int]
    lib.oracle_attn_bwd_dq.restype = ctypes.c_int
    lib.oracle_attn_bwd_dkdv.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p,
                                         ctypes.c_int, p, i64, p, p, ctypes.c_int]
    lib.oracle_attn_bwd_dkdv.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = open_library(_LIB)
    return _lib


class Oracle:
    """The oracle's entry points bound to one compiled library (the default one,
    or another build of the same source)."""

    def __init__(self, lib=None):
        self._lib = lib

    def _l(self):
        return self._lib if self._lib is not None else _load()

    def attn(self, q, k, v, *, causal=True, q_offset=0, seg_q=None, seg_k=None, rows=None, nthreads=0):
        return _attn(self._l(), q, k, v, causal=causal, q_offset=q_offset, seg_q=seg_q,
                     seg_k=seg_k, rows=rows, nthreads=nthreads)

    def weights(self, q, k, v, b, h, i, *, causal=True, q_offset=0, seg_q=None, seg_k=None):
        return _weights(self._l(), q, k, v, b, h, i, causal=causal, q_offset=q_offset,
                        seg_q=seg_q, seg_k=seg_k)

    def merge(self, o1, lse1, o2, lse2):
        return _merge(self._l(), o1, lse1, o2, lse2)

    def bwd_dq(self, q, k, v, dout, *, causal=True, q_offset=0, seg_q=None, seg_k=None, rows=None,
               nthreads=0):
        return _bwd_dq(self._l(), q, k, v, dout, causal=causal, q_offset=q_offset, seg_q=seg_q,
                       seg_k=seg_k, rows=rows, nthreads=nthreads)

    def bwd_dkdv(self, q, k, v, dout, *, causal=True, q_offset=0, seg_q=None, seg_k=None, keys=None,
                 nthreads=0):
        return _bwd_dkdv(self._l(), q, k, v, dout, causal=causal, q_offset=q_offset, seg_q=seg_q,
                         seg_k=seg_k, keys=keys, nthreads=nthreads)

    def bwd(self, q, k, v, dout, **kw):
        """dq [B,Hq,Lq,D], dk and dv [B,Hkv,Lk,D] over all rows and keys (fp64)."""
        dq = self.bwd_dq(q, k, v, dout, **kw)
        dk, dv = self.bwd_dkdv(q, k, v, dout, **kw)
        return dq, dk, dv




def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(q, k, v, seg_q, seg_k):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Lq,D], k and v [B,Hkv,Lk,D]")
    B, Hq, Lq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or Hq % k.shape[1]:
        raise ValueError("shape mismatch between q and k/v")
    if (seg_q is None) != (seg_k is None):
        raise ValueError("give both segment-id arrays or neither")
    if seg_q is not None:
        seg_q = np.ascontiguousarray(seg_q, dtype=np.int32).reshape(B, Lq)
        seg_k = np.ascontiguousarray(seg_k, dtype=np.int32).reshape(B, k.shape[2])
    return seg_q, seg_k


def _attn(lib, q, k, v, *, causal=True, q_offset=0, seg_q=None, seg_k=None, rows=None, nthreads=0):
    """Exact attention forward in fp64.

    q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] (fp32 values); seg ids [B,Lq]/[B,Lk] int32 or None.
    Key j is visible to query i iff (not causal or j <= q_offset + i) and the
    segment ids agree. rows: optional query indices to evaluate (each output row
    depends only on its own query row). Returns o [B,Hq,R,D] and lse [B,Hq,R]
    (natural log of the sum of exp over the scaled visible scores), fp64.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    seg_q, seg_k = _check(q, k, v, seg_q, seg_k)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    rows_arr = None
    nrows = Lq
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    o = np.empty((B, Hq, nrows, D), dtype=np.float64)
    lse = np.empty((B, Hq, nrows), dtype=np.float64)
    rc = lib.oracle_attn(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Lq, Lk, D, int(q_offset),
                             _ptr(seg_q), _ptr(seg_k), int(bool(causal)), _ptr(rows_arr), nrows,
                             _ptr(o), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    return o, lse


def _weights(lib, q, k, v, b, h, i, *, causal=True, q_offset=0, seg_q=None, seg_k=None):
    """Softmax weights of row (b, h, i) over all Lk keys (0 where invisible), fp64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    seg_q, seg_k = _check(q, k, v, seg_q, seg_k)
    B, Hq, Lq, D = q.shape
    w = np.empty(k.shape[2], dtype=np.float64)
    rc = lib.oracle_attn_weights(_ptr(q), _ptr(k), _ptr(v), B, Hq, k.shape[1], Lq, k.shape[2], D,
                                     int(q_offset), _ptr(seg_q), _ptr(seg_k), int(bool(causal)),
                                     int(b), int(h), int(i), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_attn_weights rejected its arguments")
    return w


def _merge(lib, o1, lse1, o2, lse2):
    """Combine results over two disjoint key sets from their log-sum-exps (fp64)."""
    o1 = np.ascontiguousarray(o1, dtype=np.float64)
    o2 = np.ascontiguousarray(o2, dtype=np.float64)
    lse1 = np.ascontiguousarray(lse1, dtype=np.float64)
    lse2 = np.ascontiguousarray(lse2, dtype=np.float64)
    if o1.shape != o2.shape or lse1.shape != lse2.shape or o1.shape[:-1] != lse1.shape:
        raise ValueError("merge operands disagree in shape")
    D = o1.shape[-1]
    rows = lse1.size
    o = np.empty_like(o1)
    lse = np.empty_like(lse1)
    lib.oracle_merge(_ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), rows, D, _ptr(o), _ptr(lse))
    return o, lse


def _bwd_dq(lib, q, k, v, dout, *, causal=True, q_offset=0, seg_q=None, seg_k=None, rows=None, nthreads=0):
    """Gradient with respect to q of a loss whose gradient with respect to o is
    `dout` [B,Hq,Lq,D], for all rows or the given query indices; fp64
    [B,Hq,R,D]."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    seg_q, seg_k = _check(q, k, v, seg_q, seg_k)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, Hq, Lq, D = q.shape
    rows_arr, nrows = None, Lq
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    dq = np.empty((B, Hq, nrows, D), dtype=np.float64)
    rc = lib.oracle_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Hq, k.shape[1], Lq, k.shape[2], D,
                                int(q_offset), _ptr(seg_q), _ptr(seg_k), int(bool(causal)), _ptr(rows_arr),
                                nrows, _ptr(dq), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_dq rejected its arguments")
    return dq


def _bwd_dkdv(lib, q, k, v, dout, *, causal=True, q_offset=0, seg_q=None, seg_k=None, keys=None, nthreads=0):
    """Gradients with respect to k and v (summed over the query heads that share
    each key/value head), for all keys or the given key indices; fp64
    [B,Hkv,K,D] each."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    seg_q, seg_k = _check(q, k, v, seg_q, seg_k)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    keys_arr, nkeys = None, Lk
    if keys is not None:
        keys_arr = np.ascontiguousarray(keys, dtype=np.int64)
        nkeys = keys_arr.size
    dk = np.empty((B, Hkv, nkeys, D), dtype=np.float64)
    dv = np.empty((B, Hkv, nkeys, D), dtype=np.float64)
    rc = lib.oracle_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Hq, Hkv, Lq, Lk, D,
                                  int(q_offset), _ptr(seg_q), _ptr(seg_k), int(bool(causal)), _ptr(keys_arr),
                                  nkeys, _ptr(dk), _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_dkdv rejected its arguments")
    return dk, dv


_default = Oracle()
attn = _default.attn
weights = _default.weights
merge = _default.merge
bwd_dq = _default.bwd_dq
bwd_dkdv = _default.bwd_dkdv
bwd = _default.bwd


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# ---- memory arithmetic of the math path (kev pull request 202) -------------

def math_path_bytes(L: int, Hq: int = 16, elem_bytes: int = 4, Lk: int | None = None) -> int:
    """Bytes of one materialised score matrix: Hq x Lq x Lk elements.

    kev pull request 202, "Why fp32 fell to the L x L kernel": a 16 x L x L fp32
    matrix, 69 GB at 32k and 275 GB at 64k per attention layer.
    """
    Lk = L if Lk is None else Lk
    return int(Hq) * int(L) * int(Lk) * int(elem_bytes)


def repeat_kv_bytes(Hq: int, L: int, D: int, elem_bytes: int = 4) -> int:
    """Bytes of K (or V) repeated to every query head: Hq x L x D elements.

    kev pull request 202, "The change": 1 GiB each at 64k for Kev-9B.
    """
    return int(Hq) * int(L) * int(D) * int(elem_bytes)


def visible_pairs(Lq, Lk, *, causal=True, q_offset=0, seg_q=None, seg_k=None):
    """Number of visible (query, key) pairs of one head, counted from the
    visibility definition itself (dense boolean mask; small inputs only)."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        vis &= j <= q_offset + i
    if seg_q is not None:
        vis &= np.asarray(seg_q).reshape(Lq, 1) == np.asarray(seg_k).reshape(1, Lk)
    return int(vis.sum())
