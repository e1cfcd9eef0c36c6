"""Algorithmic work and traffic of one attention forward (host-side accounting).

FLOPs count 4*D per visible (query, key) pair per query head: 2*D for the
score dot product and 2*D for the weighted sum of V. Softmax exponentials are
not counted, and neither is masked or skipped work. Bytes count the compulsory
HBM traffic: Q, K, V (and segment ids) read once, O and lse written once.
"""
from __future__ import annotations

import numpy as np


def visible_pairs(Lq: int, Lk: int, *, causal: bool = True, q_offset: int = 0, seg_q=None, seg_k=None) -> int:
    """Visible (query, key) pairs of one head and one batch row."""
    i = np.arange(Lq, dtype=np.int64)
    lim = np.minimum(Lk, q_offset + i + 1) if causal else np.full(Lq, Lk, dtype=np.int64)
    if seg_q is None:
        return int(lim.sum())
    seg_q = np.asarray(seg_q).reshape(-1)
    seg_k = np.asarray(seg_k).reshape(-1)
    total = 0
    order = np.argsort(seg_k, kind="stable")
    ks = seg_k[order]
    for s in np.unique(seg_q):
        pos = order[np.searchsorted(ks, s, "left"):np.searchsorted(ks, s, "right")]  # key positions with id s (sorted)
        rows = np.nonzero(seg_q == s)[0]
        total += int(np.searchsorted(pos, lim[rows], "left").sum())
    return total


def visible_pairs_rows(rows, Lk: int, *, causal: bool = True, q_offset: int = 0, seg_q=None, seg_k=None) -> int:
    """Visible (query, key) pairs of one head over the query rows `rows` only
    (seg_q: the ids of all query rows; seg_k: of all keys)."""
    rows = np.asarray(rows, dtype=np.int64)
    lim = np.minimum(Lk, q_offset + rows + 1) if causal else np.full(len(rows), Lk, dtype=np.int64)
    if seg_q is None:
        return int(lim.sum())
    sq = np.asarray(seg_q).reshape(-1)[rows]
    sk = np.asarray(seg_k).reshape(-1)
    order = np.argsort(sk, kind="stable")
    ks = sk[order]
    lo = np.searchsorted(ks, sq, "left")
    hi = np.searchsorted(ks, sq, "right")
    total = 0
    for a, b, l in zip(lo, hi, lim):
        total += int(np.searchsorted(order[a:b], l, "left"))  # positions with the row's id below its limit
    return total


def flops(B, Hq, Lq, Lk, D, **kw) -> int:
    """Algorithmic FLOPs of the forward (same pair count in every batch row unless
    per-batch segment ids are given as [B, L] arrays)."""
    seg_q, seg_k = kw.pop("seg_q", None), kw.pop("seg_k", None)
    if seg_q is None:
        return 4 * D * Hq * B * visible_pairs(Lq, Lk, **kw)
    seg_q, seg_k = np.asarray(seg_q).reshape(B, Lq), np.asarray(seg_k).reshape(B, Lk)
    return 4 * D * Hq * sum(visible_pairs(Lq, Lk, seg_q=seg_q[b], seg_k=seg_k[b], **kw) for b in range(B))


def hbm_bytes(B, Hq, Hkv, Lq, Lk, D, elem_bytes, segments=False) -> int:
    """Compulsory HBM bytes: read Q, K, V (+ ids), write O and the fp32 lse."""
    b = (2 * Hq * Lq + 2 * Hkv * Lk) * D * elem_bytes + 4 * Hq * Lq
    if segments:
        b += 4 * (Lq + Lk)
    return B * b


def bwd_flops(B, Hq, Lq, Lk, D, **kw) -> int:
    """Algorithmic FLOPs of the backward: 10 D per visible (query, key) pair per
    query head, the five products of the gradient (the scores recomputed, dP,
    dV, dQ, dK; 2 D each), i.e. 2.5 times the forward. The products that the
    two-kernel split computes twice (the scores and dP, once per kernel) are
    not counted."""
    return flops(B, Hq, Lq, Lk, D, **kw) // 4 * 10


def bwd_exec_flops(B, Hq, Lq, Lk, D, **kw) -> int:
    """Product FLOPs the backward kernels execute on visible pairs: 6 D in the
    dQ kernel (scores, dP, dQ) and 8 D in the dK/dV kernel (scores, dP, dV, dK)."""
    return flops(B, Hq, Lq, Lk, D, **kw) // 4 * 14


def bwd_hbm_bytes(B, Hq, Hkv, Lq, Lk, D, elem_bytes, segments=False) -> int:
    """Compulsory HBM bytes of the backward: read Q, K, V, O, dO and the lse,
    write dQ, dK, dV, write and read back delta (fp32)."""
    b = (4 * Hq * Lq + 4 * Hkv * Lk) * D * elem_bytes + 12 * Hq * Lq
    if segments:
        b += 4 * (Lq + Lk)
    return B * b


def score_matrix_bytes(Hq: int, Lq: int, Lk: int, elem_bytes: int = 4) -> int:
    """Bytes of the Hq x Lq x Lk score matrix an L x L (math-path) attention materialises."""
    return int(Hq) * int(Lq) * int(Lk) * int(elem_bytes)


# MI355X published peaks (dense): bf16 MFMA 2.5 PFLOP/s, fp32 157.3 TFLOP/s, HBM 8 TB/s
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6}
PEAK_HBM_GBS = 8000.0
