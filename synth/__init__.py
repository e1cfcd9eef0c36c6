"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws random tensors, rounds
fp32 draws to bf16 or fp16 bit patterns, lays out segment ids and picks sample
rows.
Both the HIP path and the CPU oracle receive exactly the bytes made here.

Workload shapes stand in for the pages' inputs (post-RoPE activations of Kev
models on long documents, and a packed pretraining run), which are not
available: 16 query heads over 4 key/value heads, head_dim 256 (system1-omni
issue 27, "The closest planned or implemented model"), at the state lengths
kev pull request 202 measures in "Measurements" (15,231 / 30,468 / 60,926).
"""
from __future__ import annotations

import numpy as np

HQ, HKV, D = 16, 4, 256


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to fp16 bit patterns, round-to-nearest-even (numpy's
    conversion; values stay well inside the fp16 range here)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen fp16 bit patterns to fp32 (exact)."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


_ROUND = {"bf16": (f32_to_bf16_bits, bf16_bits_to_f32), "f16": (f32_to_f16_bits, f16_bits_to_f32)}


class Inputs:
    """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] as fp32 values (already exact in the
    16-bit type when dtype is bf16 or f16) plus, for those, the raw bit patterns
    the device receives."""

    def __init__(self, q, k, v, dtype, seg_q=None, seg_k=None, q_offset=0, causal=True):
        self.q, self.k, self.v = q, k, v
        self.dtype = dtype
        self.seg_q, self.seg_k = seg_q, seg_k
        self.q_offset, self.causal = q_offset, causal
        if dtype in _ROUND:
            to_bits, to_f32 = _ROUND[dtype]
            self.q_bits = to_bits(q)
            self.k_bits = to_bits(k)
            self.v_bits = to_bits(v)
            self.q = to_f32(self.q_bits)
            self.k = to_f32(self.k_bits)
            self.v = to_f32(self.v_bits)
        elif dtype != "f32":
            raise ValueError("dtype must be 'f32', 'bf16' or 'f16'")


def gqa(B=1, Hq=HQ, Hkv=HKV, Lq=512, Lk=None, Dh=D, *, seed=0, scale=1.0, dtype="f32",
        q_offset=0, causal=True) -> Inputs:
    """Q, K, V drawn i.i.d. N(0,1) in fp32 from default_rng(seed), in the order
    Q, K, V, each multiplied by `scale` (a power of two keeps this exact)."""
    Lk = Lq if Lk is None else Lk
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Lq, Dh), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Lk, Dh), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Lk, Dh), dtype=np.float32)
    if scale != 1.0:
        q *= np.float32(scale)
        k *= np.float32(scale)
        v *= np.float32(scale)
    return Inputs(q, k, v, dtype, q_offset=q_offset, causal=causal)


class Grad:
    """An upstream gradient dout [B,Hq,Lq,D] drawn i.i.d. N(0,1) in fp32 from
    default_rng(seed); for bf16/f16, rounded to nearest even, with the bit
    patterns the device receives in `bits`."""

    def __init__(self, shape, seed=0, dtype="f32"):
        d = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
        self.dtype = dtype
        self.bits = None
        if dtype in _ROUND:
            to_bits, to_f32 = _ROUND[dtype]
            self.bits = to_bits(d)
            d = to_f32(self.bits)
        elif dtype != "f32":
            raise ValueError("dtype must be 'f32', 'bf16' or 'f16'")
        self.values = d


def segment_lengths(total: int, lo: int = 2048, hi: int = 32768, seed: int = 1) -> list[int]:
    """Uniform-random segment lengths in [lo, hi] from default_rng(seed), drawn
    until they cover `total`; the last one is cut to fit (it may fall below lo)."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def segment_ids(lengths) -> np.ndarray:
    """Packed ids 0, 1, 2, ... in order, one run per segment (int32)."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))


def segment_bounds(lengths) -> list[tuple[int, int]]:
    out, a = [], 0
    for n in lengths:
        out.append((a, a + n))
        a += n
    return out


class Branch:
    """Shared-prefix branch workload: a prefix (state) of S tokens and n branches
    of m query tokens each whose positions start at S (system1-omni issue 27,
    "Three differences from Cua-S1 that matter", item 3).

    Tensors, drawn in this order from default_rng(seed):
      q_b [n,Hq,m,D]  branch queries
      k_p, v_p [Hkv,S,D]  prefix keys/values
      k_b, v_b [n,Hkv,m,D]  each branch's own keys/values
    """

    def __init__(self, S=30468, n=40, m=256, Hq=HQ, Hkv=HKV, Dh=D, *, seed=0, dtype="f32"):
        rng = np.random.default_rng(seed)
        self.S, self.n, self.m = S, n, m
        self.q_b = rng.standard_normal((n, Hq, m, Dh), dtype=np.float32)
        self.k_p = rng.standard_normal((Hkv, S, Dh), dtype=np.float32)
        self.v_p = rng.standard_normal((Hkv, S, Dh), dtype=np.float32)
        self.k_b = rng.standard_normal((n, Hkv, m, Dh), dtype=np.float32)
        self.v_b = rng.standard_normal((n, Hkv, m, Dh), dtype=np.float32)
        self.dtype = dtype
        if dtype == "bf16":
            for name in ("q_b", "k_p", "v_p", "k_b", "v_b"):
                setattr(self, name, bf16_bits_to_f32(f32_to_bf16_bits(getattr(self, name))))

    def branch_layout(self):
        """Rows of all branches side by side in one sequence of n*m rows:
        q [1,Hq,n*m,D] and branch ids [n*m] (int32) for the suffix part."""
        n, m = self.n, self.m
        Hq, Dh = self.q_b.shape[1], self.q_b.shape[3]
        q = np.ascontiguousarray(self.q_b.transpose(1, 0, 2, 3).reshape(1, Hq, n * m, Dh))
        k = np.ascontiguousarray(self.k_b.transpose(1, 0, 2, 3).reshape(1, -1, n * m, Dh))
        v = np.ascontiguousarray(self.v_b.transpose(1, 0, 2, 3).reshape(1, -1, n * m, Dh))
        ids = np.repeat(np.arange(n, dtype=np.int32), m)
        return q, k, v, ids


def sample_rows(L: int, *, bounds=None, n_random: int = 512, seed: int = 2, upto: int = 4096,
                tail: int = 4096) -> np.ndarray:
    """Sorted, distinct query rows to check at large L: the first and last rows,
    every multiple of 16/32/64/128 below `upto` and within the last `tail` rows,
    each with its neighbours, the first and last rows (and neighbours) of each
    (start, end) in `bounds`, and `n_random` rows from default_rng(seed)."""
    s = {0, 1, 2, L - 2, L - 1}
    for step in (16, 32, 64, 128):
        for x in range(0, min(upto, L), step):
            s.update((x - 1, x, x + 1))
        for x in range(max(0, L - tail) // step * step, L + 1, step):
            s.update((x - 1, x, x + 1))
    for a, b in (bounds or []):
        s.update((a - 1, a, a + 1, b - 2, b - 1, b))
    rng = np.random.default_rng(seed)
    s.update(int(x) for x in rng.integers(0, L, size=n_random))
    return np.array(sorted(x for x in s if 0 <= x < L), dtype=np.int64)
