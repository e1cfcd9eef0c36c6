"""The id-range index of segment ids (gqa_attn_seg_index) and the indexed
forward and backward (gqa_attn_fwd_indexed, gqa_attn_bwd_indexed).

The index is checked entry by entry against numpy's min and max of each block
of 16 ids. The indexed calls classify the same tiles from the index that the
plain calls classify from the ids, so their outputs must equal the plain
calls' bit for bit; the plain calls are held to the oracle by the other test
files. Cases: packed ids (maxtext pull request 4929, the packed runs) and
unsorted ids from a small alphabet with ids no key has (empty rows), ragged
lengths, a query block past the keys' start (q_offset), batch 2, causal and
not, each index alone, and the long maps whose bits cover 2 tiles (more than
32,768 key tiles or row blocks).
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import synth
from gpu_util import dout_dev, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def index_ref(ids):
    """(min, max) of each block of 16 ids of each row (numpy)."""
    B, L = ids.shape
    n = (L + 15) // 16
    out = np.zeros((B, n, 2), dtype=np.int32)
    for j in range(n):
        blk = ids[:, 16 * j:16 * j + 16]
        out[:, j, 0] = blk.min(axis=1)
        out[:, j, 1] = blk.max(axis=1)
    return out


def ids_of(kind, B, L, seed):
    rng = np.random.default_rng(seed)
    if kind == "packed":
        rows = []
        for b in range(B):
            lens = synth.segment_lengths(L, max(1, L // 7), max(2, L // 3), seed=seed + b)
            rows.append(synth.segment_ids(lens))
        return np.stack(rows).astype(np.int32)
    # unsorted: ids from {0, 1, 2, 3} in runs of random length, so that some
    # tiles are single-id (full) and others mixed
    out = np.empty((B, L), dtype=np.int32)
    for b in range(B):
        x, row = 0, []
        while x < L:
            n = int(rng.integers(1, 200))
            row.append(np.full(n, rng.integers(0, 4), dtype=np.int32))
            x += n
        out[b] = np.concatenate(row)[:L]
    return out


@pytest.mark.parametrize("L", [1, 15, 16, 17, 1000, 4099])
@pytest.mark.parametrize("kind", ["packed", "unsorted"])
def test_index_values(L, kind):
    ids = ids_of(kind, 2, L, seed=L)
    ids[1, ::5] = np.iinfo(np.int32).min  # the int32 ends
    ids[0, ::7] = np.iinfo(np.int32).max
    got = gqa.seg_index(seg_dev(ids))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), index_ref(ids))


def bits_equal(a, b):
    """Equal bit patterns (NaN-free outputs; -0.0 and 0.0 kept apart)."""
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


FWD_CASES = [
    # (B, Hq, Hkv, Lq, Lk, q_offset, causal)
    (2, 8, 2, 1000, 1000, 0, True),
    (2, 8, 2, 1000, 1000, 0, False),
    (1, 16, 4, 200, 1300, 1100, True),
    (2, 4, 4, 333, 777, 0, False),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("kind", ["packed", "unsorted"])
@pytest.mark.parametrize("case", FWD_CASES)
@pytest.mark.parametrize("which", ["both", "k"])
def test_fwd_indexed_equals_plain(dtype, kind, case, which):
    B, Hq, Hkv, Lq, Lk, q_offset, causal = case
    print("case: fwd indexed", dtype, kind, case, which, flush=True)
    x = synth.gqa(B, Hq, Hkv, Lq, Lk, seed=40, dtype=dtype, q_offset=q_offset, causal=causal)
    ids_k = ids_of(kind, B, Lk, seed=41)
    ids_q = ids_k[:, q_offset:q_offset + Lq].copy() if q_offset + Lq <= Lk else ids_of(kind, B, Lq, seed=42)
    ids_q[:, ::37] = 9  # rows whose id no key has: empty
    q, k, v = to_dev(x)
    sq, sk = seg_dev(ids_q), seg_dev(ids_k)
    kw = dict(causal=causal, q_offset=q_offset, seg_q=sq, seg_k=sk)
    o0, l0 = gqa.fwd(q, k, v, **kw)
    qi = gqa.seg_index(sq) if which == "both" else None
    o1, l1 = gqa.fwd(q, k, v, seg_q_index=qi, seg_k_index=gqa.seg_index(sk), **kw)
    torch.cuda.synchronize()
    assert bits_equal(o0, o1) and bits_equal(l0, l1)


BWD_CASES = [
    (2, 8, 2, 700, 700, 0, True),
    (1, 16, 4, 200, 1300, 1100, True),
    (2, 4, 2, 500, 500, 0, False),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("kind", ["packed", "unsorted"])
@pytest.mark.parametrize("case", BWD_CASES)
@pytest.mark.parametrize("which", ["both", "q"])
def test_bwd_indexed_equals_plain(dtype, kind, case, which):
    B, Hq, Hkv, Lq, Lk, q_offset, causal = case
    print("case: bwd indexed", dtype, kind, case, which, flush=True)
    x = synth.gqa(B, Hq, Hkv, Lq, Lk, seed=43, dtype=dtype, q_offset=q_offset, causal=causal)
    g = synth.Grad(x.q.shape, seed=44, dtype=dtype)
    ids_k = ids_of(kind, B, Lk, seed=45)
    ids_q = ids_k[:, q_offset:q_offset + Lq].copy()
    ids_q[:, ::41] = 9
    q, k, v = to_dev(x)
    do = dout_dev(g)
    sq, sk = seg_dev(ids_q), seg_dev(ids_k)
    kw = dict(causal=causal, q_offset=q_offset, seg_q=sq, seg_k=sk)
    o, lse = gqa.fwd(q, k, v, **kw)
    r0 = gqa.bwd(q, k, v, o, lse, do, **kw)
    ki = gqa.seg_index(sk) if which == "both" else None
    r1 = gqa.bwd(q, k, v, o, lse, do, seg_q_index=gqa.seg_index(sq), seg_k_index=ki, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "delta"), r0, r1):
        assert bits_equal(a, b), name


def packed_ids(L):
    return synth.segment_ids(synth.segment_lengths(L, 2048, 32768, seed=1))


@pytest.mark.parametrize("dtype,Lk,Hq,Hkv", [("f32", 1100000, 4, 1), ("bf16", 2200000, 4, 1),
                                             ("f32", 600064, 16, 4)])
@pytest.mark.parametrize("kind", ["packed", "unsorted"])
def test_long_maps_fwd(dtype, Lk, Hq, Hkv, kind):
    """64 rows at the end of Lk keys: 18,752 key tiles (one per map bit) or
    34,375 (bits of 2 tiles), every workgroup's map spanning all of them."""
    Lq = 64
    print("case: fwd indexed long map", dtype, Lk, kind, flush=True)
    x = synth.gqa(1, Hq, Hkv, Lq, Lk, seed=46, dtype=dtype, q_offset=Lk - Lq)
    if kind == "packed":
        ids = packed_ids(Lk)
    else:
        ids = np.random.default_rng(47).integers(0, 3, size=Lk).astype(np.int32)
    sk = seg_dev(ids[None])
    sq = seg_dev(ids[None, Lk - Lq:])
    q, k, v = to_dev(x)
    kw = dict(causal=True, q_offset=Lk - Lq, seg_q=sq, seg_k=sk)
    o0, l0 = gqa.fwd(q, k, v, **kw)
    o1, l1 = gqa.fwd(q, k, v, seg_k_index=gqa.seg_index(sk), **kw)
    torch.cuda.synchronize()
    assert bits_equal(o0, o1) and bits_equal(l0, l1)


def test_long_row_map_bwd():
    """The dK/dV kernel's row map at L = 600,000 (37,500 16-row blocks of the
    fp32 kernel: bits of 2 blocks), packed segments, Hq = Hkv = 1."""
    L = 600000
    print("case: bwd indexed long row map fp32 L=%d" % L, flush=True)
    x = synth.gqa(1, 1, 1, L, seed=48, dtype="f32")
    g = synth.Grad(x.q.shape, seed=49, dtype="f32")
    q, k, v = to_dev(x)
    do = dout_dev(g)
    sid = seg_dev(packed_ids(L)[None])
    idx = gqa.seg_index(sid)
    o, lse = gqa.fwd(q, k, v, seg_q=sid, seg_k=sid)
    r0 = gqa.bwd(q, k, v, o, lse, do, seg_q=sid, seg_k=sid)
    r1 = gqa.bwd(q, k, v, o, lse, do, seg_q=sid, seg_k=sid, seg_q_index=idx, seg_k_index=idx)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "delta"), r0, r1):
        assert bits_equal(a, b), name


def test_packed_131072_bf16():
    """The packed bf16 workload (L = 131,072, segments of 2k-32k, seed 1):
    forward and backward through the index, equal to the plain calls."""
    L = 131072
    print("case: indexed packed bf16 L=%d" % L, flush=True)
    x = synth.gqa(1, 16, 4, L, seed=0, dtype="bf16")
    g = synth.Grad(x.q.shape, seed=1, dtype="bf16")
    q, k, v = to_dev(x)
    do = dout_dev(g)
    sid = seg_dev(packed_ids(L)[None])
    idx = gqa.seg_index(sid)
    kw = dict(seg_q=sid, seg_k=sid)
    o0, l0 = gqa.fwd(q, k, v, **kw)
    o1, l1 = gqa.fwd(q, k, v, seg_q_index=idx, seg_k_index=idx, **kw)
    r0 = gqa.bwd(q, k, v, o0, l0, do, **kw)
    r1 = gqa.bwd(q, k, v, o0, l0, do, seg_q_index=idx, seg_k_index=idx, **kw)
    torch.cuda.synchronize()
    assert bits_equal(o0, o1) and bits_equal(l0, l1)
    for name, a, b in zip(("dq", "dk", "dv", "delta"), r0, r1):
        assert bits_equal(a, b), name
