"""Segment skipping at lengths where the per-workgroup map of key tiles runs
long: past 16,384 tiles, and past 32,768 tiles, where one bit of the map
covers a group of 2 (or more) tiles. The scale of the packed run whose
per-block metadata outgrew its memory at 1,048,576 tokens (maxtext pull
request 4929, problem statement and "Effect").

Query blocks sit at the end of the key sequence (q_offset = Lk - Lq), so
every workgroup's causal range spans the whole map; the oracle checks every
output row. Packed ids are segments of uniform-random length 2k-32k (seed 1);
the unsorted case draws ids from {0, 1, 2} and gives some rows an id no key
has (empty rows). Bars as elsewhere: max|do| <= 2e-5 (fp32) / 2e-2 (bf16),
max|dlse| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_BWD, compare, dout_dev, rel_err, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def tail_block(Hq, Hkv, Lq, Lk, dtype, seed, ids_k, causal=True):
    x = synth.gqa(1, Hq, Hkv, Lq, Lk, seed=seed, dtype=dtype, q_offset=Lk - Lq, causal=causal)
    x.seg_k = ids_k[None]
    x.seg_q = ids_k[None, Lk - Lq:]
    return x


def check_all_rows(x, label, split=False):
    print("case:", label, flush=True)
    q, k, v = to_dev(x)
    kw = dict(causal=x.causal, q_offset=x.q_offset, seg_q=seg_dev(x.seg_q), seg_k=seg_dev(x.seg_k))
    o, lse = (gqa.fwd_split if split else gqa.fwd)(q, k, v, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q, seg_k=x.seg_k)
    compare(o, lse, o_ref, l_ref, x.dtype, label=label)


def packed_ids(L):
    return synth.segment_ids(synth.segment_lengths(L, 2048, 32768, seed=1))


@pytest.mark.parametrize("split", [False, True])
def test_fp32_past_16384_tiles(split):
    """fp32 (32-key tiles), 64 rows at q_offset = 600,000 over 600,064 keys:
    18,752 tiles, one per map bit; also through the split-KV launch."""
    Lk, Lq = 600064, 64
    x = tail_block(16, 4, Lq, Lk, "f32", 30, packed_ids(Lk))
    check_all_rows(x, "fp32 Lk=%d packed%s" % (Lk, " split-KV" if split else ""), split=split)


@pytest.mark.parametrize("causal", [True, False])
def test_fp32_grouped_map_packed(causal):
    """fp32, Lk = 1,100,000 (34,375 tiles: map bits of 2 tiles), Hq = 4 over
    Hkv = 1, 64 rows at the end; causal within segments, and bidirectional
    within segments."""
    Lk, Lq = 1100000, 64
    x = tail_block(4, 1, Lq, Lk, "f32", 31, packed_ids(Lk), causal=causal)
    check_all_rows(x, "fp32 Lk=%d packed causal=%s" % (Lk, causal))


def test_fp32_grouped_map_unsorted_ids():
    """Ids drawn from {0, 1, 2} at Lk = 1,100,000: every group is visible and
    none is full; rows whose id (7) no key has are empty."""
    Lk, Lq = 1100000, 64
    rng = np.random.default_rng(32)
    ids = rng.integers(0, 3, size=Lk).astype(np.int32)
    x = tail_block(4, 1, Lq, Lk, "f32", 33, ids)
    x.seg_q = x.seg_q.copy()
    x.seg_q[0, ::9] = 7
    check_all_rows(x, "fp32 Lk=%d random ids" % Lk)


def test_bf16_grouped_map_packed():
    """bf16 (64-key tiles), Lk = 2,200,000: 34,375 tiles, map bits of 2 tiles."""
    Lk, Lq = 2200000, 64
    x = tail_block(4, 1, Lq, Lk, "bf16", 34, packed_ids(Lk))
    check_all_rows(x, "bf16 Lk=%d packed" % Lk)


def test_bwd_fp32_grouped_row_map():
    """The backward's dK/dV kernel maps 16-row blocks of queries: at
    L = 600,000 (37,500 row blocks, map bits of 2 blocks; Hq = Hkv = 1) with
    packed segments, dk and dv of every key of the two shortest segments and
    of the last 16 keys of every segment, and dq of sampled rows, against the
    oracle."""
    L = 600000
    lens = synth.segment_lengths(L, 2048, 32768, seed=1)
    ids = synth.segment_ids(lens)
    bounds = synth.segment_bounds(lens)
    label = "bwd fp32 L=%d, %d packed segments, Hq = Hkv = 1" % (L, len(lens))
    print("case:", label, flush=True)
    x = synth.gqa(1, 1, 1, L, seed=35, dtype="f32")
    g = synth.Grad(x.q.shape, seed=36, dtype="f32")
    q, k, v = to_dev(x)
    do = dout_dev(g)
    sid = torch.from_numpy(ids[None]).to(q.device)
    o, lse = gqa.fwd(q, k, v, seg_q=sid, seg_k=sid)
    dq, dk, dv, _ = gqa.bwd(q, k, v, o, lse, do, seg_q=sid, seg_k=sid)
    torch.cuda.synchronize()
    short = sorted(bounds, key=lambda ab: ab[1] - ab[0])[:2]
    keys = np.unique(np.concatenate([np.arange(a, b) for a, b in short] +
                                    [np.arange(b - 16, b) for _, b in bounds])).astype(np.int64)
    rows = synth.sample_rows(L, bounds=bounds, n_random=64, upto=256, tail=256)
    seg = ids[None]
    rq = oracle.bwd_dq(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, rows=rows)
    rk, rv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, keys=keys)
    kk, rr = torch.from_numpy(keys).to(dk.device), torch.from_numpy(rows).to(dq.device)
    e = {"dq": rel_err(dq[:, :, rr], rq), "dk": rel_err(dk[:, :, kk], rk), "dv": rel_err(dv[:, :, kk], rv)}
    print("%s: %d rows, %d keys: rel max|d| dq %.3g dk %.3g dv %.3g" % (label, len(rows), len(keys), e["dq"],
                                                                       e["dk"], e["dv"]), flush=True)
    for name, err in e.items():
        assert err <= TOL_BWD["f32"], "%s: %s %.3g" % (label, name, err)
