"""Seeded random shapes through gqa_attn_fwd and gqa_attn_fwd_split against the
fp64 oracle, every output row.

Each case draws, from a seed of its own: the input type, batch 1-2, 1-3
key/value heads, a group of 1, 2, 3, 4, 6, 8, 12 or 16 query heads per
key/value head, query and key lengths from 1 to a few hundred (half the cases
below the decode bound of 32 positions, half of those without ids), causal or
not, q_offset at the end of the keys, at 0 or anywhere up to 500, segment ids absent, packed (sorted runs over the
position axis) or random over 3 values, and a split count from 1 to more than
the key tiles. So the cases reach the long-block kernels, both decode
kernels with each of their modes, the segment paths, ragged tiles, empty
rows and empty key ranges in mixtures the structured tests do not enumerate.
A failure prints the case's seed and draw. Bars as for the forward. The
backward takes its own draws (lengths up to 200) through gqa_attn_bwd, with
the bars and exact-zero checks of test_bwd_gpu.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import compare, seg_dev, to_dev
from test_bwd_gpu import check_bwd

pytestmark = pytest.mark.gpu

CASES = 240
BWD_CASES = 80


def draw(case):
    rng = np.random.default_rng(7000 + case)
    dtype = ("f32", "bf16", "f16")[case % 3]
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 4))
    rep = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    short = (case // 3) % 2 == 0  # half the cases below the decode bound, for each type
    Lq = int(rng.integers(1, 32)) if short else int(rng.integers(1, 300))
    Lk = int(rng.integers(1, 400))
    causal = bool(rng.integers(0, 2))
    where = int(rng.integers(0, 3))
    q_offset = max(Lk - Lq, 0) if where == 0 else 0 if where == 1 else int(rng.integers(0, 500))
    seg = int(rng.integers(0, 3))  # 0: none, 1: packed runs, 2: random ids
    if short and (case // 6) % 2 == 0:
        seg = 0  # the decode kernels serve calls without ids
    n_split = int(rng.choice([1, 2, 5, 17, 64]))
    return dict(dtype=dtype, B=B, Hkv=Hkv, rep=rep, Lq=Lq, Lk=Lk, causal=causal, q_offset=q_offset, where=where,
                seg=seg, n_split=n_split, seed=7000 + case, rng=rng)


def segment_arrays(d):
    """seg_q [B, Lq], seg_k [B, Lk] for the draw (None for no ids)."""
    rng, B, Lq, Lk, q0 = d["rng"], d["B"], d["Lq"], d["Lk"], d["q_offset"]
    if d["seg"] == 0:
        return None, None
    if d["seg"] == 1:
        # packed: sorted runs over positions 0 .. max(Lk, q0 + Lq); queries take
        # the id of their own position
        P = max(Lk, q0 + Lq)
        sq = np.empty((B, Lq), np.int32)
        sk = np.empty((B, Lk), np.int32)
        for b in range(B):
            n_cuts = min(P - 1, int(rng.integers(0, 6)))
            cuts = np.sort(rng.choice(np.arange(1, P), size=n_cuts, replace=False)) if n_cuts > 0 else []
            ids = np.zeros(P, np.int32)
            for c in cuts:
                ids[c:] += 1
            sk[b] = ids[:Lk]
            sq[b] = ids[q0:q0 + Lq]
        return sq, sk
    return (rng.integers(0, 3, size=(B, Lq)).astype(np.int32), rng.integers(0, 3, size=(B, Lk)).astype(np.int32))


@pytest.mark.parametrize("case", range(CASES))
def test_random_shape(case):
    d = draw(case)
    label = "case %d: %s" % (case, {k: v for k, v in d.items() if k != "rng"})
    print(label, flush=True)
    x = synth.gqa(d["B"], d["Hkv"] * d["rep"], d["Hkv"], d["Lq"], d["Lk"], seed=d["seed"], dtype=d["dtype"],
                  q_offset=d["q_offset"], causal=d["causal"])
    x.seg_q, x.seg_k = segment_arrays(d)
    q, k, v = to_dev(x)
    kw = dict(causal=x.causal, q_offset=x.q_offset, seg_q=seg_dev(x.seg_q), seg_k=seg_dev(x.seg_k))
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q, seg_k=x.seg_k)
    o, lse = gqa.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, x.dtype, label=label + " fwd")
    o2, l2 = gqa.fwd_split(q, k, v, n_split=d["n_split"], **kw)
    torch.cuda.synchronize()
    compare(o2, l2, o_ref, l_ref, x.dtype, label=label + " split")


@pytest.mark.parametrize("case", range(BWD_CASES))
def test_random_shape_backward(case):
    d = draw(10000 + case)
    d["Lq"] = 1 + d["Lq"] % 200
    d["Lk"] = 1 + d["Lk"] % 200
    d["q_offset"] = (max(d["Lk"] - d["Lq"], 0) if d["where"] == 0 else 0 if d["where"] == 1 else
                     min(d["q_offset"], 300))
    label = "bwd case %d: %s" % (case, {k: v for k, v in d.items() if k not in ("rng", "n_split")})
    x = synth.gqa(d["B"], d["Hkv"] * d["rep"], d["Hkv"], d["Lq"], d["Lk"], seed=d["seed"], dtype=d["dtype"],
                  q_offset=d["q_offset"], causal=d["causal"])
    x.seg_q, x.seg_k = segment_arrays(d)
    check_bwd(x, label, seed=d["seed"] + 1)
