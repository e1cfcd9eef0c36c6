"""The allocation-free split-KV entry point (gqa_attn_fwd_split_noalloc)
against gqa_attn_fwd_split with a caller workspace, through the C ABI: the same
kernels on the same split, so the outputs must agree bit for bit (beyond the
forward's bars, which they also meet against the oracle). Two calls in a row,
the second on a smaller input, so the second reuses the static scratch that
the first filled; and the call allocates no device memory."""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import compare, to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": gqa.GQA_F32, "bf16": gqa.GQA_BF16, "f16": gqa.GQA_F16}


def both(x, n_split):
    q, k, v = to_dev(x)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if n_split == 0:
        # the count the allocation-free call picks: the recommended one, lowered to fit the scratch
        n_split = min(gqa.split_count(B, Hq, Hkv, Lq, Lk, DT[x.dtype]),
                      max(1, gqa.NOALLOC_SCRATCH_BYTES // (B * Hq * Lq * (D + 1) * 4)))
        call_split = 0
    else:
        call_split = n_split
    o_ref, l_ref = gqa.fwd_split(q, k, v, causal=x.causal, q_offset=x.q_offset, n_split=n_split)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    gqa.fwd_split_noalloc(q, k, v, o, lse, causal=x.causal, q_offset=x.q_offset, n_split=call_split)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    return o, lse, o_ref, l_ref, free0 - free1


def test_noalloc_matches_split_twice_second_smaller():
    # 1: 16 decode rows over 60,926 bf16 keys, 64 splits (16.8 MB of partials)
    x1 = synth.gqa(1, 16, 4, 16, 60926, seed=40, dtype="bf16", q_offset=60926 - 16)
    print("case: noalloc bf16 Lq=16 Lk=60926 n_split=64", flush=True)
    o, lse, o_ref, l_ref, grown = both(x1, 64)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert grown == 0
    rows = np.arange(16)
    ro, rl = oracle.attn(x1.q, x1.k, x1.v, q_offset=x1.q_offset, rows=rows)
    compare(o, lse, ro, rl, "bf16", label="noalloc call 1")
    # 2: a smaller call: 5 rows over 9,000 fp32 keys, the library's split count
    x2 = synth.gqa(1, 16, 4, 5, 9000, seed=41, dtype="f32", q_offset=9000 - 5)
    print("case: noalloc f32 Lq=5 Lk=9000 n_split=0", flush=True)
    o, lse, o_ref, l_ref, grown = both(x2, 0)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert grown == 0
    ro, rl = oracle.attn(x2.q, x2.k, x2.v, q_offset=x2.q_offset)
    compare(o, lse, ro, rl, "f32", label="noalloc call 2")


def test_noalloc_segments_and_branch():
    # one 256-row fp32 branch over a 30,468-token prefix (+ its own 256 keys), with
    # packed ids on a bf16 call after it: the scratch holds each call's own partials
    S, m = 30468, 256
    x = synth.gqa(1, 16, 4, m, S + m, seed=42, dtype="f32", q_offset=S)
    print("case: noalloc f32 branch S=30468 m=256 n_split=8", flush=True)
    o, lse, o_ref, l_ref, grown = both(x, 8)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref) and grown == 0
    L = 3000
    lens = synth.segment_lengths(L, 100, 900, seed=43)
    ids = torch.from_numpy(synth.segment_ids(lens)[None]).to("cuda:0")
    y = synth.gqa(1, 16, 4, 64, L, seed=44, dtype="bf16", q_offset=L - 64)
    q, k, v = to_dev(y)
    sq = ids[:, L - 64:].contiguous()
    o_ref, l_ref = gqa.fwd_split(q, k, v, q_offset=L - 64, seg_q=sq, seg_k=ids, n_split=6)
    o = torch.empty_like(q)
    lse = torch.empty((1, 16, 64), dtype=torch.float32, device=q.device)
    gqa.fwd_split_noalloc(q, k, v, o, lse, q_offset=L - 64, seg_q=sq, seg_k=ids, n_split=6)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
