"""Split-KV forward (gqa_attn_fwd_split) against the fp64 oracle, element by
element, for short query blocks over long key sequences: decode rows after a
long state, one branch over a shared prefix, segments, ragged key tails, and
split counts from 1 to many, in every dtype; and against gqa_attn_fwd.

Bars as for the forward: max|do| <= 2e-5 (fp32) / 2e-2 (bf16) / 2.5e-3 (fp16),
max|dlse| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_O, compare, seg_dev, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]


def check_split(x, label, n_split=None):
    print("case:", label, "n_split", n_split, flush=True)
    q, k, v = to_dev(x)
    kw = dict(causal=x.causal, q_offset=x.q_offset, seg_q=seg_dev(x.seg_q), seg_k=seg_dev(x.seg_k))
    o, lse = gqa.fwd_split(q, k, v, n_split=n_split, **kw)
    o1, l1 = gqa.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q, seg_k=x.seg_k)
    compare(o, lse, o_ref, l_ref, x.dtype, label="%s split %s" % (label, n_split))
    # and the unsplit call agrees with it within the same bar
    assert float((o.float() - o1.float()).abs().max()) <= TOL_O[x.dtype]
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(lse))
    assert float((lse[fin] - l1[fin]).abs().max()) <= 1e-4 if fin.any() else True


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("Lq,n_split", [(1, None), (1, 2), (4, 7), (17, 64), (33, 1000)])
def test_decode_rows_after_long_state(dtype, Lq, n_split):
    Lk = 5000
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=200 + Lq, dtype=dtype, q_offset=Lk - Lq)
    check_split(x, "decode Lq=%d Lk=%d %s" % (Lq, Lk, dtype), n_split)


@pytest.mark.parametrize("dtype", DTYPES)
def test_branch_over_prefix(dtype):
    S, m = 3000, 256
    x = synth.gqa(1, 16, 4, m, S + m, seed=210, dtype=dtype, q_offset=S)
    check_split(x, "branch S=%d m=%d %s" % (S, m, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_noncausal_batch_and_ragged_keys(dtype):
    x = synth.gqa(2, 16, 4, 40, 3333, seed=220, dtype=dtype, causal=False)
    check_split(x, "B2 noncausal Lk=3333 " + dtype, 9)


@pytest.mark.parametrize("dtype", DTYPES)
def test_other_group_sizes(dtype):
    for rep in (1, 3, 6, 16):
        Hkv = 2 if rep == 16 else 4
        x = synth.gqa(1, Hkv * rep, Hkv, 8, 2100, seed=230 + rep, dtype=dtype, q_offset=2092)
        check_split(x, "rep%d %s" % (rep, dtype), 5)


@pytest.mark.parametrize("dtype", DTYPES)
def test_segments_with_empty_rows(dtype):
    Lq, Lk = 24, 4000
    rng = np.random.default_rng(240)
    sk = np.repeat(np.arange(4, dtype=np.int32), 1000)[None]
    sq = rng.integers(0, 4, size=(1, Lq)).astype(np.int32)
    sq[0, ::5] = 9  # no key has this id: empty rows (o = 0, lse = -inf)
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=241, dtype=dtype, causal=False)
    x.seg_q, x.seg_k = sq, sk
    check_split(x, "segments " + dtype, 6)


def test_split_count_one_is_the_forward():
    x = synth.gqa(1, 16, 4, 64, 640, seed=250, dtype="bf16")
    q, k, v = to_dev(x)
    o1, l1 = gqa.fwd(q, k, v)
    o2, l2 = gqa.fwd_split(q, k, v, n_split=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,Lq,Lk", [("bf16", 16, 60926), ("f32", 256, 30468 + 256)])
def test_full_size(dtype, Lq, Lk):
    # decode rows over the 64k state (bf16) and one 256-row branch over the 30k prefix (fp32)
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=260, dtype=dtype, q_offset=Lk - Lq)
    check_split(x, "full size Lq=%d Lk=%d %s" % (Lq, Lk, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_scores_far_below_zero(dtype):
    """All scores near -2,000, so each row's max is near -167 in log2 units.
    Every split but the last ends before a key tile that exists; that tile
    must stay unscored. Scoring the zeros of its copy would lift the running
    max to 0 and rescale O and l by about 2^-167, which underflows to zero.

    Bars: the fp32 rounding of these score sums is up to 1.2e-3, about 36
    times that of N(0,1) inputs (sum |q_d k_d| is about 2,000 against about
    160), so the fp32 bars are scaled by 64. For the 16-bit types the rounding
    of P dominates the output error; their bars are scaled by 2, for the
    score rounding that reaches lse."""
    x0 = synth.gqa(1, 16, 4, 16, 1000, seed=230, causal=False)
    q = np.abs(x0.q) + np.float32(2.0)
    k = -(np.abs(x0.k) + np.float32(2.0))
    x = synth.Inputs(q, k, x0.v, dtype, causal=False)
    print("case: scores far below zero", dtype, flush=True)
    qd, kd, vd = to_dev(x)
    o, lse = gqa.fwd_split(qd, kd, vd, causal=False, n_split=4)
    o1, l1 = gqa.fwd(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=False)
    scale = 64.0 if dtype == "f32" else 2.0
    compare(o, lse, o_ref, l_ref, dtype, label="far below zero, split 4", tol_scale=scale)
    compare(o1, l1, o_ref, l_ref, dtype, label="far below zero, unsplit", tol_scale=scale)
