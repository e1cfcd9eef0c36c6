"""Short query blocks (decoding: fewer than 32 positions) with no segment
ids: the launches the packed-row decode kernels serve (fp32, and 16-bit
inputs), through gqa_attn_fwd and gqa_attn_fwd_split, against the fp64
oracle, every output row.

The kernels pack the query rows of one KV head (n_rep heads x Lq positions)
into blocks of 64, 16 per wave (the fp32 kernel: groups of at most 16 or 32
rows take one block of 16 or 32 rows, whose waves each own a quarter or a
half of d), so the cases vary what that packing meets (16 rows: (4, 4),
(2, 8), (8, 2); 17-32 rows: (4, 5), (4, 8), (1, 17), (1, 31), (16, 2)):
group sizes 1..16, 3, 6, 12 and 64, and Lq 1..31 (a wave's 16 rows spanning several heads, a
last block cut short, several blocks per head), causal rows whose visible
keys end before, at and past the key sequence's end, ragged key counts (16-key
tiles in fp32, 32-key tiles in 16-bit; a ring of 4 tiles in flight), B = 2,
and split counts from 1 to more splits than tiles.

Bars as for the forward: max|do| <= 2e-5 (fp32) / 2e-2 (bf16) / 2.5e-3 (fp16),
max|dlse| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_O, compare, to_dev

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16"]


def check(x, label, n_split=None, unsplit=True, tol_scale=1.0):
    """Oracle check of gqa_attn_fwd_split (at n_split; None = the library's
    count) and, if asked, of gqa_attn_fwd on the same inputs (tol_scale as in
    gpu_util.compare)."""
    print("case:", label, "n_split", n_split, flush=True)
    q, k, v = to_dev(x)
    kw = dict(causal=x.causal, q_offset=x.q_offset)
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset)
    o, lse = gqa.fwd_split(q, k, v, n_split=n_split, **kw)
    torch.cuda.synchronize()
    compare(o, lse, o_ref, l_ref, x.dtype, label="%s split %s" % (label, n_split), tol_scale=tol_scale)
    if unsplit:
        o1, l1 = gqa.fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        compare(o1, l1, o_ref, l_ref, x.dtype, label="%s unsplit" % label, tol_scale=tol_scale)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("rep,Lq", [(4, 16), (4, 1), (4, 4), (4, 5), (4, 8), (4, 31), (1, 3), (1, 17), (1, 31),
                                    (2, 7), (2, 8), (8, 2), (8, 16), (16, 2), (16, 31), (3, 1), (3, 11),
                                    (6, 5), (12, 3), (64, 1), (64, 31)])
def test_group_sizes_and_lengths(dtype, rep, Lq):
    """Decode rows at the end of a ragged key sequence (2,017 keys: 63 full
    tiles and one of a single key)."""
    Hkv, Lk = 2, 2017
    x = synth.gqa(1, Hkv * rep, Hkv, Lq, Lk, seed=300 + 37 * rep + Lq, dtype=dtype, q_offset=Lk - Lq)
    check(x, "rep%d Lq=%d Lk=%d %s" % (rep, Lq, Lk, dtype), n_split=11)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("q_offset", [0, 1000, 2000, 2017, 2040, 1 << 40])
def test_causal_ends(dtype, q_offset):
    """Rows at q_offset + 0..15 over 2,017 keys: visible keys end inside the
    sequence (the tail is never read), at its end, or past it (every key
    visible; q_offset far beyond 2^31 included)."""
    Lq, Lk = 16, 2017
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=320, dtype=dtype, q_offset=q_offset)
    check(x, "q_offset=%d %s" % (q_offset, dtype), n_split=5)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("Lk", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 129])
def test_short_key_sequences(dtype, Lk):
    """About one ring of tiles (4 x 16 keys in fp32, 4 x 32 in 16-bit) and
    less, including a single key; splits past the last tile are empty and
    merge as nothing."""
    Lq = 3
    x = synth.gqa(1, 8, 2, Lq, Lk, seed=330 + Lk, dtype=dtype, q_offset=max(Lk - Lq, 0))
    check(x, "Lk=%d %s" % (Lk, dtype), n_split=4)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("Lq", [9, 6, 1])
def test_noncausal_batch_two(dtype, Lq):
    """B = 2, not causal; 36, 24 and 4 rows per KV head (in fp32 one, two and
    four parts of d)."""
    x = synth.gqa(2, 16, 4, Lq, 3001, seed=340 + Lq, dtype=dtype, causal=False)
    check(x, "B2 noncausal Lq=%d Lk=3001 %s" % (Lq, dtype), n_split=13)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("n_split", [1, 2, 64, 1000])
def test_split_counts(dtype, n_split):
    """The same 16 rows over 4,500 keys at 1, 2, 64 and 1,000 requested splits
    (141 tiles of 32 keys, 282 of 16: 1,000 requests give one-tile ranges)."""
    x = synth.gqa(1, 16, 4, 16, 4500, seed=350, dtype=dtype, q_offset=4500 - 16)
    check(x, "splits %d %s" % (n_split, dtype), n_split=n_split, unsplit=n_split == 1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_peaky_scores_rescale(dtype):
    """Query rows scaled by 6 (logit standard deviation about 6): the running
    max moves often, and the lazy rescale of O, l (and lr) is exercised. The
    fp32 bars scale with the logits (gpu_util.compare)."""
    x0 = synth.gqa(1, 16, 4, 16, 3000, seed=360, dtype=dtype, q_offset=3000 - 16)
    x = synth.Inputs(x0.q * np.float32(6.0), x0.k, x0.v, dtype, q_offset=3000 - 16)
    check(x, "peaky " + dtype, n_split=6, tol_scale=6.0 if dtype == "f32" else 1.0)


@pytest.mark.parametrize("dtype,Lq", [("f32", 16), ("f32", 6), ("f32", 1), ("bf16", 16), ("bf16", 1)])
def test_full_size_decode_every_row(dtype, Lq):
    """16, 6 or 1 decode positions (64, 24 or 4 rows per KV head: in fp32 one,
    two or four parts of d per row block) after 60,926 keys, at the library's
    split count (the measured decode workloads): every row of every head."""
    Lk = 60926
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=370 + Lq, dtype=dtype, q_offset=Lk - Lq)
    check(x, "full size decode %s Lq=%d" % (dtype, Lq), n_split=None, unsplit=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeat_calls_identical(dtype):
    """The kernel's result does not depend on what an earlier call left in LDS
    or in the workspace: two calls on different inputs, then the first again,
    give the first result bit for bit."""
    xa = synth.gqa(1, 16, 4, 16, 2500, seed=380, dtype=dtype, q_offset=2484)
    xb = synth.gqa(1, 16, 4, 16, 2500, seed=381, dtype=dtype, q_offset=2484)
    qa, ka, va = to_dev(xa)
    qb, kb, vb = to_dev(xb)
    oa, la = gqa.fwd_split(qa, ka, va, q_offset=2484, n_split=9)
    gqa.fwd_split(qb, kb, vb, q_offset=2484, n_split=9)
    oa2, la2 = gqa.fwd_split(qa, ka, va, q_offset=2484, n_split=9)
    torch.cuda.synchronize()
    assert torch.equal(oa, oa2) and torch.equal(la, la2)
