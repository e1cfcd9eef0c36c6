"""Context-parallel shards run one after another on one GPU.

A shard of a context-parallel split is an ordinary call. Rank r owns query
rows [a, b) and needs keys [0, b); it calls the forward (or the backward) with
Lq = b - a, Lk = b and q_offset = a. Causal balance uses a zig-zag
assignment: the rows are cut into 2N chunks, and rank r takes chunks r and
2N - 1 - r, so every rank gets one early and one late chunk. These tests run
each rank's calls on the one GPU and check the three ways of putting a split
together:

  * all-gather form (every rank holds all of K and V up to its rows): the
    shards' o and lse are the whole call's rows, bit for bit (every row's
    arithmetic depends only on that row and the key tiles, taken in the same
    order);
  * ring form (K and V pass around the ranks in N chunks): each rank's
    per-chunk partial results, combined with gqa_attn_merge, match the fp64
    oracle within the forward's bar;
  * backward: each shard's dq is the whole call's dq rows, bit for bit, and
    the shards' dk and dv, summed over ranks (the reduce-scatter of a real
    split), match the oracle within the backward's bar.

Which pages and sections this follows: the load-balanced context parallelism
of the maxtext pull request's configuration (zig-zag rows) and the ring
attention described beside it; the sums of key gradients over shards are the
chain rule, nothing more.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_BWD, compare, dout_dev, rel_err, to_dev


def zigzag_chunks(L: int, n_ranks: int):
    """Rank r's row ranges: chunks r and 2N - 1 - r of 2N near-equal chunks."""
    edges = [(L * i) // (2 * n_ranks) for i in range(2 * n_ranks + 1)]
    chunks = [(edges[i], edges[i + 1]) for i in range(2 * n_ranks)]
    return [[chunks[r], chunks[2 * n_ranks - 1 - r]] for r in range(n_ranks)]


def test_zigzag_chunks_cover_and_balance():
    """Every row belongs to exactly one rank. Under a causal mask each rank's
    visible (row, key) pairs are within 1% of the mean."""
    for L, n in ((1000, 4), (60926, 8), (30468, 2), (17, 2)):
        ranks = zigzag_chunks(L, n)
        owner = np.full(L, -1)
        for r, rng in enumerate(ranks):
            for a, b in rng:
                assert np.all(owner[a:b] == -1)
                owner[a:b] = r
        assert np.all(owner >= 0)
        if L >= 1000:
            pairs = [sum((b * (b + 1) - a * (a + 1)) // 2 for a, b in rng) for rng in ranks]
            assert max(pairs) <= 1.01 * np.mean(pairs) and min(pairs) >= 0.99 * np.mean(pairs), pairs


def _rows(t, a, b):
    return t[:, :, a:b].contiguous()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allgather_shards_equal_whole_call(dtype):
    L, N = 1000, 4
    print("case: all-gather shards %s L=%d N=%d" % (dtype, L, N), flush=True)
    x = synth.gqa(1, 16, 4, L, seed=300, dtype=dtype)
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v)
    for rng in zigzag_chunks(L, N):
        for a, b in rng:
            o_s, l_s = gqa.fwd(_rows(q, a, b), _rows(k, 0, b), _rows(v, 0, b), q_offset=a)
            torch.cuda.synchronize()
            assert torch.equal(o_s, o[:, :, a:b]), "o of rows [%d, %d)" % (a, b)
            assert torch.equal(l_s, lse[:, :, a:b]), "lse of rows [%d, %d)" % (a, b)


@pytest.mark.gpu
def test_ring_shards_match_oracle():
    """fp32 (a ring keeps its partial results in fp32). Rank r starts with its
    own key chunk and takes the others in ring order. A chunk wholly past a
    row range adds nothing and is skipped; one that starts inside the range
    is taken by the rows from its first key on (q_offset 0 relative to it)."""
    L, N = 1000, 4
    print("case: ring shards f32 L=%d N=%d" % (L, N), flush=True)
    x = synth.gqa(1, 16, 4, L, seed=301)
    q, k, v = to_dev(x)
    kv_edges = [(L * i) // N for i in range(N + 1)]
    o = torch.empty_like(q)
    lse = torch.empty(1, 16, L, device=q.device)
    for r, rng in enumerate(zigzag_chunks(L, N)):
        for a, b in rng:
            # the empty result (o = 0, lse = -inf) merges as the identity
            o_acc = torch.zeros_like(_rows(q, a, b))
            l_acc = torch.full((1, 16, b - a), float("-inf"), device=q.device)
            for step in range(N):
                c = (r - step) % N
                c0, c1 = kv_edges[c], kv_edges[c + 1]
                if c0 >= b:
                    continue  # every key of the chunk is past every row
                # rows before the chunk's first key see none of it; the rest start at lo
                lo = max(a, c0)
                part = gqa.fwd(_rows(q, lo, b), _rows(k, c0, c1), _rows(v, c0, c1), q_offset=lo - c0)
                m = gqa.merge(_rows(o_acc, lo - a, b - a), l_acc[:, :, lo - a:].contiguous(), part[0], part[1])
                o_acc[:, :, lo - a:], l_acc[:, :, lo - a:] = m
            o[:, :, a:b], lse[:, :, a:b] = o_acc, l_acc
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn(x.q, x.k, x.v)
    compare(o, lse, o_ref, lse_ref, "f32", label="ring N=%d" % N)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_shards(dtype):
    L, N = 600, 4
    print("case: backward shards %s L=%d N=%d" % (dtype, L, N), flush=True)
    x = synth.gqa(1, 16, 4, L, seed=302, dtype=dtype)
    g = synth.Grad(x.q.shape, seed=303, dtype=dtype)
    q, k, v = to_dev(x)
    do = dout_dev(g)
    o, lse = gqa.fwd(q, k, v)
    dq, _, _, _ = gqa.bwd(q, k, v, o, lse, do)
    dk_sum = torch.zeros(k.shape, dtype=torch.float64, device=k.device)
    dv_sum = torch.zeros_like(dk_sum)
    for rng in zigzag_chunks(L, N):
        for a, b in rng:
            dq_s, dk_s, dv_s, _ = gqa.bwd(_rows(q, a, b), _rows(k, 0, b), _rows(v, 0, b), _rows(o, a, b),
                                          lse[:, :, a:b].contiguous(), _rows(do, a, b), q_offset=a)
            torch.cuda.synchronize()
            assert torch.equal(dq_s, dq[:, :, a:b]), "dq of rows [%d, %d)" % (a, b)
            dk_sum[:, :, :b] += dk_s.double()
            dv_sum[:, :, :b] += dv_s.double()
    rq, rk, rv = oracle.bwd(x.q, x.k, x.v, g.values)
    for name, got, ref in (("dk", dk_sum, rk), ("dv", dv_sum, rv)):
        e = rel_err(got, ref)
        print("backward shards %s: %s summed over ranks, rel err %.3g" % (dtype, name, e), flush=True)
        assert e <= TOL_BWD[dtype], name
