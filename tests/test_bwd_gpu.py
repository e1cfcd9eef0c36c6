"""The backward's HIP path against the fp64 oracle, element by element, on
seeded inputs the oracle finishes in seconds (several tiles, ragged tails,
GQA ratios, offsets, segments, empty rows), plus determinism and the split-key
(branch) usage.

The forward runs first on the GPU (its o and lse feed the backward, as in
training); the oracle recomputes everything from q, k, v and dout.

Bar (derived; the pages state none for the backward): per gradient tensor,
max|d - d_ref| <= TOL_BWD[dtype] * max(1, max|d_ref|), with TOL_BWD the
forward's bars (fp32 2e-5, bf16 2e-2, fp16 2.5e-3) read relative to the
tensor's scale; the floor of 1 (the scale of the N(0,1) inputs) covers tensors
whose exact value is 0, such as dq and dk when every row sees a single key.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_BWD, dout_dev, rel_err, seg_dev, to_dev

pytestmark = pytest.mark.gpu

BWD_DTYPES = ["f32", "bf16", "f16"]


def run_bwd(x, g):
    q, k, v = to_dev(x)
    do = dout_dev(g)
    kw = dict(causal=x.causal, q_offset=x.q_offset, seg_q=seg_dev(x.seg_q), seg_k=seg_dev(x.seg_k))
    o, lse = gqa.fwd(q, k, v, **kw)
    dq, dk, dv, delta = gqa.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv, delta


def check_bwd(x, label, seed=1):
    print("case:", label, flush=True)
    g = synth.Grad(x.q.shape, seed=seed, dtype=x.dtype)
    dq, dk, dv, delta = run_bwd(x, g)
    kw = dict(causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q, seg_k=x.seg_k)
    rq, rk, rv = oracle.bwd(x.q, x.k, x.v, g.values, **kw)
    o_ref, lse_ref = oracle.attn(x.q, x.k, x.v, **kw)
    d_ref = np.sum(g.values.astype(np.float64) * o_ref, axis=-1)
    errs = {"dq": rel_err(dq, rq), "dk": rel_err(dk, rk), "dv": rel_err(dv, rv)}
    # delta is a row dot product of dout and o: the forward's own bar on o, times sum |dout|
    ddel = np.abs(delta.cpu().numpy().astype(np.float64) - d_ref)
    bound = 4 * TOL_BWD[x.dtype] * np.sum(np.abs(g.values.astype(np.float64)), axis=-1)
    print("%s: rel max|d| dq %.3g dk %.3g dv %.3g; max|ddelta| %.3g" % (label, errs["dq"], errs["dk"], errs["dv"],
                                                                      ddel.max()), flush=True)
    for name, e in errs.items():
        assert e <= TOL_BWD[x.dtype], "%s: %s rel err %.3g" % (label, name, e)
    assert np.all(ddel <= bound), label + ": delta"
    # rows with no visible key get dq = 0 exactly; keys no row sees get dk = dv = 0 exactly
    empty = ~np.isfinite(lse_ref)
    if empty.any():
        assert np.all(dq.float().cpu().numpy()[empty] == 0.0), label + ": empty rows"
    unseen = np.all(rk == 0.0, axis=-1) & np.all(rv == 0.0, axis=-1)
    if unseen.any():
        assert np.all(dk.float().cpu().numpy()[unseen] == 0.0) and np.all(dv.float().cpu().numpy()[unseen] == 0.0)
    return dq, dk, dv


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("L", [1, 17, 64, 65, 300])
def test_bwd_ragged_lengths(dtype, L):
    check_bwd(synth.gqa(1, 16, 4, L, seed=100 + L, dtype=dtype), "bwd L%d %s" % (L, dtype))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_peaky_logits(dtype):
    x = synth.gqa(1, 16, 4, 256, seed=120, dtype=dtype)
    x = synth.Inputs(x.q * np.float32(4.0), x.k, x.v, dtype)
    check_bwd(x, "bwd L256 qscale4 " + dtype)


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_offset_batch_two(dtype):
    check_bwd(synth.gqa(2, 16, 4, 200, 333, seed=121, dtype=dtype, q_offset=133), "bwd B2 off133 " + dtype)


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_noncausal(dtype):
    check_bwd(synth.gqa(2, 16, 4, 150, 260, seed=122, dtype=dtype, causal=False), "bwd noncausal " + dtype)


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("rep", [1, 2, 3, 6, 8, 12, 16])
def test_bwd_group_sizes(dtype, rep):
    Hkv = 2 if rep >= 8 else 4
    check_bwd(synth.gqa(1, Hkv * rep, Hkv, 160, seed=130 + rep, dtype=dtype), "bwd rep%d %s" % (rep, dtype))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_packed_segments(dtype, causal):
    L = 900
    ids = synth.segment_ids(synth.segment_lengths(L, 60, 300, seed=140))[None]
    x = synth.gqa(1, 16, 4, L, seed=141, dtype=dtype, causal=causal)
    x.seg_q = x.seg_k = ids
    check_bwd(x, "bwd packed segments %s causal=%s" % (dtype, causal))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_random_segments_empty_rows(dtype, causal):
    L = 240
    rng = np.random.default_rng(150)
    sq = rng.integers(0, 3, size=(2, L)).astype(np.int32)
    sk = rng.integers(0, 3, size=(2, L)).astype(np.int32)
    sq[:, ::37] = 9  # matches no key: empty rows
    sk[:, 5::41] = 8  # matches no query: keys no row sees
    x = synth.gqa(2, 16, 4, L, seed=151, dtype=dtype, causal=causal)
    x.seg_q, x.seg_k = sq, sk
    check_bwd(x, "bwd random segments %s causal=%s" % (dtype, causal))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("packed", [True, False])
def test_bwd_extreme_segment_ids(dtype, packed):
    """Ids at the ends of int32 (the id scans' empty-range marks): packed runs
    of INT32_MIN, -1, 0, INT32_MAX, or those four at random; some query rows
    and some keys take an id the other side lacks."""
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    L = 300
    vals = np.array([lo, -1, 0, hi], dtype=np.int32)
    if packed:
        sk = np.repeat(vals, [70, 90, 40, 100])[None]
    else:
        sk = np.random.default_rng(152).choice(vals, size=(1, L)).astype(np.int32)
    sq = sk.copy()
    sq[0, 3::53] = 9
    sk = sk.copy()
    sk[0, 7::61] = 8
    x = synth.gqa(1, 16, 4, L, seed=153, dtype=dtype)
    x.seg_q, x.seg_k = sq, sk
    check_bwd(x, "bwd ids at the int32 ends, %s %s" % ("packed" if packed else "random", dtype))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_bwd_tiny_with_segments(dtype, L):
    """Fewer id entries than one 16-byte load: the id scan's small-array path."""
    x = synth.gqa(1, 16, 4, L, seed=60 + L, dtype=dtype)
    ids = np.array([[0, 0, 1, 1, 1][:L]], dtype=np.int32)
    x.seg_q = x.seg_k = ids
    check_bwd(x, "bwd L%d with ids %s" % (L, dtype))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_deterministic(dtype):
    x = synth.gqa(1, 16, 4, 700, seed=160, dtype=dtype)
    g = synth.Grad(x.q.shape, seed=161, dtype=dtype)
    a = run_bwd(x, g)
    b = run_bwd(x, g)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_split_keys_with_merged_forward(dtype):
    """A branch over a prefix of S keys plus its own causal keys: the forward of
    the two parts merged by gqa_attn_merge, then one backward per part with the
    merged o and lse; the parts' dq add up to the whole's and each part's dk, dv
    are the whole's slices."""
    S, m = 200, 96
    x = synth.gqa(1, 16, 4, m, S + m, seed=170, dtype=dtype, q_offset=S)
    g = synth.Grad(x.q.shape, seed=171, dtype=dtype)
    q, k, v = to_dev(x)
    do = dout_dev(g)
    kp, vp = k[:, :, :S].contiguous(), v[:, :, :S].contiguous()
    kb, vb = k[:, :, S:].contiguous(), v[:, :, S:].contiguous()
    o1, l1 = gqa.fwd(q, kp, vp, causal=False)
    o2, l2 = gqa.fwd(q, kb, vb, causal=True)
    o, lse = gqa.merge(o1, l1, o2, l2)
    dq1, dk1, dv1, _ = gqa.bwd(q, kp, vp, o, lse, do, causal=False)
    dq2, dk2, dv2, _ = gqa.bwd(q, kb, vb, o, lse, do, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(x.q, x.k, x.v, g.values, q_offset=S)
    dq = dq1.double() + dq2.double()
    dk = torch.cat([dk1, dk2], dim=2)
    dv = torch.cat([dv1, dv2], dim=2)
    for name, a, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = rel_err(a, r)
        print("split keys %s: %s rel err %.3g" % (dtype, name, e), flush=True)
        assert e <= TOL_BWD[dtype], name
