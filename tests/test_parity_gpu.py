"""HIP path against the fp64 oracle, element by element, on seeded inputs the
oracle finishes in seconds (several key tiles, ragged tails, every code path).

Bars: max|do| <= 2e-5 (fp32) / 2e-2 (bf16) / 2.5e-3 (fp16, derived), max|dlse| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import DEV, TOL_LSE, TOL_O, compare, dev_tensor, run, seg_dev, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]


def check(x, label, rows=None, tol_scale=1.0):
    print("case:", label, flush=True)
    o, lse = run(x)
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q,
                               seg_k=x.seg_k, rows=rows)
    return compare(o, lse, o_ref, l_ref, x.dtype, rows=rows, label=label, tol_scale=tol_scale)


def test_small_config_fp32_scaled():
    # B=1, Hq=16, Hkv=4, D=256, L=512; Q/K/V N(0,1) x 1/sqrt(256), seed 0; no segments
    check(synth.gqa(1, 16, 4, 512, seed=0, scale=1.0 / 16, dtype="f32"), "L512 f32 scaled")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", [1.0, 8.0])
def test_unscaled_and_peaky(dtype, scale):
    """Logit std 1 and a "peaky" variant: only Q is scaled (x8 gives logit std 8).

    fp32: the rounding of the fp32 score dot products grows with the logits
    (|do| ~ u |s| |v - o|), so both bars scale with them. bf16 / fp16: the
    error is the rounding of P and of O to the input type, which does not grow
    with the logits, so the stated bars hold as they are."""
    x = synth.gqa(1, 16, 4, 512, seed=3, dtype=dtype)
    if scale != 1.0:
        x = synth.Inputs(x.q * np.float32(scale), x.k, x.v, dtype)
    check(x, "L512 %s qscale %g" % (dtype, scale), tol_scale=scale if dtype == "f32" else 1.0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("L", [1, 31, 33, 127, 1000, 2049])
def test_ragged_lengths(dtype, L):
    check(synth.gqa(1, 16, 4, L, seed=L, dtype=dtype), "L%d %s" % (L, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_batch_two_and_lq_ne_lk_noncausal(dtype):
    check(synth.gqa(2, 16, 4, 300, 777, seed=5, dtype=dtype, causal=False), "B2 Lq300 Lk777 noncausal " + dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("Lq,Lk,q_offset", [(700, 300, 0), (300, 700, 0), (200, 150, 40)])
def test_causal_lq_ne_lk(dtype, Lq, Lk, q_offset):
    """Causal with Lq != Lk: rows whose limit q_offset + i reaches past the
    last key see every key (Lq > Lk), and with Lq < Lk the keys past the last
    row's limit are unseen by every row."""
    x = synth.gqa(1, 16, 4, Lq, Lk, seed=Lq + Lk + q_offset, dtype=dtype, q_offset=q_offset)
    check(x, "causal Lq%d Lk%d off%d %s" % (Lq, Lk, q_offset, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_branch_offset(dtype):
    # one branch: m = 256 rows at positions S.. over S + m keys
    S, m = 1000, 256
    x = synth.gqa(1, 16, 4, m, S + m, seed=7, dtype=dtype, q_offset=S)
    check(x, "branch S1000 m256 " + dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rep", [1, 2, 3, 5, 6, 8, 12, 16, 64])
def test_other_group_sizes(dtype, rep):
    """Query heads per KV head: powers of two, and 3, 5, 6, 12 (a workgroup
    takes 1 or 2 heads of the group, the most of 4, 2, 1 dividing it) up to
    the largest group the library takes (64)."""
    Hkv = 1 if rep == 64 else 2 if rep >= 8 else 4
    check(synth.gqa(1, Hkv * rep, Hkv, 200, seed=rep, dtype=dtype), "rep%d %s" % (rep, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [True, False])
def test_packed_segments(dtype, causal):
    L = 3000
    lens = synth.segment_lengths(L, 100, 900, seed=11)
    ids = synth.segment_ids(lens)[None]
    x = synth.gqa(1, 16, 4, L, seed=12, dtype=dtype, causal=causal)
    x.seg_q = x.seg_k = ids
    check(x, "packed segments %s causal=%s" % (dtype, causal))


@pytest.mark.parametrize("dtype", DTYPES)
def test_unsorted_segments_and_empty_rows(dtype):
    # ids drawn at random (not packed); query id 9 matches no key: those rows are empty
    L = 700
    rng = np.random.default_rng(13)
    sq = rng.integers(0, 3, size=(2, L)).astype(np.int32)
    sk = rng.integers(0, 3, size=(2, L)).astype(np.int32)
    sq[:, ::50] = 9
    for causal in (True, False):
        x = synth.gqa(2, 16, 4, L, seed=14, dtype=dtype, causal=causal)
        x.seg_q, x.seg_k = sq, sk
        check(x, "random segments %s causal=%s" % (dtype, causal))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_tiny_with_segments(dtype, L):
    """Fewer id entries than one 16-byte load (the id scan's small-array path),
    causal and not, with a query id that no key has."""
    for causal in (True, False):
        x = synth.gqa(1, 16, 4, L, seed=50 + L, dtype=dtype, causal=causal)
        x.seg_k = np.array([[0, 0, 1, 1, 1][:L]], dtype=np.int32)
        x.seg_q = x.seg_k.copy()
        x.seg_q[0, 0] = 7
        check(x, "L%d with ids %s causal=%s" % (L, dtype, causal))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("packed", [True, False])
def test_extreme_segment_ids(dtype, packed):
    """Ids at the ends of int32, which the id scan also uses to mark an empty
    range: packed runs of INT32_MIN, -1, 0, INT32_MAX (each id once), or those
    four drawn at random; some query rows take an id no key has, so their
    rows are empty."""
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    L = 700
    vals = np.array([lo, -1, 0, hi], dtype=np.int32)
    if packed:
        ids = np.repeat(vals, [150, 200, 100, 250])[None]
    else:
        ids = np.random.default_rng(60).choice(vals, size=(1, L)).astype(np.int32)
    for causal in (True, False):
        x = synth.gqa(1, 16, 4, L, seed=61, dtype=dtype, causal=causal)
        x.seg_k = ids
        x.seg_q = ids.copy()
        x.seg_q[0, 5::97] = 7
        check(x, "ids at the int32 ends, %s %s causal=%s" % ("packed" if packed else "random", dtype, causal))


@pytest.mark.parametrize("dtype", DTYPES)
def test_causal_offset_far_past_the_keys(dtype):
    """A causal call whose query positions start 2^40 past the keys sees every
    key: it equals the non-causal call, bit for bit (the same tiles, in the
    same order, with no mask), and the oracle."""
    x = synth.gqa(2, 16, 4, 100, 300, seed=62, dtype=dtype, q_offset=1 << 40, causal=True)
    check(x, "causal q_offset=2^40 " + dtype)
    o, lse = run(x)
    q, k, v = to_dev(x)
    o2, l2 = gqa.fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [True, False])
def test_packed_segments_equal_per_segment_calls(dtype, causal):
    """Packed segments with ids give, row for row, what each segment gives as
    a call of its own (B = 1, Lq = Lk = its length, no ids). The segments
    start off the 64-key tile grid, so the sums run in another order: equal
    within the forward's bars, not bitwise."""
    L = 2000
    lens = synth.segment_lengths(L, 100, 700, seed=16)
    bounds = synth.segment_bounds(lens)
    ids = torch.from_numpy(synth.segment_ids(lens)[None]).to(DEV)
    x = synth.gqa(1, 16, 4, L, seed=17, dtype=dtype, causal=causal)
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v, causal=causal, seg_q=ids, seg_k=ids)
    print("case: packed vs per-segment %s causal=%s, %d segments" % (dtype, causal, len(lens)), flush=True)
    for a, b in bounds:
        sl = slice(a, b)
        o_s, l_s = gqa.fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                           causal=causal)
        torch.cuda.synchronize()
        do = float((o[:, :, sl].float() - o_s.float()).abs().max())
        dl = float((lse[:, :, sl] - l_s).abs().max())
        assert do <= TOL_O[dtype] and dl <= TOL_LSE, "segment [%d, %d): |do| %.3g |dlse| %.3g" % (a, b, do, dl)


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_segment_is_bitwise_the_unsegmented_call(dtype):
    x = synth.gqa(1, 16, 4, 1500, seed=15, dtype=dtype)
    q, k, v = to_dev(x)
    o0, l0 = gqa.fwd(q, k, v)
    z = torch.zeros((1, 1500), dtype=torch.int32, device=q.device)
    o1, l1 = gqa.fwd(q, k, v, seg_q=z, seg_k=z)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("dtype", DTYPES)
def test_deterministic(dtype):
    x = synth.gqa(1, 16, 4, 2000, seed=16, dtype=dtype)
    q, k, v = to_dev(x)
    a = gqa.fwd(q, k, v)
    b = gqa.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", DTYPES)
def test_batch_equals_separate_calls(dtype):
    x = synth.gqa(2, 16, 4, 640, seed=17, dtype=dtype)
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v)
    for b in range(2):
        ob, lb = gqa.fwd(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[b:b + 1], ob) and torch.equal(lse[b:b + 1], lb)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gqa_equals_repeated_kv(dtype):
    # K/V repeated to every query head (Hq = Hkv = 16) gives the grouped result
    x = synth.gqa(1, 16, 4, 900, seed=18, dtype=dtype)
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v)
    o2, l2 = gqa.fwd(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous())
    torch.cuda.synchronize()
    assert (o.float() - o2.float()).abs().max().item() <= TOL_O[dtype]
    assert (lse - l2).abs().max().item() <= 1e-4


@pytest.mark.parametrize("dtype", DTYPES)
def test_branch_two_calls_and_merge(dtype):
    # prefix part (non-causal over S keys) + suffix part (causal over the branch keys), merged,
    # equals the single call with q_offset = S over concat(prefix, branch); both against the oracle
    S, m = 1200, 200
    x = synth.gqa(1, 16, 4, m, S + m, seed=19, dtype=dtype, q_offset=S)
    q, k, v = to_dev(x)
    o1, l1 = gqa.fwd(q, k[:, :, :S].contiguous(), v[:, :, :S].contiguous(), causal=False)
    o2, l2 = gqa.fwd(q, k[:, :, S:].contiguous(), v[:, :, S:].contiguous(), causal=True)
    om, lm = gqa.merge(o1, l1, o2, l2)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, q_offset=S)
    compare(om, lm, o_ref, l_ref, dtype, label="branch merge " + dtype)
    # merge in place into o1 / l1
    gqa.merge(o1, l1, o2, l2, out=o1, out_lse=l1)
    torch.cuda.synchronize()
    assert torch.equal(o1, om) and torch.equal(l1, lm)


def test_merge_matches_oracle_merge_with_empty_rows():
    rng = np.random.default_rng(20)
    o1 = rng.standard_normal((64, 256)).astype(np.float32)
    o2 = rng.standard_normal((64, 256)).astype(np.float32)
    l1 = rng.standard_normal(64).astype(np.float32) * 3
    l2 = rng.standard_normal(64).astype(np.float32) * 3
    l1[:4] = -np.inf
    l2[2:6] = -np.inf
    o1[:4] = 0
    o2[2:6] = 0
    om, lm = gqa.merge(dev_tensor(o1), dev_tensor(l1), dev_tensor(o2), dev_tensor(l2))
    torch.cuda.synchronize()
    ro, rl = oracle.merge(o1, l1, o2, l2)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(lm.cpu().numpy()), ~fin)
    assert np.max(np.abs(om.cpu().numpy() - ro)) < 1e-5
    assert np.max(np.abs(lm.cpu().numpy()[fin] - rl[fin])) < 1e-5


def test_library_allocates_nothing():
    x = synth.gqa(1, 16, 4, 4096, seed=21, dtype="bf16")
    q, k, v = to_dev(x)
    o = torch.empty_like(q)
    lse = torch.empty((1, 16, 4096), dtype=torch.float32, device=q.device)
    # the first launch loads the library's code object on the device (with its
    # static scratch array); the calls after it must not allocate
    gqa.fwd(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        gqa.fwd(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_stream_argument_is_honoured():
    x = synth.gqa(1, 16, 4, 800, seed=22, dtype="f32")
    q, k, v = to_dev(x)
    ref = gqa.fwd(q, k, v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = gqa.fwd(q, k, v)
    s.synchronize()
    assert torch.equal(ref[0], out[0]) and torch.equal(ref[1], out[1])


def test_binding_rejects_mismatched_buffers():
    """The Python binding checks what the C interface cannot see: output
    buffers of the wrong shape or type, and mismatched segment ids, raise before
    any launch."""
    x = synth.gqa(1, 16, 4, 64, seed=18)
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v)
    with pytest.raises(ValueError):
        gqa.merge(o, lse, o, lse, out=torch.empty_like(o)[:, :, :32])
    with pytest.raises(ValueError):
        gqa.merge(o, lse, o, lse, out_lse=torch.empty(1, 16, 63, device=DEV))
    with pytest.raises(ValueError):
        gqa.fwd(q, k, v, out=torch.empty(1, 16, 64, 256, dtype=torch.bfloat16, device=DEV))
    ids = torch.zeros((1, 64), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        gqa.fwd_split(q, k, v, seg_q=ids, seg_k=ids[:, :32].contiguous())
    with pytest.raises(ValueError):
        gqa.fwd_split(q, k[:, :, :, :128].contiguous(), v[:, :, :, :128].contiguous())
