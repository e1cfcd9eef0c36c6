"""The backward at full size, in the launch configuration the benchmark times
(fp32 at L = 30,468; bf16 at L = 60,926; bf16 packed segments at
L = 131,072), against the fp64 oracle one output at a time, and against exact
identities over all keys:

  * dq on the sampled query rows of the forward's full-size tests (first and
    last rows, multiples of 16/32/64/128 near both ends, segment boundaries,
    512 random rows): each dq row depends only on its own row's softmax over
    its visible keys;
  * dk, dv on keys with short sums (the last keys of the sequence or of each
    segment: the oracle needs the statistics of only the few rows that see
    them) evaluated here;
  * dk, dv on keys with long sums (the first keys, tile edges among them, and
    keys spread over the sequence; the first 16 keys of every packed segment),
    summed over nearly every row of the four heads of a key/value head: their
    oracle values need a full pass over the sequence and are stored in
    tests/golden/bwd_long_sums.npz by tests/golden/make_bwd_golden.py, which
    calls only the oracle (with a hash of the inputs they were computed on);
  * sum_j dk_j = 0 for every key/value head and d (the ds of a row sum to 0),
    and sum_j dv_j = sum of dout over the rows of the heads that share the
    key/value head (the p of a row sum to 1), on every key, against a bar
    relative to sum_j |dk_j| (resp. |dv_j|).

Bar per tensor, as in the small backward tests: max|d - d_ref| <=
TOL_BWD[dtype] * max(1, max|d_ref|).
"""
import os

import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from golden.make_bwd_golden import fp32_keys, input_hash, packed_keys
from gpu_util import TOL_BWD, dout_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bwd_long_sums.npz")


def golden():
    return np.load(GOLDEN, allow_pickle=False)


def host(t, idx, dev):
    """Rows/keys `idx` of a [B, H, L, D] tensor on device `dev`, as fp64 on the host."""
    return t[:, :, torch.from_numpy(idx).to(dev)].float().cpu().numpy().astype(np.float64)


def check_identities(label, dtype, dk, dv, dout_values, L):
    dk_all = dk.double().cpu().numpy()
    dv_all = dv.double().cpu().numpy()
    sk = np.abs(dk_all.sum(axis=2))
    bound_k = TOL_BWD[dtype] * np.abs(dk_all).sum(axis=2)
    want_v = dout_values.astype(np.float64).reshape(1, 4, 4, L, 256).sum(axis=(2, 3))
    sv = np.abs(dv_all.sum(axis=2) - want_v)
    bound_v = TOL_BWD[dtype] * np.abs(dv_all).sum(axis=2)
    print("%s: max |sum dk| / sum|dk| %.3g, max |sum dv - sum dout| / sum|dv| %.3g" % (
        label, (sk / np.abs(dk_all).sum(axis=2)).max(), (sv / np.abs(dv_all).sum(axis=2)).max()), flush=True)
    assert np.all(sk <= bound_k), label + ": sum of dk"
    assert np.all(sv <= bound_v), label + ": sum of dv"


@pytest.mark.parametrize("dtype,L", [("f32", 30468), ("bf16", 60926)])
def test_bwd_full_size(dtype, L):
    label = "bwd %s L=%d" % (dtype, L)
    print("case:", label, flush=True)
    x = synth.gqa(1, 16, 4, L, seed=0, dtype=dtype)
    g = synth.Grad(x.q.shape, seed=1, dtype=dtype)
    q, k, v = to_dev(x)
    do = dout_dev(g)
    o, lse = gqa.fwd(q, k, v)
    dq, dk, dv, _ = gqa.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    del o, lse

    rows = synth.sample_rows(L)
    keys = np.unique(np.concatenate([np.arange(L - 64, L), [L - 65, L - 128, L - 129, L - 200]])).astype(np.int64)
    rq = oracle.bwd_dq(x.q, x.k, x.v, g.values, rows=rows)
    rk, rv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, keys=keys)
    e = {"dq": rel_err(host(dq, rows, dq.device), rq), "dk": rel_err(host(dk, keys, dk.device), rk),
         "dv": rel_err(host(dv, keys, dv.device), rv)}
    print("%s: %d rows, %d last keys: rel max|d| dq %.3g dk %.3g dv %.3g" % (label, len(rows), len(keys), e["dq"],
                                                                            e["dk"], e["dv"]), flush=True)
    for name, err in e.items():
        assert err <= TOL_BWD[dtype], "%s: %s %.3g" % (label, name, err)
    if dtype == "f32":
        gd = golden()
        assert str(gd["f32_hash"]) == input_hash(x.q, x.k, x.v, g.values), "inputs differ from the stored values'"
        keys = gd["f32_keys"]
        assert np.array_equal(keys, fp32_keys(L))
        ek, ev = rel_err(host(dk, keys, dk.device), gd["f32_dk"]), rel_err(host(dv, keys, dv.device), gd["f32_dv"])
        print("%s: %d keys with long sums (0 .. %d): rel max|d| dk %.3g dv %.3g" % (label, len(keys), keys[-1], ek,
                                                                                 ev), flush=True)
        assert ek <= TOL_BWD[dtype] and ev <= TOL_BWD[dtype], label + ": long-sum keys"
    check_identities(label, dtype, dk, dv, g.values, L)


def test_bwd_packed_segments_bf16_131072():
    """The segmented workload (bf16, L = 131,072, packed segments of 2k-32k,
    seed 1): dq on the sampled rows (segment boundaries included), dk/dv on the
    last 16 keys (here) and the first 16 keys (stored) of every segment, and the
    two identities over all keys."""
    L = 131072
    lens = synth.segment_lengths(L, 2048, 32768, seed=1)
    ids = synth.segment_ids(lens)
    bounds = synth.segment_bounds(lens)
    label = "bwd bf16 L=%d, %d packed segments" % (L, len(lens))
    print("case:", label, flush=True)
    x = synth.gqa(1, 16, 4, L, seed=0, dtype="bf16")
    g = synth.Grad(x.q.shape, seed=1, dtype="bf16")
    q, k, v = to_dev(x)
    do = dout_dev(g)
    sid = torch.from_numpy(ids[None]).to(q.device)
    o, lse = gqa.fwd(q, k, v, seg_q=sid, seg_k=sid)
    dq, dk, dv, _ = gqa.bwd(q, k, v, o, lse, do, seg_q=sid, seg_k=sid)
    torch.cuda.synchronize()
    del o, lse
    rows = synth.sample_rows(L, bounds=bounds)
    keys = np.unique(np.concatenate([np.arange(b - 16, b) for _, b in bounds])).astype(np.int64)
    seg = ids[None]
    rq = oracle.bwd_dq(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, rows=rows)
    rk, rv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, keys=keys)
    e = {"dq": rel_err(host(dq, rows, dq.device), rq), "dk": rel_err(host(dk, keys, dk.device), rk),
         "dv": rel_err(host(dv, keys, dv.device), rv)}
    print("%s: %d rows, %d last keys of segments: rel max|d| dq %.3g dk %.3g dv %.3g" % (
        label, len(rows), len(keys), e["dq"], e["dk"], e["dv"]), flush=True)
    for name, err in e.items():
        assert err <= TOL_BWD["bf16"], "%s: %s %.3g" % (label, name, err)
    gd = golden()
    assert str(gd["packed_hash"]) == input_hash(x.q, x.k, x.v, g.values, seg), "inputs differ from the stored values'"
    keys = gd["packed_keys"]
    assert np.array_equal(keys, packed_keys(lens))
    ek, ev = rel_err(host(dk, keys, dk.device), gd["packed_dk"]), rel_err(host(dv, keys, dv.device), gd["packed_dv"])
    print("%s: first 16 keys of every segment (%d keys): rel max|d| dk %.3g dv %.3g" % (label, len(keys), ek, ev),
          flush=True)
    assert ek <= TOL_BWD["bf16"] and ev <= TOL_BWD["bf16"], label + ": first keys of segments"
    check_identities(label, "bf16", dk, dv, g.values, L)
