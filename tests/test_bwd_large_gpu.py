"""The backward at full size, in the launch configuration the benchmark times
(fp32 at L = 30,468; bf16 at L = 60,926), against the fp64 oracle where it
can be evaluated one output at a time, and against exact identities over all
keys:

  * dq on sampled query rows (each dq row depends only on its own row's
    softmax over its visible keys);
  * dk, dv on the last 64 keys and a few others near the end (the oracle needs
    the statistics of only the rows that see them);
  * sum_j dk_j = 0 for every key/value head and d (the ds of a row sum to 0),
    and sum_j dv_j = sum of dout over the rows of the heads that share the
    key/value head (the p of a row sum to 1), checked on every key against a
    bar relative to sum_j |dk_j| (resp. |dv_j|).

Bar per tensor, as in the small backward tests: max|d - d_ref| <=
TOL_BWD[dtype] * max(1, max|d_ref|).
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import TOL_BWD, dout_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


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

    rows = synth.sample_rows(L, n_random=24)[::3]
    keys = np.unique(np.concatenate([np.arange(L - 64, L), [L - 65, L - 128, L - 129, L - 200]])).astype(np.int64)
    rq = oracle.bwd_dq(x.q, x.k, x.v, g.values, rows=rows)
    rk, rv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, keys=keys)
    dq_h = dq[:, :, torch.from_numpy(rows).to(dq.device)].float().cpu().numpy().astype(np.float64)
    kk = torch.from_numpy(keys).to(dk.device)
    dk_h = dk[:, :, kk].float().cpu().numpy().astype(np.float64)
    dv_h = dv[:, :, kk].float().cpu().numpy().astype(np.float64)
    e = {"dq": rel_err(dq_h, rq), "dk": rel_err(dk_h, rk), "dv": rel_err(dv_h, rv)}
    print("%s: %d rows, %d keys: rel max|d| dq %.3g dk %.3g dv %.3g" % (label, len(rows), len(keys), e["dq"],
                                                                       e["dk"], e["dv"]), flush=True)
    for name, err in e.items():
        assert err <= TOL_BWD[dtype], "%s: %s %.3g" % (label, name, err)

    # identities over every key, in fp64 on the host
    dk_all = dk.double().cpu().numpy()
    dv_all = dv.double().cpu().numpy()
    sk = np.abs(dk_all.sum(axis=2))
    bound_k = TOL_BWD[dtype] * np.abs(dk_all).sum(axis=2)
    want_v = g.values.astype(np.float64).reshape(1, 4, 4, L, 256).sum(axis=(2, 3))
    sv = np.abs(dv_all.sum(axis=2) - want_v)
    bound_v = TOL_BWD[dtype] * np.abs(dv_all).sum(axis=2)
    print("%s: max |sum dk| / sum|dk| %.3g, max |sum dv - sum dout| / sum|dv| %.3g" % (
        label, (sk / np.abs(dk_all).sum(axis=2)).max(), (sv / np.abs(dv_all).sum(axis=2)).max()), flush=True)
    assert np.all(sk <= bound_k), label + ": sum of dk"
    assert np.all(sv <= bound_v), label + ": sum of dv"


def test_bwd_packed_segments_bf16_131072():
    """The segmented workload (bf16, L = 131,072, packed segments of 2k-32k,
    seed 1): dq on sampled rows (segment boundaries included), dk/dv on the
    last 16 keys of every segment, and the two identities over all keys."""
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
    rows = synth.sample_rows(L, bounds=bounds, n_random=8, upto=256)
    keys = np.unique(np.concatenate([np.arange(b - 16, b) for _, b in bounds])).astype(np.int64)
    seg = ids[None]
    rq = oracle.bwd_dq(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, rows=rows)
    rk, rv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, seg_q=seg, seg_k=seg, keys=keys)
    dq_h = dq[:, :, torch.from_numpy(rows).to(dq.device)].float().cpu().numpy().astype(np.float64)
    kk = torch.from_numpy(keys).to(dk.device)
    e = {"dq": rel_err(dq_h, rq), "dk": rel_err(dk[:, :, kk], rk), "dv": rel_err(dv[:, :, kk], rv)}
    print("%s: %d rows, %d keys: rel max|d| dq %.3g dk %.3g dv %.3g" % (label, len(rows), len(keys), e["dq"],
                                                                       e["dk"], e["dv"]), flush=True)
    for name, err in e.items():
        assert err <= TOL_BWD["bf16"], "%s: %s %.3g" % (label, name, err)
    dk_all = dk.double().cpu().numpy()
    dv_all = dv.double().cpu().numpy()
    want_v = g.values.astype(np.float64).reshape(1, 4, 4, L, 256).sum(axis=(2, 3))
    assert np.all(np.abs(dk_all.sum(axis=2)) <= TOL_BWD["bf16"] * np.abs(dk_all).sum(axis=2)), label + ": sum dk"
    assert np.all(np.abs(dv_all.sum(axis=2) - want_v) <= TOL_BWD["bf16"] * np.abs(dv_all).sum(axis=2)), label
