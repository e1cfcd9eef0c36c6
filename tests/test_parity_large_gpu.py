"""HIP path against the fp64 oracle at the workloads' full sizes, in the launch
configuration the benchmark times, on sampled query rows (each output row
depends only on its own query row, so a sampled row is checked exactly).

Rows checked per head: the first and last rows, every multiple of 16/32/64/128
below 4096 and within the last 4096 rows (the workgroups with the longest key
loops) and its neighbours, segment and branch boundaries and their neighbours,
and 512 random rows (fixed seed). Bars: max|do| <= 2e-5 (fp32) /
2e-2 (bf16) / 2.5e-3 (fp16, derived), max|dlse| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import long_context_causal_amd as gqa
import oracle
import synth
from gpu_util import compare, dev_tensor, run, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def check_sampled(x, label, bounds=None, n_random=512):
    print("case:", label, flush=True)
    o, lse = run(x)
    L = x.q.shape[2]
    rows = synth.sample_rows(L, bounds=bounds, n_random=n_random)
    o_ref, l_ref = oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=x.seg_q,
                               seg_k=x.seg_k, rows=rows)
    compare(o, lse, o_ref, l_ref, x.dtype, rows=rows, label="%s (%d rows x 16 heads)" % (label, len(rows)))
    return o, lse


@pytest.mark.parametrize("L", [15231, 30468])
def test_fp32_state_lengths(L):
    # causal GQA forward, fp32, B=1 Hq=16 Hkv=4 D=256 at the 16k and 32k bucket lengths
    check_sampled(synth.gqa(1, 16, 4, L, seed=0, dtype="f32"), "fp32 L=%d" % L)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_64k_state_length(dtype):
    check_sampled(synth.gqa(1, 16, 4, 60926, seed=0, dtype=dtype), "%s L=60926" % dtype)


def test_shared_prefix_branches_fp32():
    """S = 30,468 prefix tokens, 40 branches of m = 256 rows at positions S..:
    the measured two-call form (prefix call over all n*m rows, segmented causal
    suffix call, lse merge) against the oracle on sampled rows of sampled
    branches, and against the single in-signature call (q_offset = S over
    concat(prefix, branch)) for two branches."""
    br = synth.Branch(S=30468, n=40, m=256, seed=0, dtype="f32")
    qb, kb, vb, ids = br.branch_layout()
    q = dev_tensor(qb)
    kp, vp = dev_tensor(br.k_p[None]), dev_tensor(br.v_p[None])
    ks, vs = dev_tensor(kb), dev_tensor(vb)
    sid = seg_dev(ids[None])
    o1, l1 = gqa.fwd(q, kp, vp, causal=False)
    o2, l2 = gqa.fwd(q, ks, vs, causal=True, seg_q=sid, seg_k=sid)
    om, lm = gqa.merge(o1, l1, o2, l2)
    torch.cuda.synchronize()
    m, S = br.m, br.S
    rows_in_branch = np.array([0, 1, 2, 15, 16, 17, 63, 64, 127, 128, 200, 254, 255])
    for b in (0, 1, 17, 39):
        k_cat = np.concatenate([br.k_p[None], br.k_b[b:b + 1]], axis=2)
        v_cat = np.concatenate([br.v_p[None], br.v_b[b:b + 1]], axis=2)
        o_ref, l_ref = oracle.attn(br.q_b[b:b + 1], k_cat, v_cat, causal=True, q_offset=S, rows=rows_in_branch)
        sel = b * m + rows_in_branch
        compare(om[:, :, sel], lm[:, :, sel], o_ref, l_ref, "f32", label="branch %d two-call form" % b)
        if b in (0, 39):
            ob, lb = gqa.fwd(dev_tensor(br.q_b[b:b + 1]), dev_tensor(k_cat), dev_tensor(v_cat), causal=True, q_offset=S)
            torch.cuda.synchronize()
            compare(ob[:, :, rows_in_branch], lb[:, :, rows_in_branch], o_ref, l_ref, "f32",
                    label="branch %d single call" % b)


def test_packed_segments_bf16_131072():
    """L = 131,072 split into segments of uniform-random length 2k-32k (seed 1),
    causal within segments; sampled rows include every segment's first and
    last rows. Also: all-zero ids give bitwise the unsegmented call."""
    L = 131072
    lens = synth.segment_lengths(L, 2048, 32768, seed=1)
    ids = synth.segment_ids(lens)
    x = synth.gqa(1, 16, 4, L, seed=0, dtype="bf16")
    x.seg_q = x.seg_k = ids[None]
    check_sampled(x, "bf16 L=131072 %d segments" % len(lens), bounds=synth.segment_bounds(lens))
    q, k, v = to_dev(x)
    z = torch.zeros((1, L), dtype=torch.int32, device=q.device)
    o0, l0 = gqa.fwd(q, k, v)
    o1, l1 = gqa.fwd(q, k, v, seg_q=z, seg_k=z)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_memory_linear_in_L():
    """Peak device memory of the fp32 forward grows linearly with L, and the
    memory beyond the inputs and outputs is zero: below a quarter of one fp32
    L x L score matrix of a single head, the bound the pages' long-row test
    applies to the attention pass, where the L x L math path needs 16 such
    matrices."""
    per_token = []
    # load the library's code object on the device first (a tiny call)
    t = torch.zeros(1, 16, 8, 256, device="cuda:0")
    gqa.fwd(t, t[:, :4].contiguous(), t[:, :4].contiguous())
    torch.cuda.synchronize()
    del t
    for L in (15231, 30468, 60926):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        q = torch.randn(1, 16, L, 256, device="cuda:0")
        k = torch.randn(1, 4, L, 256, device="cuda:0")
        v = torch.randn(1, 4, L, 256, device="cuda:0")
        o = torch.empty_like(q)
        lse = torch.empty(1, 16, L, device="cuda:0")
        io = torch.cuda.memory_allocated() - base
        free0, _ = torch.cuda.mem_get_info()
        gqa.fwd(q, k, v, out=o, lse=lse)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        peak = torch.cuda.max_memory_allocated() - base
        extra = max(peak - io, free0 - free1)
        print("L=%d peak %.3f GiB (inputs+outputs %.3f GiB), beyond them %d bytes; one-head L x L fp32 %.3f GiB, "
              "math path %.2f GiB" % (L, peak / 2 ** 30, io / 2 ** 30, extra, L * L * 4 / 2 ** 30,
                                       16 * L * L * 4 / 2 ** 30), flush=True)
        assert extra < 0.25 * L * L * 4 and extra == 0
        per_token.append(peak / L)
        del q, k, v, o, lse
    assert max(per_token) / min(per_token) < 1.01
