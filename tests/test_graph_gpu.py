"""The forward entry points captured in a HIP graph and replayed.

The library launches its kernels on the caller's stream, issues no memset and
allocates nothing inside a call, so a call can be captured. Each case
captures one call, then replays the graph several times. Between the replays
it runs eager calls on other inputs that write the same outputs (and, for the
split paths, the same workspace or static scratch), with synchronizations in
between. Every replay's o and lse must equal the eager call's bit for bit.
"""
import pytest
import torch

import long_context_causal_amd as gqa
import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def replay_check(call, other, o, lse, label, reps=3):
    print("case:", label, flush=True)
    call()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(reps):
        other()  # eager work on other inputs into the same outputs
        torch.cuda.synchronize()
        assert not (torch.equal(o, o_ref) and torch.equal(lse, l_ref)), "the eager call left the outputs unchanged"
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "%s: replay %d differs" % (label, r)


def inputs(seed, Lq, Lk, dtype="bf16"):
    return to_dev(synth.gqa(1, 16, 4, Lq, Lk, seed=seed, dtype=dtype, q_offset=Lk - Lq))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_replays(dtype):
    Lq = Lk = 700
    q, k, v = inputs(400, Lq, Lk, dtype)
    q2, k2, v2 = inputs(401, Lq, Lk, dtype)
    o = torch.empty_like(q)
    lse = torch.empty(1, 16, Lq, dtype=torch.float32, device=q.device)
    replay_check(lambda: gqa.fwd(q, k, v, out=o, lse=lse), lambda: gqa.fwd(q2, k2, v2, out=o, lse=lse), o, lse,
                 "forward " + dtype)


@pytest.mark.parametrize("Lq,dtype", [(16, "bf16"), (48, "bf16"), (16, "f32"), (1, "f32")])
def test_split_replays(Lq, dtype):
    """16 positions (the decode kernels; fp32 also 1 position, its split-d
    mode) and 48 (the long-block kernel's split launch), 9 splits over 5,000
    keys, with the caller's workspace."""
    Lk = 5000
    q, k, v = inputs(410 + Lq, Lq, Lk, dtype)
    q2, k2, v2 = inputs(420 + Lq, Lq, Lk, dtype)
    o = torch.empty_like(q)
    lse = torch.empty(1, 16, Lq, dtype=torch.float32, device=q.device)
    ws = torch.empty(gqa.split_workspace(1, 16, Lq, 256, 9), dtype=torch.uint8, device=q.device)
    kw = dict(q_offset=Lk - Lq, n_split=9, out=o, lse=lse, workspace=ws)
    replay_check(lambda: gqa.fwd_split(q, k, v, **kw), lambda: gqa.fwd_split(q2, k2, v2, **kw), o, lse,
                 "split Lq=%d %s" % (Lq, dtype))


def test_noalloc_replays():
    """The allocation-free split call (partials in the library's static
    scratch), decode shape."""
    Lq, Lk = 16, 5000
    q, k, v = inputs(430, Lq, Lk)
    q2, k2, v2 = inputs(431, Lq, Lk)
    o = torch.empty_like(q)
    lse = torch.empty(1, 16, Lq, dtype=torch.float32, device=q.device)
    kw = dict(q_offset=Lk - Lq, n_split=9)
    replay_check(lambda: gqa.fwd_split_noalloc(q, k, v, o, lse, **kw),
                 lambda: gqa.fwd_split_noalloc(q2, k2, v2, o, lse, **kw), o, lse, "noalloc split")
