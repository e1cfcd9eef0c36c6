"""Checks that pin the fp64 oracle to something other than itself.

Every pin takes an oracle instance (the default build, or a deliberately broken
build in the mutation test) and raises AssertionError when the oracle disagrees
with: a 50-digit brute force on tiny inputs, a closed form, or an invariant the
pages state. Sources, by page and section:
  * kev pull request 202, "Why fp32 fell to the L x L kernel" (the math path)
    and "The change" (K/V repetition per query head gives the same attention as
    grouped-query attention; the test plan says the outputs match).
  * maxtext pull request 4929, problem statement: with one segment per example
    the ids are constant and the non-segmented kernel gives the same result.
  * system1-omni issue 27, "Three differences from Cua-S1 that matter", item 3:
    a branch's positions restart at the state length, so a branch row sees the
    whole state plus its own causal suffix.
"""
import numpy as np

import brute

SCALE_D = lambda D: 1.0 / np.sqrt(D)  # noqa: E731  (1/sqrt(D), the stated scale)


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _grid(a, step=2.0 ** -8):
    """Round to multiples of `step` so that later sums and small multiples stay exact in fp32."""
    return (np.round(a / step) * step).astype(np.float32)


def _case(B, Hq, Hkv, Lq, Lk, D, seed, scale=1.0):
    return (_rand((B, Hq, Lq, D), seed, scale), _rand((B, Hkv, Lk, D), seed + 1, scale),
            _rand((B, Hkv, Lk, D), seed + 2))


BRUTE_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, q_offset, segments, input scale
    (1, 4, 2, 7, 7, 8, True, 0, False, 1.0),
    (2, 8, 2, 6, 9, 4, True, 3, False, 1.0),
    (1, 2, 2, 12, 12, 2, False, 0, False, 2.0),
    (2, 4, 1, 10, 10, 1, True, 0, True, 1.0),
    (1, 8, 4, 9, 12, 8, True, 3, True, 1.5),
    (2, 4, 4, 5, 11, 4, False, 0, True, 1.0),
    (1, 1, 1, 12, 12, 8, True, 0, True, 3.0),
]


def pin_brute_force(orc):
    """Oracle within 1e-12 of the 50-digit brute force (explicit repetition,
    explicit mask matrix, unshifted softmax) on tiny inputs, covering GQA ratios
    1-4, causal on and off, q_offset 0 and 3, segments and empty rows."""
    for n, (B, Hq, Hkv, Lq, Lk, D, causal, off, seg, sc) in enumerate(BRUTE_CASES):
        q, k, v = _case(B, Hq, Hkv, Lq, Lk, D, 100 + 7 * n, sc)
        sq = sk = None
        if seg:
            rng = np.random.default_rng(500 + n)
            sq = rng.integers(0, 3, size=(B, Lq)).astype(np.int32)
            sk = rng.integers(0, 3, size=(B, Lk)).astype(np.int32)
            sq[:, 0] = 7  # a query id no key has: an empty row when causal is off
        o, lse = orc.attn(q, k, v, causal=causal, q_offset=off, seg_q=sq, seg_k=sk)
        ob, lb = brute.attn(q, k, v, causal=causal, q_offset=off, seg_q=sq, seg_k=sk)
        assert np.array_equal(np.isinf(lse), np.isinf(lb)), "empty-row pattern differs (case %d)" % n
        fin = np.isfinite(lb)
        assert np.max(np.abs(lse[fin] - lb[fin])) < 1e-12, "lse differs (case %d)" % n
        assert np.max(np.abs(o - ob)) < 1e-12, "o differs (case %d)" % n
        assert np.all(o[~fin] == 0.0)


def pin_rows_sum_to_one(orc):
    """Softmax weights of every row are non-negative, zero on invisible keys and
    sum to 1 within 1e-14."""
    q, k, v = _case(2, 4, 2, 9, 13, 8, 11, 2.0)
    seg = np.array([[0, 0, 0, 1, 1, 1, 1, 2, 2], [0, 0, 0, 0, 0, 0, 1, 1, 1]], dtype=np.int32)
    segk = np.concatenate([seg, np.full((2, 4), 2, dtype=np.int32)], axis=1)
    for b in range(2):
        for h in range(4):
            for i in range(9):
                w = orc.weights(q, k, v, b, h, i, causal=True, q_offset=4, seg_q=seg, seg_k=segk)
                j = np.arange(13)
                invisible = (j > 4 + i) | (segk[b] != seg[b, i])
                assert np.all(w >= 0) and np.all(w[invisible] == 0)
                assert abs(w.sum() - 1.0) < 1e-14


def pin_gqa_equals_repeat(orc):
    """Grouped-query attention equals attention on K/V repeated per query head
    (contiguous groups: head h uses key/value head h // (Hq/Hkv)), bitwise."""
    q, k, v = _case(2, 16, 4, 21, 21, 16, 21)
    o, lse = orc.attn(q, k, v)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, lse2 = orc.attn(q, kr, vr)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_one_segment_equals_none(orc):
    """Constant segment ids give exactly the non-segmented result."""
    q, k, v = _case(2, 4, 2, 17, 17, 8, 31)
    o, lse = orc.attn(q, k, v)
    s = np.full((2, 17), 5, dtype=np.int32)
    o2, lse2 = orc.attn(q, k, v, seg_q=s, seg_k=s)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_packed_equals_per_segment(orc):
    """Packed segments: each segment's rows equal causal attention run on that
    segment alone (block-diagonal causal mask), bitwise; batch rows use their
    own ids."""
    lens = [[5, 9, 3, 7], [12, 12]]
    q, k, v = _case(2, 4, 2, 24, 24, 8, 41)
    seg = np.stack([np.repeat(np.arange(len(l)), l) for l in lens]).astype(np.int32)
    o, lse = orc.attn(q, k, v, seg_q=seg, seg_k=seg)
    for b in range(2):
        a = 0
        for n in lens[b]:
            sl = slice(a, a + n)
            o1, l1 = orc.attn(q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl])
            assert np.array_equal(o[b:b + 1, :, sl], o1) and np.array_equal(lse[b:b + 1, :, sl], l1)
            a += n


def pin_prefix_branch(orc):
    """A branch of m rows with positions starting at S (q_offset = S) over
    concat(prefix, branch keys) equals rows S..S+m-1 of plain causal attention
    over the concatenated sequence, bitwise."""
    S, m = 13, 6
    q, k, v = _case(1, 4, 2, S + m, S + m, 8, 51)
    o_full, l_full = orc.attn(q, k, v)
    o_b, l_b = orc.attn(q[:, :, S:], k, v, q_offset=S)
    assert np.array_equal(o_full[:, :, S:], o_b) and np.array_equal(l_full[:, :, S:], l_b)


def pin_merge_identity(orc):
    """Attention over a disjoint union of key sets equals the log-sum-exp merge
    of the two parts (prefix keys, non-causal; branch keys, causal), 1e-13."""
    S, m = 11, 7
    q, k, v = _case(1, 4, 2, m, S + m, 8, 61, 1.5)
    o_full, l_full = orc.attn(q, k, v, q_offset=S)
    o1, l1 = orc.attn(q, k[:, :, :S], v[:, :, :S], causal=False)
    o2, l2 = orc.attn(q, k[:, :, S:], v[:, :, S:], causal=True)
    o, l = orc.merge(o1, l1, o2, l2)
    assert np.max(np.abs(o - o_full)) < 1e-13 and np.max(np.abs(l - l_full)) < 1e-13
    e = np.full_like(l1, -np.inf)
    oz, lz = orc.merge(o1, e, np.zeros_like(o1), e)
    assert np.all(oz == 0) and np.all(np.isneginf(lz))


def pin_zero_q(orc):
    """Q = 0: every visible key has weight 1/|A(i)|, so O_i is the mean of the
    visible V rows and lse_i = ln |A(i)|."""
    _, k, v = _case(1, 4, 2, 10, 14, 8, 71)
    q = np.zeros((1, 4, 10, 8), dtype=np.float32)
    o, lse = orc.attn(q, k, v, q_offset=3)
    for h in range(4):
        for i in range(10):
            n = min(14, 3 + i + 1)
            assert abs(lse[0, h, i] - np.log(n)) < 1e-14
            assert np.max(np.abs(o[0, h, i] - v[0, h // 2, :n].astype(np.float64).mean(axis=0))) < 1e-14


def pin_first_row(orc):
    """Causal row 0 with q_offset 0 sees key 0 only: O_0 = V_0 and
    lse_0 = s * q_0 . k_0 with s = 1/sqrt(D)."""
    q, k, v = _case(1, 8, 2, 5, 5, 16, 81, 2.0)
    o, lse = orc.attn(q, k, v)
    for h in range(8):
        g = h // 4
        assert np.array_equal(o[0, h, 0], v[0, g, 0].astype(np.float64))
        ref = SCALE_D(16) * np.dot(q[0, h, 0].astype(np.float64), k[0, g, 0].astype(np.float64))
        assert abs(lse[0, h, 0] - ref) < 1e-13


def pin_two_keys(orc):
    """A row with exactly two visible keys: O = sigma(s0-s1) V0 + sigma(s1-s0) V1,
    lse = logaddexp(s0, s1) (numpy), with s = q.k / sqrt(D)."""
    q, k, v = _case(1, 2, 1, 4, 4, 4, 91, 2.0)
    o, lse = orc.attn(q, k, v)
    qd, kd, vd = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    for h in range(2):
        s0 = qd[0, h, 1] @ kd[0, 0, 0] / 2.0
        s1 = qd[0, h, 1] @ kd[0, 0, 1] / 2.0
        w0 = 1.0 / (1.0 + np.exp(s1 - s0))
        assert abs(lse[0, h, 1] - np.logaddexp(s0, s1)) < 1e-13
        assert np.max(np.abs(o[0, h, 1] - (w0 * vd[0, 0, 0] + (1 - w0) * vd[0, 0, 1]))) < 1e-13


def pin_constant_v(orc):
    """V rows all equal to c: every non-empty row gives O = c."""
    q, k, _ = _case(1, 4, 2, 9, 9, 8, 101, 3.0)
    c = np.random.default_rng(5).standard_normal(8).astype(np.float32)
    v = np.broadcast_to(c, (1, 2, 9, 8)).copy()
    o, _ = orc.attn(q, k, v)
    assert np.max(np.abs(o - c.astype(np.float64))) < 1e-14


def pin_key_shift(orc):
    """Adding one vector u to every key leaves O unchanged and shifts lse_i by
    s * q_i . u (softmax is invariant to a per-row constant)."""
    q, k, v = _case(1, 4, 2, 8, 8, 8, 111)
    k = _grid(k)
    u = np.array([0.5, -0.25, 1.0, 0.0, 0.75, -1.0, 0.125, 2.0], dtype=np.float32)  # exact in fp32 sums
    o, lse = orc.attn(q, k, v)
    o2, lse2 = orc.attn(q, k + u, v)
    assert np.max(np.abs(o - o2)) < 1e-12
    shift = SCALE_D(8) * (q.astype(np.float64) @ u.astype(np.float64))
    assert np.max(np.abs(lse2 - lse - shift)) < 1e-12


def pin_linear_in_v(orc):
    """O is linear in V: O(aV1 + bV2) = a O(V1) + b O(V2)."""
    q, k, v1 = _case(1, 4, 2, 8, 8, 8, 121)
    v1, v2 = _grid(v1), _grid(_rand(v1.shape, 9))
    o1, _ = orc.attn(q, k, v1)
    o2, _ = orc.attn(q, k, v2)
    o3, _ = orc.attn(q, k, 2.0 * v1 - 0.5 * v2)
    assert np.max(np.abs(o3 - (2.0 * o1 - 0.5 * o2))) < 1e-13


def pin_row_subset(orc):
    """Evaluating a subset of rows gives the same values as the full run."""
    q, k, v = _case(1, 4, 2, 15, 15, 8, 131)
    o, lse = orc.attn(q, k, v)
    rows = np.array([0, 3, 14, 7])
    o2, lse2 = orc.attn(q, k, v, rows=rows)
    assert np.array_equal(o[:, :, rows], o2) and np.array_equal(lse[:, :, rows], lse2)


# ---- backward ---------------------------------------------------------------
# The backward is the gradient of the forward above (the pages train at these
# lengths: kev pull request 202, the title of the change; system1-omni issue 27,
# the model trains end to end). Pins: automatic differentiation of an explicit
# math-path forward, central differences of the oracle's own forward, and exact
# identities of the softmax gradient.

BWD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, q_offset, segments, input scale
    (1, 4, 2, 7, 7, 8, True, 0, False, 1.0),
    (2, 8, 2, 6, 9, 4, True, 3, False, 1.5),
    (1, 2, 2, 9, 9, 4, False, 0, False, 2.0),
    (2, 4, 1, 10, 10, 2, True, 0, True, 1.0),
    (1, 8, 4, 9, 12, 8, True, 3, True, 1.0),
    (2, 4, 4, 5, 11, 4, False, 0, True, 1.0),
]


def _bwd_case(n):
    B, Hq, Hkv, Lq, Lk, D, causal, off, seg, sc = BWD_CASES[n]
    q, k, v = _case(B, Hq, Hkv, Lq, Lk, D, 300 + 7 * n, sc)
    do = _rand((B, Hq, Lq, D), 900 + n)
    sq = sk = None
    if seg:
        rng = np.random.default_rng(700 + n)
        sq = rng.integers(0, 3, size=(B, Lq)).astype(np.int32)
        sk = rng.integers(0, 3, size=(B, Lk)).astype(np.int32)
        sq[:, 0] = 7  # no key has this id: an empty row when causal is off
    return q, k, v, do, dict(causal=causal, q_offset=off, seg_q=sq, seg_k=sk)


def _autograd_math_path(q, k, v, do, causal, q_offset, seg_q, seg_k):
    """Gradients by torch autograd (CPU, fp64) of the math path: K/V repeated to
    every query head by indexing, the full score matrix, an explicit boolean
    visibility matrix and a softmax from its definition; rows with no visible
    key output zero."""
    import torch
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    idx = torch.tensor([h // (Hq // Hkv) for h in range(Hq)])
    kr, vr = tk[:, idx], tv[:, idx]
    s = torch.matmul(tq, kr.transpose(-1, -2)) / np.sqrt(D)
    i = torch.arange(Lq)[:, None]
    j = torch.arange(Lk)[None, :]
    vis = torch.ones((B, 1, Lq, Lk), dtype=torch.bool)
    if causal:
        vis = vis & (j <= q_offset + i)
    if seg_q is not None:
        vis = vis & (torch.tensor(seg_q)[:, None, :, None] == torch.tensor(seg_k)[:, None, None, :])
    s = torch.where(vis, s, torch.tensor(-np.inf, dtype=torch.float64))
    m = s.amax(dim=-1, keepdim=True)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m)).detach()
    e = torch.where(vis, torch.exp(s - m), torch.zeros_like(s))
    z = e.sum(dim=-1, keepdim=True)
    p = e / torch.where(z > 0, z, torch.ones_like(z))
    o = torch.matmul(p, vr)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_bwd_autograd(orc):
    """dq, dk, dv within 1e-12 (relative to the largest gradient) of automatic
    differentiation of the explicit math path, on tiny inputs covering GQA
    ratios 1-4, causal on and off, q_offset 0 and 3, segments and empty rows."""
    for n in range(len(BWD_CASES)):
        q, k, v, do, kw = _bwd_case(n)
        dq, dk, dv = orc.bwd(q, k, v, do, **kw)
        rq, rk, rv = _autograd_math_path(q, k, v, do, **kw)
        for name, a, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            err = np.max(np.abs(a - r)) / max(1.0, np.max(np.abs(r)))
            assert err < 1e-12, "%s differs from autograd (case %d): %g" % (name, n, err)


def pin_bwd_finite_differences(orc):
    """Central differences of the oracle's forward loss sum(o * dout) with
    respect to single entries of q, k and v agree with the gradients to 1e-7
    (relative; step 2^-12 on entries that are multiples of 2^-8, exact in fp32)."""
    B, Hq, Hkv, Lq, Lk, D = 1, 4, 2, 8, 10, 8
    q, k, v = (_grid(x) for x in _case(B, Hq, Hkv, Lq, Lk, D, 151))
    do = _rand((B, Hq, Lq, D), 152)
    kw = dict(causal=True, q_offset=2)
    dq, dk, dv = orc.bwd(q, k, v, do, **kw)

    def loss(q_, k_, v_):
        o, _ = orc.attn(q_, k_, v_, **kw)
        return float(np.sum(o * do.astype(np.float64)))

    h = 2.0 ** -12
    rng = np.random.default_rng(153)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            ix = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[ix] += h
            xm[ix] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[ix]) <= 1e-7 * max(1.0, abs(g[ix])), "d%s%s: fd %r vs %r" % (name, ix, fd, g[ix])


def pin_bwd_sum_identities(orc):
    """Exact identities of the softmax gradient: the ds_ij of a row sum to zero,
    so sum_j dk_j = 0 for every key/value head; the p_ij of a non-empty row sum
    to one, so sum_j dv_j = sum of dout over the non-empty rows of the heads that
    share the key/value head; a row with a single visible key (causal row 0) has
    dq = 0."""
    q, k, v, do, kw = _bwd_case(4)
    dq, dk, dv = orc.bwd(q, k, v, do, **kw)
    _, lse = orc.attn(q, k, v, **kw)
    Hq, Hkv = q.shape[1], k.shape[1]
    rep = Hq // Hkv
    scale = np.max(np.abs(dk))
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-13 * max(1.0, scale) * k.shape[2]
    nonempty = np.isfinite(lse)[..., None]
    want = (do.astype(np.float64) * nonempty).reshape(q.shape[0], Hkv, rep, q.shape[2], -1).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - want)) < 1e-12
    q0, k0, v0 = _case(1, 4, 2, 6, 6, 8, 161)
    do0 = _rand((1, 4, 6, 8), 162)
    dq0 = orc.bwd_dq(q0, k0, v0, do0)
    assert np.max(np.abs(dq0[:, :, 0])) < 1e-15


def pin_bwd_gqa_equals_repeat(orc):
    """The GQA gradient equals the gradient taken on K/V repeated per query head
    with dk, dv then summed over each group of heads (1e-13); dq is identical."""
    q, k, v = _case(1, 8, 2, 11, 11, 8, 171)
    do = _rand(q.shape, 172)
    dq, dk, dv = orc.bwd(q, k, v, do)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    dq2, dk2, dv2 = orc.bwd(q, kr, vr, do)
    assert np.array_equal(dq, dq2)
    assert np.max(np.abs(dk - dk2.reshape(1, 2, 4, 11, 8).sum(axis=2))) < 1e-13
    assert np.max(np.abs(dv - dv2.reshape(1, 2, 4, 11, 8).sum(axis=2))) < 1e-13


def pin_bwd_subsets(orc):
    """Gradients for a subset of rows (dq) or keys (dk, dv) equal the full run
    bitwise."""
    q, k, v, do, kw = _bwd_case(1)
    dq, dk, dv = orc.bwd(q, k, v, do, **kw)
    rows, keys = np.array([5, 0, 3]), np.array([8, 2, 0, 7])
    assert np.array_equal(orc.bwd_dq(q, k, v, do, rows=rows, **kw), dq[:, :, rows])
    dks, dvs = orc.bwd_dkdv(q, k, v, do, keys=keys, **kw)
    assert np.array_equal(dks, dk[:, :, keys]) and np.array_equal(dvs, dv[:, :, keys])


BWD_PINS = [pin_bwd_autograd, pin_bwd_finite_differences, pin_bwd_sum_identities, pin_bwd_gqa_equals_repeat,
            pin_bwd_subsets]


ALL_PINS = [pin_brute_force, pin_rows_sum_to_one, pin_gqa_equals_repeat, pin_one_segment_equals_none,
            pin_packed_equals_per_segment, pin_prefix_branch, pin_merge_identity, pin_zero_q,
            pin_first_row, pin_two_keys, pin_constant_v, pin_key_shift, pin_linear_in_v,
            pin_row_subset] + BWD_PINS
