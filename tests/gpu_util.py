"""Helpers for the GPU tests: move synthetic inputs to the device, run the HIP
path, and compare with the oracle element by element."""
import numpy as np
import torch

import long_context_causal_amd as gqa

# fp32 and bf16: the stated bars. fp16 (no stated bar): the bf16 bar scaled by
# the ratio of the two types' unit roundoffs, 2^-11 / 2^-8, since the rounding
# of P and of O to the input type dominates both.
TOL_O = {"f32": 2e-5, "bf16": 2e-2, "f16": 2e-2 / 8}
TOL_LSE = 1e-4
DEV = "cuda:0"
# backward (no stated bar): per gradient tensor, max|d - d_ref| <= TOL_BWD *
# max(1, max|d_ref|), the forward's bars read relative to the tensor's scale
TOL_BWD = {"f32": 2e-5, "bf16": 2e-2, "f16": 2.5e-3}


def dout_dev(g):
    """synth.Grad -> device tensor with the same bytes."""
    if g.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(g.values)).to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(g.bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if g.dtype == "bf16" else torch.float16)


def rel_err(a, ref):
    """max|a - ref| / max(1, max|ref|); a a device tensor or a host array."""
    a = a.float().cpu().numpy().astype(np.float64) if torch.is_tensor(a) else a
    return np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1.0)


def dev_tensor(values_f32, bits=None, dtype="f32"):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(values_f32)).to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def to_dev(x):
    """synth.Inputs -> (q, k, v) device tensors with the same bytes."""
    if x.dtype == "f32":
        return dev_tensor(x.q), dev_tensor(x.k), dev_tensor(x.v)
    return (dev_tensor(None, x.q_bits, x.dtype), dev_tensor(None, x.k_bits, x.dtype),
            dev_tensor(None, x.v_bits, x.dtype))


def seg_dev(s):
    return None if s is None else torch.from_numpy(np.ascontiguousarray(s, dtype=np.int32)).to(DEV)


def run(x, **kw):
    q, k, v = to_dev(x)
    o, lse = gqa.fwd(q, k, v, causal=x.causal, q_offset=x.q_offset, seg_q=seg_dev(x.seg_q),
                     seg_k=seg_dev(x.seg_k), **kw)
    torch.cuda.synchronize()
    return o, lse


def compare(o, lse, o_ref, lse_ref, dtype, rows=None, label="", tol_scale=1.0):
    """Element-wise check; o/lse device outputs, refs fp64 (optionally on a row subset).

    The bars are those stated for N(0,1) inputs (logit standard deviation 1).
    `tol_scale` widens both: fp32 stress inputs whose logits are tol_scale times
    larger pass it, since the fp32 rounding of the score dot products grows in
    proportion; 16-bit inputs keep 1 (their error is the rounding of P and O)."""
    o_h = o.float().cpu().numpy().astype(np.float64)
    l_h = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o_h, l_h = o_h[:, :, rows], l_h[:, :, rows]
    assert o_h.shape == o_ref.shape and l_h.shape == lse_ref.shape
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(l_h), np.isneginf(lse_ref)), label + ": empty-row pattern differs"
    assert np.all(o_h[~fin] == 0.0), label + ": empty rows must give o = 0"
    do = np.abs(o_h - o_ref)
    dl = np.abs(l_h[fin] - lse_ref[fin]) if fin.any() else np.zeros(1)
    worst = np.unravel_index(np.argmax(do), do.shape)
    msg = "%s: max|do| = %.3g at %s (|o| = %.3g), max|dlse| = %.3g" % (
        label, do.max(), tuple(int(i) for i in worst), abs(o_ref[worst]), dl.max())
    print(msg, flush=True)
    assert do.max() <= TOL_O[dtype] * tol_scale, msg
    assert dl.max() <= TOL_LSE * tol_scale, msg
    return do.max(), dl.max()
