"""MI355X (gfx950) exact causal grouped-query attention, memory linear in L:
the forward, the lse merge of split key sets, and the backward.

A thin ctypes binding over ``libgqa_attn.so`` (C ABI in ``include/gqa_attn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata and passes device pointers, sizes and the current
HIP stream. PyTorch is used for device memory and streams only. There is no
fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa_attn.so")

GQA_F32, GQA_BF16, GQA_F16 = 0, 1, 2
STATUS = {0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_SHAPE", 3: "GQA_ERR_UNSUPPORTED",
          4: "GQA_ERR_ALIGN", 5: "GQA_ERR_LAUNCH", 6: "GQA_ERR_ALIAS", 7: "GQA_ERR_WORKSPACE"}
EXPORTS = ("gqa_attn_fwd", "gqa_attn_merge", "gqa_attn_bwd", "gqa_attn_fwd_split", "gqa_attn_fwd_split_noalloc",
           "gqa_attn_split_workspace", "gqa_attn_split_count", "gqa_attn_seg_index_bytes", "gqa_attn_seg_index",
           "gqa_attn_fwd_indexed", "gqa_attn_bwd_indexed", "gqa_attn_strerror", "gqa_attn_version")
SEG_BLOCK = 16  # ids per entry of an id-range index (gqa_attn_seg_index)
NOALLOC_SCRATCH_BYTES = 64 << 20  # GQA_NOALLOC_SCRATCH_BYTES

_lib = None


class GqaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


def load_library():
    """Load libgqa_attn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgqa_attn.so is not built at %s; run __graft_entry__.build() "
                               "or python -m long_context_causal_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        i64, p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gqa_attn_fwd.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, c_int, c_int, p]
        lib.gqa_attn_fwd.restype = c_int
        lib.gqa_attn_merge.argtypes = [p, p, p, p, p, p, i64, i64, c_int, p]
        lib.gqa_attn_merge.restype = c_int
        lib.gqa_attn_bwd.argtypes = [p] * 10 + [i64] * 7 + [p, p, c_int, c_int, p]
        lib.gqa_attn_bwd.restype = c_int
        lib.gqa_attn_fwd_split.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, c_int, c_int,
                                           c_int, p, i64, p]
        lib.gqa_attn_fwd_split.restype = c_int
        lib.gqa_attn_fwd_split_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, c_int,
                                                   c_int, c_int, p]
        lib.gqa_attn_fwd_split_noalloc.restype = c_int
        lib.gqa_attn_split_workspace.argtypes = [i64, i64, i64, i64, c_int]
        lib.gqa_attn_split_workspace.restype = i64
        lib.gqa_attn_split_count.argtypes = [i64, i64, i64, i64, i64, c_int]
        lib.gqa_attn_split_count.restype = c_int
        lib.gqa_attn_seg_index_bytes.argtypes = [i64, i64]
        lib.gqa_attn_seg_index_bytes.restype = i64
        lib.gqa_attn_seg_index.argtypes = [p, i64, i64, p, i64, p]
        lib.gqa_attn_seg_index.restype = c_int
        lib.gqa_attn_fwd_indexed.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, p, p, c_int,
                                             c_int, p]
        lib.gqa_attn_fwd_indexed.restype = c_int
        lib.gqa_attn_bwd_indexed.argtypes = [p] * 10 + [i64] * 7 + [p, p, p, p, c_int, c_int, p]
        lib.gqa_attn_bwd_indexed.restype = c_int
        lib.gqa_attn_strerror.argtypes = [c_int]
        lib.gqa_attn_strerror.restype = ctypes.c_char_p
        lib.gqa_attn_version.argtypes = []
        lib.gqa_attn_version.restype = c_int
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().gqa_attn_strerror(int(code)).decode()


def version() -> tuple[int, int]:
    v = load_library().gqa_attn_version()
    return v >> 16, v & 0xFFFF


def fwd_raw(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype, stream) -> int:
    """Direct call of gqa_attn_fwd with integer pointers; returns the status code."""
    return load_library().gqa_attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                                       int(causal), int(dtype), stream)


def bwd_raw(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
            causal, dtype, stream) -> int:
    """Direct call of gqa_attn_bwd with integer pointers; returns the status code."""
    return load_library().gqa_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D,
                                       q_offset, seg_q, seg_k, int(causal), int(dtype), stream)


def seg_index_bytes(B, L) -> int:
    """Bytes of the id-range index of B rows of L segment ids."""
    return int(load_library().gqa_attn_seg_index_bytes(B, L))


def seg_index_raw(seg, B, L, index, index_bytes, stream) -> int:
    """Direct call of gqa_attn_seg_index with integer pointers; returns the status code."""
    return load_library().gqa_attn_seg_index(seg, B, L, index, index_bytes, stream)


def fwd_indexed_raw(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, seg_q_index, seg_k_index,
                    causal, dtype, stream) -> int:
    """Direct call of gqa_attn_fwd_indexed with integer pointers; returns the status code."""
    return load_library().gqa_attn_fwd_indexed(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                                               seg_q_index, seg_k_index, int(causal), int(dtype), stream)


def bwd_indexed_raw(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                    seg_q_index, seg_k_index, causal, dtype, stream) -> int:
    """Direct call of gqa_attn_bwd_indexed with integer pointers; returns the status code."""
    return load_library().gqa_attn_bwd_indexed(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D,
                                               q_offset, seg_q, seg_k, seg_q_index, seg_k_index, int(causal),
                                               int(dtype), stream)


def fwd_split_raw(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype, n_split,
                  workspace, workspace_bytes, stream) -> int:
    """Direct call of gqa_attn_fwd_split with integer pointers; returns the status code."""
    return load_library().gqa_attn_fwd_split(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                                             int(causal), int(dtype), int(n_split), workspace, workspace_bytes,
                                             stream)


def fwd_split_noalloc_raw(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype, n_split,
                          stream) -> int:
    """Direct call of gqa_attn_fwd_split_noalloc with integer pointers; returns the status code."""
    return load_library().gqa_attn_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                                                     int(causal), int(dtype), int(n_split), stream)


def split_workspace(B, Hq, Lq, D, n_split) -> int:
    """Workspace bytes of a split-KV forward with n_split ranges."""
    return int(load_library().gqa_attn_split_workspace(B, Hq, Lq, D, int(n_split)))


def split_count(B, Hq, Hkv, Lq, Lk, dtype) -> int:
    """The library's recommended split count for a shape (dtype: GQA_* code)."""
    return int(load_library().gqa_attn_split_count(B, Hq, Hkv, Lq, Lk, int(dtype)))


def merge_raw(o1, lse1, o2, lse2, o, lse, rows, D, dtype, stream) -> int:
    """Direct call of gqa_attn_merge with integer pointers; returns the status code."""
    return load_library().gqa_attn_merge(o1, lse1, o2, lse2, o, lse, rows, D, int(dtype), stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return GQA_F32
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float16:
        return GQA_F16
    raise TypeError("tensors must be float32, bfloat16 or float16, got %s" % t.dtype)


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def seg_index(seg, *, out=None, stream=None):
    """Id-range index of int32 segment ids seg [B, L]: for each block of 16
    consecutive ids of a row their (min, max), an int32 tensor [B, ceil(L/16), 2].
    fwd() and bwd() take it (seg_q_index, seg_k_index) in place of scanning the
    ids in every workgroup; results are the same bit for bit."""
    import torch
    _check_dev(seg, out)
    if seg.dtype != torch.int32 or seg.dim() != 2:
        raise TypeError("segment ids must be an int32 [B, L] tensor")
    B, L = seg.shape
    shape = (B, (L + SEG_BLOCK - 1) // SEG_BLOCK, 2)
    out = torch.empty(shape, dtype=torch.int32, device=seg.device) if out is None else out
    if tuple(out.shape) != shape or out.dtype != torch.int32:
        raise ValueError("index must be an int32 tensor of shape %s" % (shape,))
    rc = seg_index_raw(seg.data_ptr(), B, L, out.data_ptr(), out.numel() * 4, _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return out


def _check_index(idx, B, L, name):
    import torch
    if idx is None:
        return None
    _check_dev(idx)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, (L + SEG_BLOCK - 1) // SEG_BLOCK, 2):
        raise ValueError("%s must be seg_index() of the matching ids" % name)
    return idx.data_ptr()


def fwd(q, k, v, *, causal=True, q_offset=0, seg_q=None, seg_k=None, out=None, lse=None, stream=None,
        seg_q_index=None, seg_k_index=None):
    """Attention forward: q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] (fp32, bf16 or fp16, same dtype),
    optional int32 segment ids seg_q [B,Lq] / seg_k [B,Lk]. Returns (o, lse) with
    o like q and lse [B,Hq,Lq] fp32. Work is enqueued on `stream` (default: the
    current stream). seg_q_index / seg_k_index: optional seg_index() of the ids
    (the call then goes to gqa_attn_fwd_indexed)."""
    import torch
    _check_dev(q, k, v, seg_q, seg_k, out, lse)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Lq,D] and k, v [B,Hkv,Lk,D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q and k/v disagree in batch or head size")
    if (seg_q is None) != (seg_k is None):
        raise ValueError("give both segment-id tensors or neither")
    if seg_q is not None:
        if seg_q.dtype != torch.int32 or seg_k.dtype != torch.int32:
            raise TypeError("segment ids must be int32")
        if seg_q.numel() != B * Lq or seg_k.numel() != B * Lk:
            raise ValueError("segment ids must be [B,Lq] and [B,Lk]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
        raise ValueError("out must match q and lse must be [B,Hq,Lq] float32")
    qi, ki = _check_index(seg_q_index, B, Lq, "seg_q_index"), _check_index(seg_k_index, B, Lk, "seg_k_index")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Lq, Lk, D,
            int(q_offset), None if seg_q is None else seg_q.data_ptr(), None if seg_k is None else seg_k.data_ptr())
    if qi is None and ki is None:
        rc = fwd_raw(*args, causal, dt, _stream_ptr(stream))
    else:
        rc = fwd_indexed_raw(*args, qi, ki, causal, dt, _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return out, lse


def merge(o1, lse1, o2, lse2, *, out=None, out_lse=None, stream=None):
    """Log-sum-exp merge of two results over disjoint key sets of the same rows
    (o* [..., D], lse* [...] float32). out/out_lse may be o1/lse1 (in place)."""
    import torch
    _check_dev(o1, lse1, o2, lse2, out, out_lse)
    if o1.shape != o2.shape or lse1.shape != lse2.shape or tuple(o1.shape[:-1]) != tuple(lse1.shape):
        raise ValueError("merge operands disagree in shape")
    if lse1.dtype != torch.float32 or lse2.dtype != torch.float32 or o2.dtype != o1.dtype:
        raise TypeError("lse must be float32 and o1/o2 share a dtype")
    dt = _dtype_code(o1)
    out = torch.empty_like(o1) if out is None else out
    out_lse = torch.empty_like(lse1) if out_lse is None else out_lse
    if out.shape != o1.shape or out.dtype != o1.dtype or out_lse.shape != lse1.shape or \
            out_lse.dtype != torch.float32:
        raise ValueError("out must match o1 and out_lse must match lse1 (float32)")
    rc = merge_raw(o1.data_ptr(), lse1.data_ptr(), o2.data_ptr(), lse2.data_ptr(), out.data_ptr(),
                   out_lse.data_ptr(), lse1.numel(), o1.shape[-1], dt, _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return out, out_lse


def bwd(q, k, v, o, lse, dout, *, causal=True, q_offset=0, seg_q=None, seg_k=None, dq=None, dk=None, dv=None,
        delta=None, stream=None, seg_q_index=None, seg_k_index=None):
    """Attention backward: gradients with respect to q, k and v of a loss whose
    gradient with respect to the forward output o is `dout` (like q). o and lse
    are the forward's outputs for the same arguments (or the merged ones of a
    split key set). Returns (dq, dk, dv, delta): dq like q, dk and dv like k,
    delta [B,Hq,Lq] float32 (the row dot products dout . o). seg_q_index /
    seg_k_index: optional seg_index() of the ids (gqa_attn_bwd_indexed)."""
    import torch
    _check_dev(q, k, v, o, lse, dout, seg_q, seg_k, dq, dk, dv, delta)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B,Hq,Lq,D] and k, v [B,Hkv,Lk,D]")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o and dout must share a dtype")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q and k/v disagree in batch or head size")
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
        raise ValueError("lse must be [B,Hq,Lq] float32")
    if (seg_q is None) != (seg_k is None):
        raise ValueError("give both segment-id tensors or neither")
    if seg_q is not None:
        if seg_q.dtype != torch.int32 or seg_k.dtype != torch.int32:
            raise TypeError("segment ids must be int32")
        if seg_q.numel() != B * Lq or seg_k.numel() != B * Lk:
            raise ValueError("segment ids must be [B,Lq] and [B,Lk]")
    dt = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if delta is None else delta
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape or delta.shape != (B, Hq, Lq):
        raise ValueError("gradient buffers must match q, k, v and delta [B,Hq,Lq]")
    if any(t.dtype != q.dtype for t in (dq, dk, dv)) or delta.dtype != torch.float32:
        raise TypeError("gradients share q's dtype; delta is float32")
    qi, ki = _check_index(seg_q_index, B, Lq, "seg_q_index"), _check_index(seg_k_index, B, Lk, "seg_k_index")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, Hq, Hkv, Lq, Lk, D, int(q_offset),
            None if seg_q is None else seg_q.data_ptr(), None if seg_k is None else seg_k.data_ptr())
    if qi is None and ki is None:
        rc = bwd_raw(*args, causal, dt, _stream_ptr(stream))
    else:
        rc = bwd_indexed_raw(*args, qi, ki, causal, dt, _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return dq, dk, dv, delta


def fwd_split(q, k, v, *, causal=True, q_offset=0, seg_q=None, seg_k=None, n_split=None, out=None, lse=None,
              workspace=None, stream=None):
    """Split-KV forward: the same result as fwd() (up to the order of fp32
    sums), for short query blocks over long key sequences. n_split defaults to
    the library's recommendation for the shape; workspace (a uint8 device
    tensor) is allocated when not given. Returns (o, lse)."""
    import torch
    _check_dev(q, k, v, seg_q, seg_k, out, lse, workspace)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Lq,D] and k, v [B,Hkv,Lk,D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q and k/v disagree in batch or head size")
    if (seg_q is None) != (seg_k is None):
        raise ValueError("give both segment-id tensors or neither")
    if seg_q is not None:
        if seg_q.dtype != torch.int32 or seg_k.dtype != torch.int32:
            raise TypeError("segment ids must be int32")
        if seg_q.numel() != B * Lq or seg_k.numel() != B * Lk:
            raise ValueError("segment ids must be [B,Lq] and [B,Lk]")
    dt = _dtype_code(q)
    if n_split is None:
        n_split = split_count(B, Hq, Hkv, Lq, Lk, dt)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
        raise ValueError("out must match q and lse must be [B,Hq,Lq] float32")
    nbytes = split_workspace(B, Hq, Lq, D, n_split)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Lq,
                       Lk, D, int(q_offset), None if seg_q is None else seg_q.data_ptr(),
                       None if seg_k is None else seg_k.data_ptr(), causal, dt, n_split, workspace.data_ptr(),
                       workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return out, lse


def fwd_split_noalloc(q, k, v, out, lse, *, causal=True, q_offset=0, seg_q=None, seg_k=None, n_split=0,
                      stream=None):
    """Split-KV forward through the allocation-free entry point: the partial
    results use the library's static per-GPU scratch, so neither the call nor
    this binding allocates (out and lse are the caller's). n_split = 0 takes
    the library's count that fits the scratch. Calls overlapping on one GPU race."""
    import torch
    _check_dev(q, k, v, seg_q, seg_k, out, lse)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Lq,D] and k, v [B,Hkv,Lk,D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q and k/v disagree in batch or head size")
    if (seg_q is None) != (seg_k is None):
        raise ValueError("give both segment-id tensors or neither")
    if seg_q is not None:
        if seg_q.dtype != torch.int32 or seg_k.dtype != torch.int32:
            raise TypeError("segment ids must be int32")
        if seg_q.numel() != B * Lq or seg_k.numel() != B * Lk:
            raise ValueError("segment ids must be [B,Lq] and [B,Lk]")
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32:
        raise ValueError("out must match q and lse must be [B,Hq,Lq] float32")
    rc = fwd_split_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                               Hkv, Lq, Lk, D, int(q_offset), None if seg_q is None else seg_q.data_ptr(),
                               None if seg_k is None else seg_k.data_ptr(), causal, _dtype_code(q), n_split,
                               _stream_ptr(stream))
    if rc != 0:
        raise GqaError(rc, strerror(rc))
    return out, lse
