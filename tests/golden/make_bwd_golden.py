"""Writes tests/golden/bwd_long_sums.npz: the fp64 oracle's dk and dv at keys
whose gradient sums run over (nearly) every query row of every head, for the
two full-size backward workloads. A key's dk and dv need the softmax statistics
of every row that sees it, which is a full pass of the oracle over the
sequence (minutes of CPU). So the values are computed once, by this script,
which calls only the oracle, and stored.

Inputs (the same the GPU tests draw; a hash of their bytes is stored with the
values so that a change of the generator is caught):
  fp32:  synth.gqa(1, 16, 4, 30468, seed=0), dout synth.Grad(seed=1); causal.
  bf16 packed: synth.gqa(1, 16, 4, 131072, seed=0, dtype="bf16"), dout
         synth.Grad(seed=1, dtype="bf16"), segment ids from
         synth.segment_lengths(131072, 2048, 32768, seed=1); causal within segments.
Keys: fp32, the first keys, the 32- and 64-key tile edges among the first 256
keys, and keys spread over the sequence; packed, the first 16 keys of every
segment. Values are stored as float32 (their relative rounding, 6e-8, is far
below the test bars).

Usage: python tests/golden/make_bwd_golden.py   (about 15-30 minutes on 8 cores)
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(HERE, "bwd_long_sums.npz")


def input_hash(*arrays):
    """sha256 of each array's shape and of every 997th element (a change of the
    random generator or of the rounding changes these)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(repr(a.shape).encode())
        h.update(np.ascontiguousarray(np.ravel(a)[::997]).tobytes())
    return h.hexdigest()


def fp32_keys(L):
    ks = {0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 255, 256}
    ks.update(int(x) for x in np.linspace(512, L - 512, 18).astype(np.int64))
    return np.array(sorted(ks), dtype=np.int64)


def packed_keys(lens):
    return np.concatenate([np.arange(a, a + 16) for a, _ in synth.segment_bounds(lens)]).astype(np.int64)


def main():
    out = {}
    t0 = time.time()
    L = 30468
    x = synth.gqa(1, 16, 4, L, seed=0, dtype="f32")
    g = synth.Grad(x.q.shape, seed=1, dtype="f32")
    keys = fp32_keys(L)
    dk, dv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, keys=keys)
    out["f32_keys"] = keys
    out["f32_dk"] = dk.astype(np.float32)
    out["f32_dv"] = dv.astype(np.float32)
    out["f32_hash"] = np.array(input_hash(x.q, x.k, x.v, g.values))
    print("fp32 L=%d: %d keys, %.0f s" % (L, len(keys), time.time() - t0), flush=True)
    del x, g

    t0 = time.time()
    L = 131072
    lens = synth.segment_lengths(L, 2048, 32768, seed=1)
    ids = synth.segment_ids(lens)[None]
    x = synth.gqa(1, 16, 4, L, seed=0, dtype="bf16")
    g = synth.Grad(x.q.shape, seed=1, dtype="bf16")
    keys = packed_keys(lens)
    dk, dv = oracle.bwd_dkdv(x.q, x.k, x.v, g.values, seg_q=ids, seg_k=ids, keys=keys)
    out["packed_keys"] = keys
    out["packed_dk"] = dk.astype(np.float32)
    out["packed_dv"] = dv.astype(np.float32)
    out["packed_hash"] = np.array(input_hash(x.q, x.k, x.v, g.values, ids))
    print("bf16 packed L=%d: %d keys, %.0f s" % (L, len(keys), time.time() - t0), flush=True)
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
