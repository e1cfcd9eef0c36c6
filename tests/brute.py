"""Brute-force attention for tiny inputs, independent of the oracle's code.

It follows the math path the pages describe (kev pull request 202, "Why fp32
fell to the L x L kernel"): K and V are first repeated to every query head
(the repetition of "The change"), the full score matrix and an explicit 0/1
visibility matrix are built, and the softmax is taken straight from its
definition, exp(s) / sum exp(s), with no max shift, in 50-digit arithmetic.
"""
import mpmath
import numpy as np


def attn(q, k, v, *, causal=True, q_offset=0, seg_q=None, seg_k=None, dps=50):
    mpmath.mp.dps = dps
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    rep = Hq // Hkv
    # explicit repetition: query head h reads key/value head h // rep
    k_rep = np.stack([k[:, h // rep] for h in range(Hq)], axis=1)
    v_rep = np.stack([v[:, h // rep] for h in range(Hq)], axis=1)
    inv_sqrt_d = 1 / mpmath.sqrt(D)
    o = np.zeros((B, Hq, Lq, D))
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        vis = [[1 if ((not causal or j <= q_offset + i) and
                      (seg_q is None or int(seg_q[b][i]) == int(seg_k[b][j]))) else 0
                for j in range(Lk)] for i in range(Lq)]
        for h in range(Hq):
            S = [[inv_sqrt_d * mpmath.fsum(mpmath.mpf(float(q[b, h, i, d])) * mpmath.mpf(float(k_rep[b, h, j, d]))
                                            for d in range(D))
                  for j in range(Lk)] for i in range(Lq)]
            for i in range(Lq):
                E = [vis[i][j] * mpmath.exp(S[i][j]) for j in range(Lk)]
                Z = mpmath.fsum(E)
                if Z == 0:
                    lse[b, h, i] = -np.inf
                    continue
                lse[b, h, i] = float(mpmath.log(Z))
                for d in range(D):
                    o[b, h, i, d] = float(mpmath.fsum(E[j] * mpmath.mpf(float(v_rep[b, h, j, d])) for j in range(Lk)) / Z)
    return o, lse
