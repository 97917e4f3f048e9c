"""Exact-arithmetic brute force for tiny attention problems.

TEST INFRASTRUCTURE ONLY (used to pin the C oracle; never by the HIP path).

Logits are computed exactly: every fp16 value and the float32 scale are
dyadic rationals, so ``fractions.Fraction`` holds q.k and scale*(q.k) with no
rounding at all.  The only roundings are one conversion of (s_j - m) to
double before ``math.exp``, the correctly rounded sums of ``math.fsum`` and
the final divide and log.  This is a different evaluation order and precision
from the C oracle, so agreement to ~1e-12 relative pins the oracle's indexing,
masking and normalisation.

Definition followed: softmax(scale * Q K^T + causal mask) V with LSE, causal
meaning key j visible to query i iff j <= i (query length = key length, as in
the case table of "An Optimal Mapper Meets a Real GPU", section
"Experiment one").
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _exact(x: np.ndarray):
    """Nested lists of Fractions equal to the fp16 values."""
    return [[Fraction(float(t)) for t in row] for row in x]


def exact_logits(qh, kh, scale: float, causal: bool):
    """Exact scaled logits for one head: list of rows, None where masked.
    With Sq query rows and Sk keys, causal keeps key j for query i iff
    j <= i + Sk - Sq (bottom-right; j <= i when Sq = Sk)."""
    Sq, Sk = qh.shape[0], kh.shape[0]
    qe, ke = _exact(qh), _exact(kh)
    sc = Fraction(float(np.float32(scale)))
    out = []
    for i in range(Sq):
        row = []
        for j in range(Sk):
            if causal and j > i + Sk - Sq:
                row.append(None)
            else:
                row.append(sc * sum((a * b for a, b in zip(qe[i], ke[j])), Fraction(0)))
        out.append(row)
    return out


def attn_fwd(q, k, v, causal: bool, scale: float):
    """(O, LSE) as float64 arrays for fp16 inputs q [B, H, Sq, D] and
    k, v [B, H, Sk, D] (Sq = Sk for the square case)."""
    B, H, S, D = q.shape
    Sk = k.shape[2]
    o = np.zeros((B, H, S, D), dtype=np.float64)
    lse = np.zeros((B, H, S), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = exact_logits(q[b, h], k[b, h], scale, causal)
            vv = v[b, h].astype(np.float64)
            for i in range(S):
                vis = [j for j in range(Sk) if s[i][j] is not None]
                m = max(s[i][j] for j in vis)
                p = {j: math.exp(float(s[i][j] - m)) for j in vis}
                l = math.fsum(p.values())
                for d in range(D):
                    o[b, h, i, d] = math.fsum(p[j] * float(vv[j, d]) for j in vis) / l
                lse[b, h, i] = float(m) + math.log(l)
    return o, lse
