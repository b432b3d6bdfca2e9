"""Pure-Python brute force of the same definitions, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (same rule as flce_ref): an independent second
implementation with scalar loops, math.fsum/math.exp/math.log and no NumPy, used
to pin the vectorised oracle (axis, index and broadcasting mistakes there show up
as disagreements here).  Definitions as in flce_ref: scaled logits of a linear
head, log-sum-exp, target log-prob, entropy of the softmax, and the chain-rule
gradients of a*logprob + b*entropy (Liger-Kernel FSLCE commit, "Summary";
SkyRL PR 2141, "Summary").
"""
from __future__ import annotations

import math
import struct


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def solve(X, W, t, ignore_index, scale, grad_logprob=None, grad_entropy=None):
    """X: list of rows (floats), W: list of vocab rows (floats), t: list of ints."""
    M, V, H = len(X), len(W), len(W[0])
    s = float(struct.unpack("<f", struct.pack("<f", scale))[0])
    out = dict(logprob=[], lse=[], entropy=[], dX=[[0.0] * H for _ in range(M)],
               dW=[[0.0] * H for _ in range(V)])
    for m in range(M):
        z = [s * math.fsum(X[m][k] * W[v][k] for k in range(H)) for v in range(V)]
        zmax = max(z)
        lse = zmax + math.log(math.fsum(math.exp(zv - zmax) for zv in z))
        p = [math.exp(zv - lse) for zv in z]
        valid = (t[m] != ignore_index) and 0 <= t[m] < V
        ent = -math.fsum(pv * (zv - lse) for pv, zv in zip(p, z))
        out["lse"].append(lse)
        out["logprob"].append(z[t[m]] - lse if valid else 0.0)
        out["entropy"].append(ent if valid else 0.0)
        a = (grad_logprob[m] if grad_logprob is not None else 0.0) if valid else 0.0
        b = (grad_entropy[m] if grad_entropy is not None else 0.0) if valid else 0.0
        Ez = math.fsum(pv * zv for pv, zv in zip(p, z))
        for v in range(V):
            d = a * ((1.0 if v == t[m] else 0.0) - p[v]) + b * p[v] * (Ez - z[v])
            for k in range(H):
                out["dX"][m][k] += s * d * W[v][k]
                out["dW"][v][k] += s * d * X[m][k]
    return out
