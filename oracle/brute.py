"""Attention by brute force: scalar Python loops, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A second, deliberately different code path for the definition
softmax(Q K^T / sqrt(d_k)) V (FlashAttention (UR), section "The problem of
standard attention"): no numpy, no max subtraction, sums by ``math.fsum``.
Masks as in ``oracle.attention``: causal keeps j <= i; key padding keeps
j < seqlens[b] (clamped to [0, N]); an empty row gives O = 0, LSE = -inf.
Inputs must be small enough that exp(s) neither overflows nor underflows.
"""
import math


def attention_brute(q, k, v, scale, causal=False, seqlens=None):
    """q, k, v: nested sequences [B][H][N][d]. Returns (O, LSE) as nested lists."""
    B, H, N = len(q), len(q[0]), len(q[0][0])
    d = len(q[0][0][0]) if N else 0
    dv = len(v[0][0][0]) if N else 0
    o_all, lse_all = [], []
    for b in range(B):
        valid = N if seqlens is None else min(max(int(seqlens[b]), 0), N)
        o_b, lse_b = [], []
        for h in range(H):
            o_h, lse_h = [], []
            for i in range(N):
                keys = [j for j in range(N) if j < valid and (not causal or j <= i)]
                if not keys:
                    o_h.append([0.0] * dv)
                    lse_h.append(-math.inf)
                    continue
                w = []
                for j in keys:
                    s = float(scale) * math.fsum(float(q[b][h][i][c]) * float(k[b][h][j][c]) for c in range(d))
                    w.append(math.exp(s))
                total = math.fsum(w)
                o_h.append([math.fsum(wj * float(v[b][h][j][c]) for wj, j in zip(w, keys)) / total for c in range(dv)])
                lse_h.append(math.log(total))
            o_b.append(o_h)
            lse_b.append(lse_h)
        o_all.append(o_b)
        lse_all.append(lse_b)
    return o_all, lse_all
