"""Gradients of exact attention by the chain rule, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages quote their speed-ups for training (FlashAttention (UR), "Experimental
results"; FlashAttention-2 (HI), "Performance and efficiency"), which needs the
gradients of the attention output, but they print no backward algorithm.  What
is computed here is therefore the derivative of the forward definition
(``attention.attention``) written out, for a loss L whose gradient with respect
to O is dO:

    S = scale * Q K^T,  P = softmax(S) along each row over the allowed keys,
    O = P V

    dV = P^T dO                          (O is linear in V)
    dP = dO V^T                          (O is linear in P)
    dS_ij = P_ij (dP_ij - D_i),  D_i = sum_k P_ik dP_ik
                                         (the Jacobian of a row softmax)
    dQ = scale * dS K,   dK = scale * dS^T Q

Masked scores are constants (-inf), so they carry no gradient: their P is 0
and so is their dS.  A row with no allowed key has O = 0 whatever Q, K, V are,
so it contributes nothing.  With grouped heads (``attention.kv_head``) a
key/value head's gradient is the sum over the query heads that read it.

D_i equals dO_i . O_i (sum_k P_ik dO_i . V_k = dO_i . sum_k P_ik V_k); the
oracle uses the softmax Jacobian's own form above, not that identity.
"""
import numpy as np

from .attention import _f64, _valid_len, kv_head, softmax_matrix

__all__ = ["attention_backward"]


def attention_backward(q, k, v, do, scale, causal=False, seqlens=None, row_block=1024):
    """(dQ [B, H, N, d], dK [B, H_kv, N, d], dV [B, H_kv, N, d]) in float64.

    q and do are [B, H, N, d]; k and v are [B, H_kv, N, d] with H_kv dividing H.
    Masks as in ``attention.attention`` (causal j <= i; keys j >= seqlens[b]
    dropped, lengths clamped to [0, N]).  The rows of a head are taken
    ``row_block`` at a time, which only bounds the memory: dQ of a row needs only
    that row, and dK, dV are sums over rows.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    if do.shape != q.shape or k.shape[0] != B or k.shape[3] != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("q, k, v, do shapes disagree")
    H_kv = k.shape[1]
    kv_head(0, H, H_kv)   # checks that H_kv divides H
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros((B, H_kv, N, v.shape[3]))
    for b in range(B):
        L = _valid_len(seqlens, b, N)
        for h in range(H):
            g = kv_head(h, H, H_kv)
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                p, _, _ = softmax_matrix(q[b, h, rows], k[b, g], scale, rows, L, causal)   # [R, N]
                dp = do[b, h, rows] @ v[b, g].T
                dsum = (p * dp).sum(axis=1)
                ds = p * (dp - dsum[:, None])
                dv[b, g] += p.T @ do[b, h, rows]
                dq[b, h, rows] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv
