"""The exact attention forward pass by its definition, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed: Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, computed
as standard attention does it, with the score matrix S held in full
(FlashAttention (UR), section "The problem of standard attention").  The softmax
runs along each row of S, over the keys.  ``scale`` is passed in rather than
derived from d, so the caller can hand over the exact float32 value a kernel
receives (for d = 64 it is 1/8; for d = 128, float32(1/sqrt(128))).

Masking is listed among the fused operations (FlashAttention (UR), section
"Fusing the operations into one CUDA kernel") without a definition; the reading
used here:

* causal: query i may attend to key j only when j <= i (queries and keys share
  the index range 0..N-1, so the two usual alignments coincide);
* key padding: batch b has ``seqlens[b]`` valid keys, values clamped to [0, N];
  keys j >= seqlens[b] are dropped for every query of that batch.  Query rows are
  not dropped: rows i >= seqlens[b] are still computed over the valid keys.
* both masks combine with AND.  A row with no allowed key gets O = 0 and
  LSE = -inf.

LSE (row log-sum-exp, natural log) is not on the pages; it is defined here as
LSE_i = log(sum_{j allowed} exp(s_ij)), computed stably as m_i + log(l_i).
"""
import numpy as np

__all__ = ["allowed_mask", "softmax_matrix", "attention_rows", "attention", "kv_head", "decode_allowed", "attention_decode",
           "merge_partials", "e4m3_decode", "attention_fp8"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _valid_len(seqlens, b, n_keys):
    if seqlens is None:
        return n_keys
    return int(min(max(int(seqlens[b]), 0), n_keys))


def allowed_mask(rows, n_keys, valid_len, causal):
    """Boolean [len(rows), n_keys]: True where query row i may attend to key j."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys, dtype=np.int64)
    allowed = np.broadcast_to(j[None, :] < valid_len, (rows.size, n_keys)).copy()
    if causal:
        allowed &= j[None, :] <= rows[:, None]
    return allowed


def softmax_matrix(q_rows, k_head, scale, rows, valid_len, causal):
    """Rows of P = softmax(scale * Q K^T) for one head, masked entries exactly 0.

    q_rows [R, d] holds the query rows listed in ``rows``; k_head [N, d] holds all
    keys of the head.  S is materialised for these rows.  Returns (P, m, l) with
    m the row max of the allowed scores and l = sum_j exp(s_ij - m_i); for a row
    with no allowed key P is all zero, m = -inf and l = 0.
    """
    q_rows = _f64(q_rows)
    k_head = _f64(k_head)
    s = float(scale) * (q_rows @ k_head.T)                    # S, [R, N]
    allowed = allowed_mask(rows, k_head.shape[0], valid_len, causal)
    nonempty = allowed.any(axis=1)
    s_allowed = np.where(allowed, s, -np.inf)
    m = s_allowed.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    shift = np.where(nonempty, m, 0.0)
    w = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - shift[:, None]), 0.0)
    l = w.sum(axis=1)
    p = np.divide(w, l[:, None], out=np.zeros_like(w), where=nonempty[:, None])
    return p, m, l


def kv_head(h, n_heads, n_kv_heads):
    """Key/value head read by query head h.

    FlashAttention (UR), section "FlashAttention-2 (2023)", names multi-query
    attention (all query heads share one key/value head) among the supported
    architectures.  The reading used here is the grouped form that contains it:
    with H_kv key/value heads, H_kv dividing H, query heads
    g*(H/H_kv) .. (g+1)*(H/H_kv)-1 share key/value head g.  H_kv = H is ordinary
    multi-head attention and H_kv = 1 is multi-query attention.
    """
    if n_kv_heads < 1 or n_heads % n_kv_heads:
        raise ValueError("the number of key/value heads must divide the number of query heads")
    return h // (n_heads // n_kv_heads)


def attention_rows(q, k, v, scale, causal, seqlens, b, h, rows):
    """O and LSE of the listed query rows of head (b, h) only.

    q is [B, H, N, d]; k, v are [B, H_kv, N, d] (H_kv = H, or a divisor of H for
    grouped / multi-query attention, see ``kv_head``).  Returns O [len(rows), d]
    and LSE [len(rows)] in float64.  Used where the whole output is too large to
    check one by one.
    """
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = k.shape[2]
    valid = _valid_len(seqlens, b, n_keys)
    g = kv_head(h, q.shape[1], k.shape[1])
    p, m, l = softmax_matrix(_f64(q[b, h][rows]), k[b, g], scale, rows, valid, causal)
    o = p @ _f64(v[b, g])
    nonempty = l > 0
    lse = np.full(rows.size, -np.inf)
    lse[nonempty] = m[nonempty] + np.log(l[nonempty])
    return o, lse


def attention(q, k, v, scale, causal=False, seqlens=None, row_block=2048):
    """Full forward pass: O [B, H, N, d] and LSE [B, H, N], float64.

    k and v may have fewer heads than q (grouped / multi-query attention, see
    ``kv_head``).

    The score matrix is built per head, ``row_block`` query rows at a time, which
    only bounds the memory: the softmax of a row never looks at another row.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H, N, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("q, k, v shapes disagree")
    kv_head(0, H, k.shape[1])   # checks that H_kv divides H
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = attention_rows(q, k, v, scale, causal, seqlens, b, h, rows)
    return o, lse


# ---------------------------------------------------------------------------------
# Decoding: a few new queries against a long key/value cache.
# ---------------------------------------------------------------------------------
def decode_allowed(n_q, n_keys, valid_len, causal):
    """Boolean [n_q, n_keys] mask of the decode problem.

    The pages mention inference kernels built on the same method (FlashAttention
    (UR), section on specialised solutions) without defining their masks.  The
    reading used here: batch b holds valid_len valid keys (positions
    0 .. valid_len-1, the cache); its n_q queries are the LAST n_q positions of
    that sequence, query i at position valid_len - n_q + i.  Every query sees
    the valid keys; causal additionally drops keys after its own position
    (j <= valid_len - n_q + i).  With n_q = n_keys = valid_len this is the
    causal mask of ``attention``.
    """
    i = np.arange(n_q, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    allowed = np.broadcast_to(j < valid_len, (n_q, n_keys)).copy()
    if causal:
        allowed &= j <= valid_len - n_q + i
    return allowed


def attention_decode(q, k, v, scale, causal=False, seqlens=None):
    """O [B, H, Nq, d] and LSE [B, H, Nq] of the decode problem, float64.

    q is [B, H, Nq, d]; k and v are [B, H_kv, Nk, d] (H_kv divides H, see
    ``kv_head``); seqlens [B] gives each batch's valid cache length (clamped to
    [0, Nk]; None = Nk).  The softmax is the definition itself: S in full, row
    max shift, normalised weights, rows with no key give O = 0, LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = _valid_len(seqlens, b, Nk)
        allowed = decode_allowed(Nq, Nk, L, causal)
        nonempty = allowed.any(axis=1)
        for h in range(H):
            g = kv_head(h, H, k.shape[1])
            s = float(scale) * (q[b, h] @ k[b, g].T)
            m = np.where(allowed, s, -np.inf).max(axis=1, initial=-np.inf)
            shift = np.where(nonempty, m, 0.0)
            w = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - shift[:, None]), 0.0)
            l = w.sum(axis=1)
            p = np.divide(w, l[:, None], out=np.zeros_like(w), where=nonempty[:, None])
            o[b, h] = p @ v[b, g]
            lse[b, h, nonempty] = m[nonempty] + np.log(l[nonempty])
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention over disjoint key sets: o_parts [..., S, d], lse_parts [..., S].

    For partial results O_s = softmax over key set s, LSE_s = log sum over set s,
    the result over the union is LSE = log sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s (the online-softmax combination of
    FlashAttention (UR), section "Online computation of softmax", applied to
    whole partial results).  Sets with LSE_s = -inf contribute nothing; if all
    are empty, O = 0 and LSE = -inf.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=-1)
    finite = np.isfinite(m)
    mm = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - mm[..., None]), 0.0)
    tot = w.sum(axis=-1)
    lse = np.where(finite, mm + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.einsum("...s,...sd->...d", np.divide(w, np.where(finite, tot, 1.0)[..., None]), o_parts)
    return o, lse


# ---------------------------------------------------------------------------------
# FP8 inputs.
# ---------------------------------------------------------------------------------
def e4m3_decode(codes):
    """Values of 8-bit floats in the OCP e4m3 ("E4M3FN") format, float64.

    FlashAttention (UR), section "FlashAttention-3 (2024)", names FP8 support
    without a format; the reading used here is the 8-bit format with 1 sign bit,
    4 exponent bits (bias 7) and 3 mantissa bits, no infinities, and NaN only
    for the all-ones exponent-and-mantissa code (0x7F, 0xFF):
      exponent field 0:    (-1)^s * (m / 8) * 2^-6         (subnormal, and zero)
      exponent field e>0:  (-1)^s * (1 + m / 8) * 2^(e - 7)
    so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def attention_fp8(q8, k8, v8, scale, descale, causal=False, seqlens=None):
    """O and LSE (float64) of attention over FP8 inputs with per-tensor scales.

    q8, k8, v8 hold e4m3 codes (uint8, shapes as for ``attention``); the tensors
    they stand for are descale[0] * decode(q8), descale[1] * decode(k8) and
    descale[2] * decode(v8).  The result is the definition applied to those
    tensors: the exact answer for the quantised inputs.
    """
    sq, sk, sv = (float(x) for x in descale)
    return attention(sq * e4m3_decode(q8), sk * e4m3_decode(k8), sv * e4m3_decode(v8), scale, causal, seqlens)
