"""Pins for an attention oracle: checks that tie it to facts outside itself.

Every pin takes ``fn(q, k, v, scale, causal, seqlens) -> (O, LSE)`` on float64
arrays of shape [B, H, N, d] and raises AssertionError when ``fn`` disagrees with
what the pages or plain mathematics fix:

* the defining formula softmax(Q K^T / sqrt(d_k)) V, row-wise softmax
  (FlashAttention (UR), section "The problem of standard attention");
* its special cases: equal value rows, Q = 0, a dominant score, N = 1, two keys;
* brute force by scalar loops on tiny inputs (``oracle.brute``);
* invariances that hold for the definition (key/value permutation, a shift of
  every key, folding the scale into Q, padding = truncation, the causal last row);
* a library routine (torch's scaled_dot_product_attention on CPU in float64);
* hand-derived fixtures in tests/golden/.

``tests/test_oracle.py`` runs them on the oracle and on deliberately broken
copies of it, so a pin set too weak to catch a plausible mistake shows up.
"""
import json
import math
import os

import numpy as np
import torch

from oracle import attention_brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASK_CASES = [(False, None), (True, None), (False, "pad"), (True, "pad")]


def _rng(seed):
    return np.random.default_rng(seed)


def _seqlens_for(kind, B, N, rng):
    if kind is None:
        return None
    return rng.integers(0, N + 1, size=B)


def _allowed(i, j, L, causal):
    return j < L and (not causal or j <= i)


def _lens(seqlens, B, N):
    return [N if seqlens is None else min(max(int(seqlens[b]), 0), N) for b in range(B)]


def pin_brute_force(fn):
    """Agreement with scalar-loop brute force for every N in 1..8 and every L in 0..N."""
    rng = _rng(11)
    for N in range(1, 9):
        for causal in (False, True):
            for L in [None] + list(range(0, N + 1)):
                B, H, d = 1, 2, 3
                q = rng.normal(size=(B, H, N, d))
                k = rng.normal(size=(B, H, N, d))
                v = rng.normal(size=(B, H, N, 4))
                seqlens = None if L is None else np.array([L])
                scale = 0.37
                o, lse = fn(q, k, v, scale, causal, seqlens)
                ob, lseb = attention_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, seqlens)
                ob = np.array(ob)
                lseb = np.array(lseb)
                assert o.shape == ob.shape, (o.shape, ob.shape)
                np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12, err_msg=f"O N={N} causal={causal} L={L}")
                np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12, err_msg=f"LSE N={N} causal={causal} L={L}")


def pin_identity_values(fn):
    """V = identity makes O = P: entries >= 0, masked entries exactly 0, rows sum to 1."""
    rng = _rng(12)
    B, H, N, d = 2, 2, 6, 5
    for causal, kind in MASK_CASES:
        q = rng.normal(size=(B, H, N, d)) * 2.0
        k = rng.normal(size=(B, H, N, d)) * 2.0
        v = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
        seqlens = _seqlens_for(kind, B, N, rng)
        o, _ = fn(q, k, v, 0.9, causal, seqlens)
        lens = _lens(seqlens, B, N)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    row = o[b, h, i]
                    allowed = [_allowed(i, j, lens[b], causal) for j in range(N)]
                    assert np.all(row >= 0.0)
                    for j in range(N):
                        if not allowed[j]:
                            assert row[j] == 0.0, (b, h, i, j, causal, lens[b])
                    if any(allowed):
                        assert abs(row.sum() - 1.0) <= 1e-12, (row.sum(), causal, lens[b])
                    else:
                        assert np.all(row == 0.0)


def pin_equal_value_rows(fn):
    """If every value row equals u, every non-empty output row equals u."""
    rng = _rng(13)
    B, H, N, d = 2, 3, 9, 4
    for causal, kind in MASK_CASES:
        q = rng.normal(size=(B, H, N, d))
        k = rng.normal(size=(B, H, N, d))
        u = rng.normal(size=(B, H, 1, 5))
        v = np.broadcast_to(u, (B, H, N, 5)).copy()
        seqlens = _seqlens_for(kind, B, N, rng)
        o, _ = fn(q, k, v, 0.5, causal, seqlens)
        lens = _lens(seqlens, B, N)
        for b in range(B):
            for i in range(N):
                n_allowed = sum(_allowed(i, j, lens[b], causal) for j in range(N))
                if n_allowed:
                    np.testing.assert_allclose(o[b, :, i], u[b, :, 0], rtol=0, atol=1e-12)


def pin_zero_queries(fn):
    """Q = 0: O_i is the mean of the allowed value rows and LSE_i = ln |A_i|."""
    rng = _rng(14)
    B, H, N, d = 2, 2, 7, 3
    for causal, kind in MASK_CASES:
        q = np.zeros((B, H, N, d))
        k = rng.normal(size=(B, H, N, d))
        v = rng.normal(size=(B, H, N, 4))
        seqlens = _seqlens_for(kind, B, N, rng)
        o, lse = fn(q, k, v, 1.3, causal, seqlens)
        lens = _lens(seqlens, B, N)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    js = [j for j in range(N) if _allowed(i, j, lens[b], causal)]
                    if not js:
                        assert np.all(o[b, h, i] == 0.0) and lse[b, h, i] == -np.inf
                        continue
                    np.testing.assert_allclose(o[b, h, i], v[b, h, js].mean(axis=0), rtol=0, atol=1e-12)
                    assert abs(lse[b, h, i] - math.log(len(js))) <= 1e-12


def pin_dominant_score(fn):
    """A key whose score beats every other allowed key by 50 selects its value row.

    Query i points along axis i with length 10; the chosen key pi(i) carries 5 on
    axis i and every other key 0 there, so s_{i,pi(i)} = 50 and s_ij = 0 otherwise
    (scale 1).  Then O_i = v_{pi(i)} within N e^-50 max|v| and LSE_i = 50 within
    N e^-50.  pi is not the identity, so a transposed S or a reversed V fails.
    """
    rng = _rng(15)
    N = 8
    d = N
    B, H = 1, 1
    for causal, L in [(False, None), (True, None), (False, 5), (True, 6)]:
        Lv = N if L is None else L
        if causal:
            pi = [min(i // 2, Lv - 1) for i in range(N)]
        else:
            pi = [(N - 1 - i) % Lv for i in range(N)]
        q = np.zeros((B, H, N, d))
        k = np.zeros((B, H, N, d))
        for i in range(N):
            q[0, 0, i, i] = 10.0
            k[0, 0, pi[i], i] = 5.0
        v = rng.normal(size=(B, H, N, 3))
        seqlens = None if L is None else np.array([L])
        o, lse = fn(q, k, v, 1.0, causal, seqlens)
        tol = N * math.exp(-50.0) * 4.0 * float(np.abs(v).max())
        for i in range(N):
            if causal and pi[i] > i:
                continue
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, pi[i]], rtol=0, atol=max(tol, 1e-14))
            assert abs(lse[0, 0, i] - 50.0) <= 1e-12


def pin_closed_forms(fn):
    """N = 1: O = v0, LSE = s00.  Two keys: logistic weights.  Causal row 0: O0 = v0."""
    rng = _rng(16)
    q = rng.normal(size=(1, 1, 1, 4))
    k = rng.normal(size=(1, 1, 1, 4))
    v = rng.normal(size=(1, 1, 1, 3))
    o, lse = fn(q, k, v, 0.7, False, None)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.7 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14

    q = rng.normal(size=(1, 1, 2, 4))
    k = rng.normal(size=(1, 1, 2, 4))
    v = rng.normal(size=(1, 1, 2, 3))
    scale = 0.45
    o, lse = fn(q, k, v, scale, False, None)
    for i in range(2):
        s0 = scale * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = scale * float(q[0, 0, i] @ k[0, 0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(o[0, 0, i], w0 * v[0, 0, 0] + w1 * v[0, 0, 1], rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) <= 1e-13

    q = rng.normal(size=(2, 2, 5, 4))
    k = rng.normal(size=(2, 2, 5, 4))
    v = rng.normal(size=(2, 2, 5, 3))
    o, lse = fn(q, k, v, 0.3, True, None)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0]), rtol=0, atol=1e-14)


def pin_invariances(fn):
    """Properties of the definition that a wrong index or sign breaks."""
    rng = _rng(17)
    B, H, N, d = 2, 2, 10, 6
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, 5))
    scale = 0.41

    # joint permutation of key and value rows (non-causal, no padding)
    perm = rng.permutation(N)
    o1, l1 = fn(q, k, v, scale, False, None)
    o2, l2 = fn(q, k[:, :, perm], v[:, :, perm], scale, False, None)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)

    # a vector u added to every key row shifts row i of S by scale * q_i . u
    for causal in (False, True):
        u = rng.normal(size=(B, H, 1, d))
        o1, l1 = fn(q, k, v, scale, causal, None)
        o2, l2 = fn(q, k + u, v, scale, causal, None)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        shift = scale * np.einsum("bhnc,bhc->bhn", q, u[:, :, 0])
        np.testing.assert_allclose(l2, l1 + shift, rtol=0, atol=1e-12)

    # the scale can be folded into Q
    for causal in (False, True):
        o1, l1 = fn(q, k, v, scale, causal, None)
        o2, l2 = fn(q * scale, k, v, 1.0, causal, None)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)

    # padding to L keys is truncating K and V to their first L rows
    for causal in (False, True):
        for L in (1, 4, N):
            o1, l1 = fn(q, k, v, scale, causal, np.array([L, L]))
            if causal:
                # truncation keeps the same (i, j) pairs for rows i < L only
                o2, l2 = fn(q[:, :, :L], k[:, :, :L], v[:, :, :L], scale, True, None)
                np.testing.assert_allclose(o1[:, :, :L], o2, rtol=0, atol=1e-12)
                np.testing.assert_allclose(l1[:, :, :L], l2, rtol=0, atol=1e-12)
                # and rows i >= L see exactly the L valid keys
                o3, l3 = fn(q, k, v, scale, False, np.array([L, L]))
                np.testing.assert_allclose(o1[:, :, L:], o3[:, :, L:], rtol=0, atol=1e-12)
            else:
                for i in range(N):
                    o2, l2 = fn(q[:, :, i:i + 1], k[:, :, :L], v[:, :, :L], scale, False, None)
                    np.testing.assert_allclose(o1[:, :, i], o2[:, :, 0], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l1[:, :, i], l2[:, :, 0], rtol=0, atol=1e-12)

    # the causal last row sees every key
    o1, l1 = fn(q, k, v, scale, True, None)
    o2, l2 = fn(q, k, v, scale, False, None)
    np.testing.assert_allclose(o1[:, :, -1], o2[:, :, -1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1[:, :, -1], l2[:, :, -1], rtol=0, atol=1e-12)


def pin_library_sdpa(fn):
    """Agreement with torch.nn.functional.scaled_dot_product_attention (CPU, float64)."""
    rng = _rng(18)
    B, H, N, d = 2, 3, 33, 16
    for causal, kind in MASK_CASES:
        q = rng.normal(size=(B, H, N, d))
        k = rng.normal(size=(B, H, N, d))
        v = rng.normal(size=(B, H, N, d))
        seqlens = None if kind is None else rng.integers(1, N + 1, size=B)
        scale = 0.29
        o, lse = fn(q, k, v, scale, causal, seqlens)
        lens = _lens(seqlens, B, N)
        mask = np.zeros((B, 1, N, N), dtype=bool)
        for b in range(B):
            for i in range(N):
                for j in range(N):
                    mask[b, 0, i, j] = _allowed(i, j, lens[b], causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(mask), scale=scale).numpy()
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        s = scale * np.einsum("bhic,bhjc->bhij", q, k)
        s = np.where(mask, s, -np.inf)
        lse_ref = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    arr = lambda x: np.array(x, dtype=np.float64)  # noqa: E731  (strings such as "-inf" parse)
    return g, arr(g["q"]), arr(g["k"]), arr(g["v"])


def golden_names():
    return sorted(n for n in os.listdir(GOLDEN) if n.endswith(".json"))


def pin_golden(fn):
    """Hand-derived fixtures in tests/golden/ (each file states its derivation)."""
    for name in golden_names():
        g, q, k, v = _load_golden(name)
        for case in g["cases"]:
            seqlens = None if case["seqlens"] is None else np.array(case["seqlens"])
            o, lse = fn(q, k, v, g["scale"], case["causal"], seqlens)
            o_ref = np.array(case["o"], dtype=np.float64)
            lse_ref = np.array(case["lse"], dtype=np.float64)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13, err_msg=f"{name} {case}")
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13, err_msg=f"{name} {case}")


ALL_PINS = [
    pin_brute_force,
    pin_identity_values,
    pin_equal_value_rows,
    pin_zero_queries,
    pin_dominant_score,
    pin_closed_forms,
    pin_invariances,
    pin_library_sdpa,
    pin_golden,
]
