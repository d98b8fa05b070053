"""The CPU oracle against its pins (CPU only).

The pins live in tests/oracle_pins.py.  Besides running them on the oracle, this
file checks that the pins are strong enough: each test in
``test_pins_catch_planted_mistake`` plants one plausible mistake in a copy of
the oracle, on the CPU, and requires at least one pin to fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_rows, softmax_matrix
from exact_io_aware_57_amd.inputs import WORKLOADS, make_inputs, random_qkv
from tests import oracle_pins


def oracle_fn(q, k, v, scale, causal, seqlens):
    return attention(q, k, v, scale, causal, seqlens)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_fn)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.normal(size=(40, 16))
    k = rng.normal(size=(64, 16))
    rows = np.arange(40) + 10
    for causal in (False, True):
        for L in (64, 30, 1):
            p, m, l = softmax_matrix(q, k, 0.25, rows, L, causal)
            assert np.all(p >= 0)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
            s = 0.25 * q @ k.T
            for r, i in enumerate(rows):
                allowed = [j for j in range(64) if j < L and (not causal or j <= i)]
                assert m[r] == s[r, allowed].max()


# ---------------------------------------------------------------------------
# The pages' exactness claim: processing the keys block by block with a running
# max and a running sum of exponentials gives the exact softmax result
# (FlashAttention (UR), section "Online computation of softmax"; FlashAttention-2
# (HI), "Performance and efficiency": exact and deterministic).  This block-wise
# routine is test-only; it pins the claim, not any GPU code.
# ---------------------------------------------------------------------------
def online_blockwise(q, k, v, scale, causal, seqlens, block):
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        L = N if seqlens is None else min(max(int(seqlens[b]), 0), N)
        for h in range(H):
            m = np.full(N, -np.inf)        # running max of the scores seen so far
            l = np.zeros(N)                # running sum of exp(score - m)
            acc = np.zeros((N, v.shape[-1]))  # running sum of exp(score - m) * v
            for j0 in range(0, N, block):
                js = np.arange(j0, min(N, j0 + block))
                s = scale * (q[b, h] @ k[b, h, js].T)
                allowed = (js[None, :] < L) & ((~np.full((N, 1), causal)) | (js[None, :] <= np.arange(N)[:, None]))
                s = np.where(allowed, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                p = np.exp(s - ref[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, js]
                m = m_new
            nonempty = l > 0
            o[b, h, nonempty] = acc[nonempty] / l[nonempty, None]
            lse[b, h, nonempty] = m[nonempty] + np.log(l[nonempty])
    return o, lse


@pytest.mark.parametrize("block", [1, 3, 64, 128])
@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True), (True, True)])
def test_online_softmax_is_exact(block, causal, padded):
    rng = np.random.default_rng(block)
    B, H, N, d = 2, 2, 150, 16
    q = rng.normal(size=(B, H, N, d)) * 2
    k = rng.normal(size=(B, H, N, d)) * 2
    v = rng.normal(size=(B, H, N, d))
    seqlens = np.array([0, 77]) if padded else None
    o1, l1 = attention(q, k, v, 0.3, causal, seqlens)
    o2, l2 = online_blockwise(q, k, v, 0.3, causal, seqlens, block)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_rows_match_full():
    q, k, v, seqlens = random_qkv(2, 2, 300, 64, torch.float32, 1.0, seed=5, len_range=(100, 300))
    q, k, v = (x.double().numpy() for x in (q, k, v))
    for causal in (False, True):
        o, lse = attention(q, k, v, 0.125, causal, seqlens.numpy(), row_block=64)
        rows = np.array([0, 1, 63, 64, 150, 299])
        o_r, lse_r = attention_rows(q, k, v, 0.125, causal, seqlens.numpy(), 1, 1, rows)
        np.testing.assert_array_equal(o_r, o[1, 1, rows])
        np.testing.assert_array_equal(lse_r, lse[1, 1, rows])


def test_bf16_inputs_are_read_exactly():
    q, k, v, _ = random_qkv(1, 1, 16, 64, torch.bfloat16, 1.0, seed=3)
    for t in (q, k, v):
        x = t.float().double().numpy()
        # float64 holds every bf16 value exactly: converting back gives the same bits
        assert torch.equal(torch.from_numpy(x).to(torch.bfloat16), t)
        # and each has at most 8 significant bits: mantissa * 2^8 is an integer
        m, _ = np.frexp(x)
        assert np.all(m * 2.0 ** 8 == np.round(m * 2.0 ** 8))
    qf, kf, vf = (t.float().double().numpy() for t in (q, k, v))
    o, lse = attention(qf, kf, vf, 0.125)
    assert o.dtype == np.float64 and np.isfinite(o).all() and np.isfinite(lse).all()


def test_workload_table_matches_the_stated_shapes():
    w = WORKLOADS
    assert (w[1].B, w[1].H, w[1].N, w[1].d, w[1].dtype, w[1].causal) == (1, 1, 128, 64, "fp32", False)
    assert (w[2].B, w[2].H, w[2].N, w[2].d, w[2].len_range, w[2].causal) == (16, 16, 512, 64, (256, 512), False)
    assert (w[3].B, w[3].H, w[3].N, w[3].d, w[3].causal) == (8, 12, 1024, 64, True)
    assert (w[4].B, w[4].H, w[4].N, w[4].d, w[4].causal) == (2, 8, 4096, 64, False)
    assert (w[5].B, w[5].H, w[5].N, w[5].d, w[5].causal, w[5].std) == (1, 32, 16384, 128, True, 0.5)
    assert w[5].scale == float(np.float32(1.0 / math.sqrt(128.0)))
    assert w[2].scale == 0.125


def test_inputs_are_seeded_and_rounded():
    a = make_inputs(2)
    b = make_inputs(2)
    for name in ("q", "k", "v", "seqlens"):
        assert torch.equal(a[name], b[name])
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (16, 16, 512, 64)
    s = a["seqlens"]
    assert s.dtype == torch.int32 and int(s.min()) >= 256 and int(s.max()) <= 512
    c = make_inputs(2, seed=99)
    assert not torch.equal(a["q"], c["q"])
    t = make_inputs(1)
    assert t["q"].dtype == torch.float32 and t["seqlens"] is None


# ---------------------------------------------------------------------------
# Planted mistakes: each copy of the oracle below carries one bug.  Every one of
# them must fail at least one pin.
# ---------------------------------------------------------------------------
def _naive(q, k, v, scale, causal, seqlens, bug=None):
    B, H, N, d = q.shape
    Nk = k.shape[2]
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), -np.inf)
    if bug == "no_scale":
        scale = 1.0
    if bug == "sqrt_d":
        scale = 1.0 / math.sqrt(d)
    for b in range(B):
        L = Nk if seqlens is None else min(max(int(seqlens[b]), 0), Nk)
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            if bug == "transpose_s" and N == Nk:
                s = s.T
            i = np.arange(N)[:, None]
            j = np.arange(Nk)[None, :]
            allowed = np.broadcast_to(j < L, (N, Nk)).copy()
            if bug == "pad_off_by_one":
                allowed = np.broadcast_to(j <= L, (N, Nk)).copy()
            if bug == "pad_masks_queries":
                allowed = np.broadcast_to(i < L, (N, Nk)).copy()
            if causal:
                if bug == "causal_strict":
                    allowed &= j < i
                elif bug == "causal_reversed":
                    allowed &= j >= i
                else:
                    allowed &= j <= i
            if bug == "drop_last_key":
                allowed[:, -1] = False
            vv = v[b, h][::-1] if bug == "v_reversed" else v[b, h]
            for r in range(N):
                js = np.nonzero(allowed[r])[0]
                if js.size == 0:
                    if bug == "empty_row_nan":
                        o[b, h, r] = np.nan
                    continue
                if bug == "softmax_over_queries":
                    col = s[:, js]
                    w = np.exp(col[r] - col.max(axis=0))
                    w = w / np.exp(col - col.max(axis=0)).sum(axis=0)
                    o[b, h, r] = w @ vv[js]
                    lse[b, h, r] = math.log(w.sum())
                    continue
                m = s[r, js].max()
                w = np.exp(s[r, js] - m)
                l = w.sum()
                o[b, h, r] = (w @ vv[js]) if bug == "unnormalised" else (w @ vv[js]) / l
                if bug == "lse_no_max":
                    lse[b, h, r] = math.log(l)
                elif bug == "lse_log2":
                    lse[b, h, r] = (m + math.log(l)) / math.log(2.0)
                else:
                    lse[b, h, r] = m + math.log(l)
    return o, lse


BUGS = ["no_scale", "sqrt_d", "transpose_s", "softmax_over_queries", "causal_strict", "causal_reversed",
        "pad_off_by_one", "pad_masks_queries", "drop_last_key", "v_reversed", "unnormalised",
        "lse_no_max", "lse_log2", "empty_row_nan"]


def test_unplanted_copy_passes_every_pin():
    for pin in oracle_pins.ALL_PINS:
        pin(lambda q, k, v, s, c, L: _naive(q, k, v, s, c, L))


@pytest.mark.parametrize("bug", BUGS)
def test_pins_catch_planted_mistake(bug):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lambda q, k, v, s, c, L: _naive(q, k, v, s, c, L, bug=bug))
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {bug!r}"


def test_oracle_exports():
    assert oracle.attention is attention and callable(oracle.attention_brute)


# ---------------------------------------------------------------------------------
# Grouped / multi-query attention (FlashAttention (UR), section "FlashAttention-2
# (2023)": multi-query attention among the supported architectures).
# ---------------------------------------------------------------------------------
def _brute_grouped(q, k, v, scale, causal, seqlens):
    """Expected output written out head by head: query head h of a group of
    H / H_kv consecutive heads reads key/value head h // (H / H_kv); each head is
    then plain attention, computed by the scalar brute force."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    group = H // Hkv
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros(q.shape[:3])
    for h in range(H):
        g = h // group
        ob, lb = oracle.attention_brute(q[:, h:h + 1].tolist(), k[:, g:g + 1].tolist(), v[:, g:g + 1].tolist(), scale, causal,
                                        seqlens)
        o[:, h] = np.array(ob)[:, 0]
        lse[:, h] = np.array(lb)[:, 0]
    return o, lse


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 2), (4, 1), (3, 1)])
@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True), (True, True)])
def test_grouped_heads_match_brute_force(H, Hkv, causal, padded):
    rng = np.random.default_rng(100 + 10 * H + Hkv)
    B, N, d = 2, 7, 5
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, Hkv, N, d))
    v = rng.normal(size=(B, Hkv, N, 3))
    seqlens = rng.integers(0, N + 1, size=B) if padded else None
    o, lse = attention(q, k, v, 0.7, causal, seqlens)
    o_ref, lse_ref = _brute_grouped(q, k, v, 0.7, causal, seqlens)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_multi_query_heads_share_keys_and_values():
    # H_kv = 1: two query heads with equal queries give equal outputs; different
    # queries over the same keys/values give outputs in the convex hull of V.
    rng = np.random.default_rng(7)
    q = rng.normal(size=(1, 3, 6, 4))
    q[0, 2] = q[0, 0]
    k = rng.normal(size=(1, 1, 6, 4))
    v = rng.normal(size=(1, 1, 6, 2))
    o, _ = attention(q, k, v, 0.5, False)
    np.testing.assert_array_equal(o[0, 0], o[0, 2])
    assert np.all(o[0] <= v[0, 0].max(axis=0) + 1e-12) and np.all(o[0] >= v[0, 0].min(axis=0) - 1e-12)


def test_grouped_pin_catches_a_wrong_head_map(monkeypatch):
    # Planted on the CPU: interleaved instead of consecutive groups.
    import importlib
    oa = importlib.import_module("oracle.attention")   # the module (the package re-exports a function of that name)
    monkeypatch.setattr(oa, "kv_head", lambda h, n, nkv: h % nkv)
    with pytest.raises(AssertionError):
        test_grouped_heads_match_brute_force(4, 2, False, False)


def test_head_counts_must_divide():
    q = np.zeros((1, 4, 3, 2))
    k = np.zeros((1, 3, 3, 2))
    with pytest.raises(ValueError):
        attention(q, k, k, 1.0)


# ---------------------------------------------------------------------------------
# Decoding against a key/value cache, and the merge of partial results.
# ---------------------------------------------------------------------------------
def _brute_decode(q, k, v, scale, causal, seqlens):
    """Row by row with math.exp / math.fsum and no max shift: query i of batch b
    sees key j iff j < L_b and (not causal or j <= L_b - Nq + i)."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = Nk if seqlens is None else min(max(int(seqlens[b]), 0), Nk)
        for h in range(H):
            g = h // (H // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk) if j < L and (not causal or j <= L - Nq + i)]
                if not keys:
                    continue
                w = [math.exp(scale * math.fsum(q[b, h, i, c] * k[b, g, j, c] for c in range(d))) for j in keys]
                tot = math.fsum(w)
                o[b, h, i] = [math.fsum(wj * v[b, g, j, c] for wj, j in zip(w, keys)) / tot for c in range(v.shape[3])]
                lse[b, h, i] = math.log(tot)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,H,Hkv", [(1, 9, 2, 2), (3, 9, 4, 2), (4, 4, 2, 1), (5, 11, 3, 1)])
def test_decode_matches_brute_force(Nq, Nk, H, Hkv, causal):
    rng = np.random.default_rng(Nq * 100 + Nk)
    B, d = 3, 4
    q = rng.normal(size=(B, H, Nq, d))
    k = rng.normal(size=(B, Hkv, Nk, d))
    v = rng.normal(size=(B, Hkv, Nk, 2))
    for seqlens in (None, np.array([0, 2, Nk])):
        o, lse = oracle.attention_decode(q, k, v, 0.6, causal, seqlens)
        o_ref, lse_ref = _brute_decode(q, k, v, 0.6, causal, seqlens)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_decode_agrees_with_full_attention():
    # Nq = Nk = L: the decode causal mask is the ordinary causal mask; Nq = 1 on the
    # whole cache is the last row of causal (and of non-causal) attention.
    rng = np.random.default_rng(3)
    q = rng.normal(size=(2, 2, 6, 3))
    k = rng.normal(size=(2, 2, 6, 3))
    v = rng.normal(size=(2, 2, 6, 3))
    o, lse = oracle.attention_decode(q, k, v, 0.8, True)
    o2, lse2 = attention(q, k, v, 0.8, True)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)
    o1, l1 = oracle.attention_decode(q[:, :, -1:], k, v, 0.8, True)
    np.testing.assert_allclose(o1[:, :, 0], o2[:, :, -1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1[:, :, 0], lse2[:, :, -1], rtol=0, atol=1e-13)


def test_decode_causal_mask_is_bottom_aligned():
    m = oracle.decode_allowed(2, 6, 5, True)
    assert m.tolist() == [[True, True, True, True, False, False], [True, True, True, True, True, False]]
    assert not oracle.decode_allowed(3, 6, 1, True)[0].any()   # query before the first key: empty row


@pytest.mark.parametrize("splits", [[0, 4, 9], [0, 1, 2, 9], [0, 9], [0, 3, 3, 9]])
def test_merge_of_key_chunks_is_the_whole(splits):
    # attention over key chunks [a, b), merged, equals attention over all keys
    rng = np.random.default_rng(len(splits))
    q = rng.normal(size=(1, 2, 3, 4))
    k = rng.normal(size=(1, 2, 9, 4))
    v = rng.normal(size=(1, 2, 9, 5))
    parts_o, parts_l = [], []
    for a, b in zip(splits[:-1], splits[1:]):
        o, l = oracle.attention_decode(q, k[:, :, a:b], v[:, :, a:b], 0.5, False)
        parts_o.append(o)
        parts_l.append(l)
    om, lm = oracle.merge_partials(np.stack(parts_o, axis=-2), np.stack(parts_l, axis=-1))
    o_ref, l_ref = _brute_decode(q, k, v, 0.5, False, None)
    np.testing.assert_allclose(om, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, l_ref, rtol=0, atol=1e-12)


def test_merge_of_empty_parts():
    o, l = oracle.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)
