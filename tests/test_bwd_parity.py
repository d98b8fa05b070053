"""GPU parity of the backward pass (fa_bwd) against the float64 oracle.

Tolerance, derived from the arithmetic of the kernels.  With the exact softmax
P, dP = dO V^T, D_i = dO_i . O_i, dS = P (dP - D) of the oracle, the kernels
differ from the exact gradients only by:

* the LSE and O they are given (LSE_in, O_in): P is recomputed as
  exp(S - LSE_in), relative error e_L = exp(|LSE_in - LSE|) - 1, and D from
  O_in, absolute error sum_c |dO_ic| |O_in,ic - O_ic|;
* P rounded to bf16 as the operand of dV and dS rounded to bf16 as the operand
  of dQ and dK (relative 2^-8 each, the unit roundoff of bf16's 8-bit
  significand);
* float32 accumulation of the products (at most 2^-12 of the sum of absolute
  terms at these lengths) and the bf16 rounding of the outputs (2^-8).

So, elementwise,
    |dS err| <= 2^-8 |dS| + e_L P (|dP| + |D|) + P |D err|
    |dV err| <= (2^-8 + e_L + 2^-12) P^T |dO| + 2^-8 |dV|
    |dK err| <= scale (|dS err|^T |Q| + 2^-12 |dS|^T |Q|) + 2^-8 |dK|
    |dQ err| <= scale (|dS err| |K| + 2^-12 |dS| |K|) + 2^-8 |dQ|
and the tests require the measured error to stay within twice that bound (plus
1e-6 absolute), and the normwise relative error within 2^-6.  The inputs fed to
the backward pass are either the oracle's O (rounded to bf16) and LSE (rounded
to float32) or the GPU forward pass's own outputs (end to end).
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_57_amd import binding
from exact_io_aware_57_amd.inputs import random_qkv_grouped
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -8


def say(msg):
    print(msg, flush=True)


def np64(t):
    return t.detach().float().cpu().double().numpy()


def bounds(q, k, v, do, scale, causal, seqlens, o_in, lse_in, row_block=1024):
    """Elementwise error bounds (dQ, dK, dV) and exact (O, LSE), float64; the
    rows of a head are taken row_block at a time (dK, dV bounds are sums over
    rows)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    o_ex, lse_ex = oracle.attention(q, k, v, scale, causal, seqlens)
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = N if seqlens is None else min(max(int(seqlens[b]), 0), N)
        for h in range(H):
            g = oracle.kv_head(h, H, H_kv)
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                p, _, _ = oracle.softmax_matrix(q[b, h, rows], k[b, g], scale, rows, L, causal)
                dp = do[b, h, rows] @ v[b, g].T
                dsum = (p * dp).sum(axis=1)
                ds = p * (dp - dsum[:, None])
                fin = np.isfinite(lse_ex[b, h, rows])
                e_l = np.zeros(rows.size)
                e_l[fin] = np.expm1(np.abs(lse_in[b, h, rows][fin] - lse_ex[b, h, rows][fin]))
                d_err = (np.abs(do[b, h, rows]) * np.abs(o_in[b, h, rows] - o_ex[b, h, rows])).sum(axis=1)
                d_err += 2.0 ** -20 * (np.abs(do[b, h, rows]) * np.abs(o_ex[b, h, rows])).sum(axis=1)
                ds_err = U * np.abs(ds) + e_l[:, None] * p * (np.abs(dp) + np.abs(dsum)[:, None]) + p * d_err[:, None]
                bv[b, g] += ((U + 2.0 ** -12) * p + e_l[:, None] * p).T @ np.abs(do[b, h, rows])
                bk[b, g] += scale * ((ds_err + 2.0 ** -12 * np.abs(ds)).T @ np.abs(q[b, h, rows]))
                bq[b, h, rows] = scale * ((ds_err + 2.0 ** -12 * np.abs(ds)) @ np.abs(k[b, g]))
    return bq, bk, bv, o_ex, lse_ex


def run_backward(q, k, v, do, o_in, lse_in, scale, causal, seqlens):
    dev = [x.to(DEV) for x in (q, k, v, o_in, do)]
    lse_d = lse_in.to(DEV)
    sd = None if seqlens is None else seqlens.to(DEV)
    dq, dk, dv = binding.attention_backward(dev[0], dev[1], dev[2], dev[3], lse_d, dev[4], scale, causal, sd)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(q, k, v, do, scale, causal, seqlens, tag, end_to_end=False):
    """Backward on the GPU against the oracle, within the derived bounds."""
    qn, kn, vn, gn = (np64(x) for x in (q, k, v, do))
    sl = None if seqlens is None else seqlens.numpy()
    if end_to_end:
        o_g, l_g = binding.attention_forward(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal,
                                             None if seqlens is None else seqlens.to(DEV))
        torch.cuda.synchronize()
        o_in, lse_in = o_g.cpu(), l_g.cpu()
    else:
        o_ex, lse_ex = oracle.attention(qn, kn, vn, scale, causal, sl)
        o_in = torch.from_numpy(o_ex).to(torch.bfloat16)
        lse_in = torch.from_numpy(lse_ex).to(torch.float32)
    say(f"[bwd] {tag}: q {tuple(q.shape)} k {tuple(k.shape)} causal={causal} "
        f"seqlens={None if seqlens is None else seqlens.tolist()} end_to_end={end_to_end}")
    dq, dk, dv = run_backward(q, k, v, do, o_in, lse_in, scale, causal, seqlens)
    rq, rk, rv = oracle.attention_backward(qn, kn, vn, gn, scale, causal, sl)
    bq, bk, bv, _, _ = bounds(qn, kn, vn, gn, scale, causal, sl, np64(o_in), lse_in.double().numpy())
    for name, got, ref, bnd in (("dQ", dq, rq, bq), ("dK", dk, rk, bk), ("dV", dv, rv, bv)):
        g = np64(got)
        assert np.isfinite(g).all(), f"{name}: non-finite"
        err = np.abs(g - ref)
        lim = 2.0 * (bnd + U * np.abs(ref)) + 1e-6
        worst = (err / lim).max()
        rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
        say(f"[bwd] {tag}: {name} max err {err.max():.3e} (worst err/bound {worst:.3f}) normwise rel {rel:.3e}")
        assert worst <= 1.0, f"{name}: error exceeds the derived bound"
        assert rel <= 2.0 ** -6 or np.linalg.norm(ref) < 1e-6, f"{name}: normwise error {rel}"
    return dq, dk, dv


def inputs(B, H, H_kv, N, d, seed, len_range=None, std=1.0):
    q, k, v, sl = random_qkv_grouped(B, H, H_kv, N, d, torch.bfloat16, std, seed, len_range)
    gen = torch.Generator(device="cpu").manual_seed(seed + 7919)
    do = torch.randn((B, H, N, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do, sl


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2), (6, 1)])
def test_backward_parity(H, H_kv, d, causal):
    for n, lens in [(200, None), (333, (1, 333))]:
        q, k, v, do, sl = inputs(2, H, H_kv, n, d, 50 + H_kv + n + d, lens)
        check(q, k, v, do, 1.0 / math.sqrt(d), causal, sl, f"H={H}/{H_kv} n={n} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_ragged_lengths(d, causal):
    for n in [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 255, 257, 500]:
        q, k, v, do, _ = inputs(1, 2, 2, n, d, 3000 + n)
        check(q, k, v, do, 1.0 / math.sqrt(d), causal, None, f"ragged n={n} d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_padding_lengths(causal):
    n = 300
    q, k, v, do, _ = inputs(6, 2, 1, n, 128, 17)
    sl = torch.tensor([0, 1, 63, 64, 65, n], dtype=torch.int32)
    dq, dk, dv = check(q, k, v, do, 0.0884, causal, sl, "padding")
    # a batch with no valid key gets no gradient at all; keys past the length get none
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    assert torch.all(dk[2, :, 63:] == 0) and torch.all(dv[4, :, 65:] == 0)


@pytest.mark.parametrize("d,causal", [(64, False), (128, True), (128, False)])
def test_backward_end_to_end(d, causal):
    """Forward on the GPU, its O and LSE into the backward pass, against the
    oracle's exact gradients (the bound includes the forward pass's errors)."""
    q, k, v, do, sl = inputs(2, 8, 2, 700, d, 77 + d, (300, 700), std=0.5)
    check(q, k, v, do, 1.0 / math.sqrt(d), causal, sl, f"end to end d={d}", end_to_end=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_grid(d, causal):
    """At least 256 workgroups of 256 queries (B = 4, H = 16, five query tiles
    of 256 per head), so dQ runs in the 8-wave ping-pong form: grouped heads,
    per-batch lengths from 1 to N and a ragged last tile of 76 queries."""
    q, k, v, do, sl = inputs(4, 16, 4, 1100, d, 400 + d + int(causal), (1, 1100))
    check(q, k, v, do, 1.0 / math.sqrt(d), causal, sl, f"large grid d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_grid_padding(causal):
    """The ping-pong dQ path with an empty batch, a one-key batch and a full
    one: the empty batch gets no gradient, keys past a length get none."""
    q, k, v, do, _ = inputs(4, 16, 8, 1100, 128, 650 + int(causal))
    sl = torch.tensor([0, 1, 700, 1100], dtype=torch.int32)
    dq, dk, dv = check(q, k, v, do, 0.0884, causal, sl, "large grid padding")
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    assert torch.all(dk[1, :, 1:] == 0) and torch.all(dv[2, :, 700:] == 0)


def test_backward_long_sequence():
    """A few thousand keys: many query tiles per key tile, every key tile of a
    head in flight."""
    q, k, v, do, _ = inputs(1, 2, 1, 4096, 128, 99, std=0.5)
    check(q, k, v, do, 0.0884, True, None, "n=4096 causal")


def test_backward_deterministic_and_streams():
    q, k, v, do, sl = inputs(2, 8, 4, 777, 128, 5, (100, 777))
    o_ex, lse_ex = oracle.attention(np64(q), np64(k), np64(v), 0.0884, True, sl.numpy())
    o_in, lse_in = torch.from_numpy(o_ex).to(torch.bfloat16), torch.from_numpy(lse_ex).to(torch.float32)
    a = run_backward(q, k, v, do, o_in, lse_in, 0.0884, True, sl)
    b = run_backward(q, k, v, do, o_in, lse_in, 0.0884, True, sl)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    s = torch.cuda.Stream(device=DEV)
    dev = [x.to(DEV) for x in (q, k, v, o_in, do)]
    lse_d, sd = lse_in.to(DEV), sl.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = binding.attention_backward(dev[0], dev[1], dev[2], dev[3], lse_d, dev[4], 0.0884, True, sd,
                                       stream=s.cuda_stream)
    s.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_backward_guard_bands_untouched():
    B, H, H_kv, N, d = 2, 4, 2, 130, 64
    q, k, v, do, _ = inputs(B, H, H_kv, N, d, 21)
    o_ex, lse_ex = oracle.attention(np64(q), np64(k), np64(v), 0.125, False)
    dev = [x.to(DEV) for x in (q, k, v, torch.from_numpy(o_ex).to(torch.bfloat16), do)]
    lse_d = torch.from_numpy(lse_ex).to(torch.float32).to(DEV)
    nq, nk = B * H * N * d, B * H_kv * N * d
    bufs = [torch.full((n + 512,), 7.0, dtype=torch.bfloat16, device=DEV) for n in (nq, nk, nk)]
    dq = bufs[0][:nq].view(B, H, N, d)
    dk = bufs[1][:nk].view(B, H_kv, N, d)
    dv = bufs[2][:nk].view(B, H_kv, N, d)
    binding.attention_backward(dev[0], dev[1], dev[2], dev[3], lse_d, dev[4], 0.125, False, None, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf, n in zip(bufs, (nq, nk, nk)):
        assert torch.all(buf[n:] == 7.0)


def test_backward_long_context_full_size():
    """The configuration bench.py times (B = 1, H = 32, N = 16384, d = 128,
    causal, O and LSE from the GPU forward pass): head 0 checked in full
    against the oracle within the derived bound, heads 13 and 31 on sampled dQ
    rows (a dQ row needs only its own row of the attention matrix)."""
    q, k, v, do, _ = inputs(1, 32, 32, 16384, 128, 9, std=0.5)
    scale = float(np.float32(1.0 / math.sqrt(128.0)))
    dev = [x.to(DEV) for x in (q, k, v, do)]
    o, lse = binding.attention_forward(dev[0], dev[1], dev[2], scale, True, None)
    dq, dk, dv = binding.attention_backward(dev[0], dev[1], dev[2], o, lse, dev[3], scale, True, None)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    say("[bwd] long context: head 0 in full")
    sl = slice(0, 1)
    qn, kn, vn, gn = (np64(x[:, sl]) for x in (q, k, v, do))
    rq, rk, rv = oracle.attention_backward(qn, kn, vn, gn, scale, True, None)
    bq, bk, bv, _, _ = bounds(qn, kn, vn, gn, scale, True, None, np64(o[:, sl]), np64(lse[:, sl]))
    for name, got, ref, bnd in (("dQ", dq[:, sl], rq, bq), ("dK", dk[:, sl], rk, bk), ("dV", dv[:, sl], rv, bv)):
        err = np.abs(np64(got) - ref)
        worst = (err / (2.0 * (bnd + U * np.abs(ref)) + 1e-6)).max()
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        say(f"[bwd] long context head 0: {name} worst err/bound {worst:.3f} normwise rel {rel:.3e}")
        assert worst <= 1.0 and rel <= 2.0 ** -6
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 8191, 16383], rng.integers(0, 16384, size=24)]))
    for h in (13, 31):
        qh, kh, vh, gh = (np64(x[0, h]) for x in (q, k, v, do))
        p, _, _ = oracle.softmax_matrix(qh[rows], kh, scale, rows, 16384, True)
        dp = gh[rows] @ vh.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        ref = scale * (ds @ kh)
        err = np.abs(np64(dq[0, h, rows]) - ref)
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        say(f"[bwd] long context head {h} sampled dQ rows: max err {err.max():.3e} normwise rel {rel:.3e}")
        assert rel <= 2.0 ** -6


def test_backward_random_shapes():
    """Twelve shapes drawn from a fixed seed: head sizes 64 and 128, grouped
    heads, causal or not, key-padding lengths including zero, and grids on both
    sides of the ping-pong dQ threshold (ceil(N / 256) * B * H >= 256)."""
    import random
    rng = random.Random(7)
    for c in range(12):
        d = rng.choice([64, 128])
        H_kv, G = rng.choice([1, 2, 4]), rng.choice([1, 2, 4])
        if c % 3 == 0:
            B, H, N = rng.choice([2, 4]), 16, rng.randint(600, 1300)
            H_kv = 16 // G
        else:
            B, H, N = rng.choice([1, 2, 3]), H_kv * G, rng.randint(1, 700)
        causal = rng.random() < 0.5
        use_len = rng.random() < 0.5
        seed = rng.randint(0, 10 ** 6)
        q, k, v, do, sl = inputs(B, H, H_kv, N, d, seed, (0, N) if use_len else None)
        if use_len:
            sl[rng.randrange(B)] = 0
        check(q, k, v, do, 1.0 / math.sqrt(d), causal, sl, f"random {c}: B{B} H{H}/{H_kv} N{N} d{d} causal={causal}")
