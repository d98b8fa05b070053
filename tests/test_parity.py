"""GPU parity: the HIP path (through the C-ABI) against the float64 CPU oracle.

Tolerances.  bf16 outputs: max-abs <= 1e-2 and mean-abs <= 1e-3 on O.  fp32
path: max-abs <= 1e-5 on O and LSE.  LSE of the bf16 path: max-abs <= 1e-3,
derived from the arithmetic.  Every kernel takes LSE = ln2 * (m + log2 l) from
a float32 sum l of the exponentials before they are rounded to bf16, so the
error is the float32 error of the scores, at most d 2^-24 scale
sum_c |q_c| |k_c| (up to 6e-4 on the rising-score inputs, whose scores reach
about 110, and below 1e-4 elsewhere), plus the relative error of v_exp_f32
(about 2^-22 per term) and the float32 rounding of the sum (a few hundred
roundings of 2^-24 at most, below 2e-5), plus the rounding of log2f: below
1e-3 in all.  (The normaliser of O is a separate sum, over the rounded P that
the second product uses, in the kernels that keep one.)

The five stated workloads are held to those bounds against the exact oracle.
For the other shapes (a handful of keys per row) rounding the exact answer to
bf16 alone already costs up to ~9e-4 mean-abs, so there the mean-abs bound is
taken against the oracle rounded to bf16 (the distance to the correctly rounded
answer); the max-abs bound stays against the exact oracle.
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_57_amd import binding
from exact_io_aware_57_amd.inputs import make_inputs, random_qkv, random_qkv_grouped, workload
import oracle
from tests.fullhead import map_heads, oracle_head

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_LSE = 1e-2, 1e-3, 1e-3
F32_MAX, F32_LSE = 1e-5, 1e-5

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def gpu_forward(q, k, v, scale, causal, seqlens, want_lse=True):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    sd = None if seqlens is None else seqlens.to(DEV)
    o, lse = binding.attention_forward(qd, kd, vd, scale, causal, sd, want_lse=want_lse)
    torch.cuda.synchronize()
    return o, lse


def np64(t):
    return t.detach().float().cpu().double().numpy()


def check_against_oracle(q, k, v, scale, causal, seqlens, fp32, tag, stated_workload=False):
    say(f"[parity] {tag}: B,H,N,d={tuple(q.shape)} causal={causal} padded={seqlens is not None}")
    o, lse = gpu_forward(q, k, v, scale, causal, seqlens)
    o_ref, lse_ref = oracle.attention(np64(q), np64(k), np64(v), scale, causal,
                                      None if seqlens is None else seqlens.numpy())
    og, lg = np64(o), np64(lse)
    assert np.isfinite(og).all(), "non-finite output"
    err = np.abs(og - o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin), "LSE -inf pattern differs"
    assert np.all(lg[~fin] == -np.inf)
    lerr = np.abs(lg[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    rounded = torch.from_numpy(o_ref).to(torch.bfloat16).double().numpy()
    err_r = np.abs(og - rounded)
    say(f"[parity] {tag}: O max {err.max():.3e} mean {err.mean():.3e} (vs bf16-rounded oracle: mean {err_r.mean():.3e})"
        f"  LSE max {lerr:.3e}")
    if fp32:
        assert err.max() <= F32_MAX
        assert lerr <= F32_LSE
    else:
        assert err.max() <= BF16_MAX
        assert (err.mean() if stated_workload else err_r.mean()) <= BF16_MEAN
        assert lerr <= BF16_LSE
    return og, lg, o_ref, lse_ref


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_workload_parity_full(index):
    inp = make_inputs(index)
    check_against_oracle(inp["q"], inp["k"], inp["v"], inp["scale"], inp["causal"], inp["seqlens"],
                         fp32=workload(index).dtype == "fp32", tag=f"workload {index}", stated_workload=True)


def full_size_stats(og, lg, q, k, v, scale, causal, seqlens=None):
    """Every row of every head of a full-size output against the oracle.

    og [B, H, N, d] and lg [B, H, N] are the GPU results as float64 arrays.  The
    heads are spread over host threads.  Returns (O max err, O mean err, LSE max
    err, worst head as (b, h))."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))

    def one(bh):
        b, h = bh
        g = oracle.kv_head(h, H, Hkv)
        L = None if seqlens is None else int(seqlens[b])
        o_ref, lse_ref = oracle_head(qn[b, h], kn[b, g], vn[b, g], scale, causal, L)
        e = np.abs(og[b, h] - o_ref)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg[b, h]), fin), f"LSE -inf pattern differs in head {(b, h)}"
        el = np.abs(lg[b, h][fin] - lse_ref[fin]).max() if fin.any() else 0.0
        return e.max(), e.sum(), el

    heads = [(b, h) for b in range(B) for h in range(H)]
    res = map_heads(one, heads)
    worst = max(range(len(res)), key=lambda i: res[i][0])
    return (max(r[0] for r in res), sum(r[1] for r in res) / og.size, max(r[2] for r in res), heads[worst])


def test_long_context_full_size():
    """Long-context causal d=128 at full size (B=1, H=32, N=16384, std 0.5),
    the configuration bench.py times: every row of all 32 heads, O and LSE,
    against the oracle at the stated bounds, plus exact properties of row 0 and
    of every row."""
    inp = make_inputs(5)
    q, k, v = inp["q"], inp["k"], inp["v"]
    say(f"[parity] long context full size {tuple(q.shape)}")
    o, lse = gpu_forward(q, k, v, inp["scale"], True, None)
    og, lg = o.float().cpu(), lse.cpu()
    assert torch.isfinite(og).all() and torch.isfinite(lg).all()
    emax, emean, lmax, wh = full_size_stats(og.double().numpy(), lg.double().numpy(), q, k, v, inp["scale"], True)
    say(f"[parity] long context all {q.shape[1]} heads x {q.shape[2]} rows: O max {emax:.3e} (head {wh}) "
        f"mean {emean:.3e} LSE max {lmax:.3e}")
    assert emax <= BF16_MAX and emean <= BF16_MEAN and lmax <= BF16_LSE
    # causal row 0 attends to key 0 only: O_0 = v_0 exactly, LSE_0 = scale * q0.k0
    assert torch.equal(o[0, :, 0].cpu(), v[0, :, 0])
    s00 = inp["scale"] * (q[0, :, 0].double() * k[0, :, 0].double()).sum(-1)
    assert torch.allclose(lg[0, :, 0].double(), s00, atol=1e-5, rtol=0)
    # every row is a convex combination of value rows: within the column range of V
    vmax = v.float().abs().amax(dim=(2, 3)).cpu()
    assert (og.abs().amax(dim=(2, 3)) <= vmax * (1 + 2 ** -7)).all()


def check_listed_heads(q, k, v, scale, causal, seqlens, heads, tag):
    """Full-size call; every row of the listed (b, h) heads against the oracle
    at the stated bounds (heads computed in parallel on the host)."""
    say(f"[parity] {tag}: q {tuple(q.shape)} k {tuple(k.shape)} causal={causal} padded={seqlens is not None}")
    o, lse = gpu_forward(q, k, v, scale, causal, seqlens)
    og, lg = np64(o), np64(lse)
    assert np.isfinite(og).all()
    H, Hkv = q.shape[1], k.shape[1]
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))

    def one(bh):
        b, h = bh
        g = oracle.kv_head(h, H, Hkv)
        o_ref, lse_ref = oracle_head(qn[b, h], kn[b, g], vn[b, g], scale, causal,
                                     None if seqlens is None else int(seqlens[b]))
        e = np.abs(og[b, h] - o_ref)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg[b, h]), fin)
        el = np.abs(lg[b, h][fin] - lse_ref[fin]).max() if fin.any() else 0.0
        return e.max(), e.sum(), e.size, el

    res = map_heads(one, list(heads))
    worst, worst_l = max(r[0] for r in res), max(r[3] for r in res)
    mean = sum(r[1] for r in res) / sum(r[2] for r in res)
    say(f"[parity] {tag}: O max {worst:.3e} mean {mean:.3e} LSE max {worst_l:.3e}")
    assert worst <= BF16_MAX and mean <= BF16_MEAN and worst_l <= BF16_LSE


# Grids large enough for the 8-wave kernel at head size 64 (at least 256
# workgroups of 256 rows; causal: 4096 keys or more); head size 128 takes it
# from 1024 keys up on grids of more than 128 such workgroups.  The small
# shapes elsewhere in this file run the 4-wave kernel.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_kernel(d, causal):
    B, H, N = 2, 16, (8192 if causal else 2048)
    q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=31 + d + causal)
    check_listed_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (1, 9), (1, 15)], f"large grid d={d}")


def check_full_heads(q, k, v, scale, causal, seqlens, heads, tag):
    """Full-size call; every row of the listed (b, h) heads against the oracle.

    Element bound 1e-2 + 2^-7 |O|: the absolute 1e-2 of the other tests covers
    rows that average many values (|O| well below 1), while rows dominated by
    one key have |O| up to max |V| (about 4 here), where rounding O to bf16
    alone costs up to 2^-8 |O| and the bf16-rounded weights (each within 2^-8
    of its value), normalised by the sum of the unrounded ones, another
    2^-8 |O|."""
    say(f"[parity] {tag}: q {tuple(q.shape)} k {tuple(k.shape)} causal={causal} "
        f"seqlens={None if seqlens is None else seqlens.tolist()}")
    o, lse = gpu_forward(q, k, v, scale, causal, seqlens)
    assert torch.isfinite(o).all()
    H, Hkv, N = q.shape[1], k.shape[1], q.shape[2]
    worst, worst_l, total, count = 0.0, 0.0, 0.0, 0
    for b, h in heads:
        g = oracle.kv_head(h, H, Hkv)
        sl = None if seqlens is None else seqlens[b:b + 1].numpy()
        o_ref, lse_ref = oracle.attention_rows(np64(q[b:b + 1, h:h + 1]), np64(k[b:b + 1, g:g + 1]),
                                               np64(v[b:b + 1, g:g + 1]), scale, causal, sl, 0, 0, np.arange(N))
        og, lg = np64(o[b, h]), np64(lse[b, h])
        e = np.abs(og - o_ref)
        worst, total, count = max(worst, (e / (BF16_MAX + 2.0 ** -7 * np.abs(o_ref))).max()), total + e.sum(), count + e.size
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.all(og[~fin] == 0.0)
        if fin.any():
            worst_l = max(worst_l, np.abs(lg[fin] - lse_ref[fin]).max())
    say(f"[parity] {tag}: O worst err/bound {worst:.3f} mean {total / count:.3e} LSE max {worst_l:.3e}")
    assert worst <= 1.0 and total / count <= BF16_MEAN and worst_l <= BF16_LSE


def ramp_keys(q, k, growth):
    """Scores that grow along the keys: a shared direction u added to every query
    and, with a weight rising linearly to ``growth``, to every key.  The row max
    then moves up tile after tile, so the kernels must move their reference max
    (and rescale what they have accumulated) many times per row."""
    d, N = q.shape[-1], q.shape[-2]
    u = torch.ones(d) / math.sqrt(d)
    ramp = torch.linspace(0.0, growth, N)[:, None] * u
    return (q.float() + 4.0 * u).to(q.dtype), (k.float() + ramp).to(k.dtype)


# Full grids (256 heads or more): ragged lengths, padding, scores that keep
# rising (the rare path that moves a row's reference max and rescales its
# accumulators); every row of a few heads checked.  Head size 64 runs the
# 4-wave kernel at every length here, head size 128 the 4-wave kernel under
# 1024 keys and the 8-wave kernel from there, head size 256 the 8-wave kernel.
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_full_heads_ragged(d, causal):
    B, H = (1, 256) if not causal else (2, 256)
    for N in ((300, 511, 700, 1300) if not causal else (520, 777, 1300)):
        q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=N + causal + d)
        check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (0, 77), (B - 1, 255)],
                         f"large grid full heads N={N} d={d}")


# Shapes on both sides of each kernel-choice threshold of the bf16 forward
# pass (grid size G in workgroups of 256 query rows, key range N): every row
# of the first, a middle and the last head against the oracle.
@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 32, 1024, 128, False), (1, 33, 1024, 128, False),    # G = 128 (two key groups) | 132 (8-wave)
    (1, 32, 1024, 128, True), (1, 33, 1024, 128, True),
    (1, 64, 1023, 128, False), (1, 48, 767, 128, True),      # under 1024 keys: 4-wave; 767 keys, small grid
    (1, 64, 2048, 64, False), (1, 31, 2048, 64, False),      # G = 512 (8-wave) | 248 (4-wave)
    (1, 64, 2047, 64, False),                                # 2047 keys: 4-wave
    (1, 32, 4096, 64, True), (1, 32, 4095, 64, True),        # causal d = 64 from 4096 keys
    (1, 32, 2048, 256, True), (1, 31, 2048, 256, True),      # G = 256 (8-wave) | 248 (head-size-256 kernel)
])
def test_kernel_choice_thresholds(B, H, N, d, causal):
    q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=7 * N + H + d + int(causal))
    check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (0, H // 2), (B - 1, H - 1)],
                     f"threshold B={B} H={H} N={N} d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_full_heads_long_keys_d64(causal):
    # head size 64 with at least 2048 keys: 128-key tiles, in the 8-wave kernel
    # (non-causal) or in the 4-wave kernel (causal heads under 4096 keys)
    B, H, N = 1, 128, 2100
    q, k, v, _ = random_qkv(B, H, N, 64, torch.bfloat16, 1.0, seed=41 + causal)
    check_full_heads(q, k, v, 0.125, causal, None, [(0, 0), (0, 127)], "large grid full heads d=64 N=2100")
    q, k = ramp_keys(q, k, 120.0)
    check_full_heads(q, k, v, 0.125, causal, None, [(0, 1)], "large grid full heads d=64 N=2100 rising scores")


@pytest.mark.parametrize("causal", [False, True])
def test_long_keys_full_heads_d64_small_grid(causal):
    """Head size 64, 2048 keys or more, small grids.  Two heads of 8 (136
    workgroups of 128 rows) run the 4-wave kernel with the keys split over two
    groups of waves and 128-key tiles (a padded batch leaves the second group
    with few or no tiles); 24 heads (408 workgroups) run it with one key group
    (non-causal) or with two and 64-key tiles (causal).  Ragged tail, padding
    and rising scores."""
    B, H, N = 2, 4, 2100
    q, k, v, _ = random_qkv(B, H, N, 64, torch.bfloat16, 1.0, seed=51 + causal)
    check_full_heads(q, k, v, 0.125, causal, None, [(0, 0), (1, 3)], "4-wave 128-key tiles d=64 N=2100")
    sl = torch.tensor([2049, 700], dtype=torch.int32)
    check_full_heads(q, k, v, 0.125, causal, sl, [(0, 1), (1, 2)], "4-wave 128-key tiles d=64 N=2100 padding")
    q, k = ramp_keys(q, k, 120.0)
    check_full_heads(q, k, v, 0.125, causal, None, [(1, 0)], "4-wave 128-key tiles d=64 N=2100 rising scores")
    q, k, v, _ = random_qkv(1, 24, N, 64, torch.bfloat16, 1.0, seed=53 + causal)
    check_full_heads(q, k, v, 0.125, causal, None, [(0, 0), (0, 23)], "4-wave d=64 N=2100 24 heads")


@pytest.mark.parametrize("d,N", [(64, 1000), (128, 700)])
@pytest.mark.parametrize("causal", [False, True])
def test_small_grid_rising_scores(d, N, causal):
    """The 4-wave kernel with 64-key tiles (head size 64) and 32-key tiles (head
    size 128) on small grids, with scores that rise along the keys: the tile
    sums of P keep exceeding 2^8, so the tile max is computed and the reference
    moved many times per row; plus a gentle ramp that keeps P under 2^8 while
    the reference lags behind the true max."""
    for growth in (120.0, 6.0):
        q, k, v, _ = random_qkv(1, 2, N, d, torch.bfloat16, 1.0, seed=91 + d + causal + int(growth))
        q, k = ramp_keys(q, k, growth)
        check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (0, 1)],
                         f"4-wave small grid rising scores d={d} N={N} growth={growth}")


def test_long_keys_full_heads_d64_causal_large_grid():
    """Causal head size 64 with 4096 keys or more on 256 workgroups or more:
    the 8-wave kernel's 128-key tiles; every row of two heads."""
    B, H, N = 1, 16, 4100
    q, k, v, _ = random_qkv(B, H, N, 64, torch.bfloat16, 1.0, seed=57)
    check_full_heads(q, k, v, 0.125, True, None, [(0, 0), (0, 15)], "8-wave 128-key tiles causal d=64 N=4100")
    q, k = ramp_keys(q, k, 120.0)
    check_full_heads(q, k, v, 0.125, True, None, [(0, 7)], "8-wave 128-key tiles causal d=64 N=4100 rising scores")


@pytest.mark.parametrize("d,H", [(64, 1), (64, 2), (128, 2)])
def test_very_long_single_sequence(d, H):
    """One causal sequence of 32768 positions, every row of every head against
    the oracle.  Head size 64 with one head (256 workgroups of 128 rows) runs
    the 4-wave kernel with two key groups and 128-key tiles, each group
    streaming up to 128 tiles; with two heads (256 workgroups of 256 rows) the
    8-wave kernel with 128-key tiles; head size 128 with two heads the 8-wave
    kernel with 64-key tiles."""
    B, N = 1, 32768
    q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=99 + d + H)
    check_listed_heads(q, k, v, 1.0 / math.sqrt(d), True, None, [(0, h) for h in range(H)],
                       f"single sequence N={N} d={d} H={H}")


@pytest.mark.parametrize("causal", [False, True])
def test_long_keys_full_heads_d128_tiny_grid(causal):
    """Head size 128 from 768 keys on grids of at most 128 workgroups of 256
    rows runs the 4-wave kernel with the keys split over two groups of waves
    and 64-key tiles: every row of each head, ragged tails, padding (one row
    block with no keys for the second group) and rising scores."""
    for N in (768, 1024, 1500, 2100):
        q, k, v, _ = random_qkv(1, 2, N, 128, torch.bfloat16, 1.0, seed=61 + N + causal)
        check_full_heads(q, k, v, 1.0 / math.sqrt(128), causal, None, [(0, 0), (0, 1)],
                         f"two key groups d=128 tiny grid N={N}")
    q, k = ramp_keys(q, k, 120.0)
    check_full_heads(q, k, v, 1.0 / math.sqrt(128), causal, None, [(0, 1)], "two key groups d=128 rising scores")
    q, k, v, _ = random_qkv(2, 1, 1500, 128, torch.bfloat16, 1.0, seed=67 + causal)
    sl = torch.tensor([1025, 60], dtype=torch.int32)
    check_full_heads(q, k, v, 1.0 / math.sqrt(128), causal, sl, [(0, 0), (1, 0)], "two key groups d=128 tiny grid padding")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_large_grid_full_heads_padding(d):
    B, H, N = 6, 128, 600
    q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=17 + d)
    sl = torch.tensor([0, 1, 63, 257, 599, 600], dtype=torch.int32)
    for causal in (False, True):
        check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, sl, [(0, 3), (1, 5), (2, 0), (3, 127), (4, 64), (5, 9)],
                         f"large grid full heads padding causal={causal} d={d}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_full_heads_rising_scores(d, causal):
    B, H, N = 2, 256, 1100
    q, k, v, _ = random_qkv(B, H, N, d, torch.bfloat16, 1.0, seed=23 + causal + d)
    q, k = ramp_keys(q, k, 120.0)
    check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (1, 200)],
                     f"large grid full heads rising scores d={d}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(8, 4), (8, 2), (6, 1)])
def test_grouped_query_parity(H, H_kv, d, causal):
    for n, lens in [(200, None), (333, (1, 333))]:
        q, k, v, seqlens = random_qkv_grouped(2, H, H_kv, n, d, torch.bfloat16, 1.0, seed=40 + H_kv + n, len_range=lens)
        check_against_oracle(q, k, v, 1.0 / math.sqrt(d), causal, seqlens, fp32=False,
                             tag=f"grouped H={H} H_kv={H_kv} n={n} d={d}")


@pytest.mark.parametrize("d,N", [(64, 2100), (128, 1500)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_query_long_keys_small_grid(d, N, causal):
    """Grouped heads on the path small grids take with long key ranges: the
    4-wave kernel with two key groups (128-key tiles at d = 64, 64-key tiles at
    d = 128)."""
    q, k, v, seqlens = random_qkv_grouped(2, 4, 2, N, d, torch.bfloat16, 1.0, seed=80 + d + causal, len_range=(N // 2, N))
    check_full_heads(q, k, v, 1.0 / math.sqrt(d), causal, seqlens, [(0, 0), (0, 3), (1, 1)],
                     f"grouped long keys small grid d={d} N={N}")


def test_grouped_query_fp32():
    q, k, v, seqlens = random_qkv_grouped(2, 4, 2, 150, 64, torch.float32, 1.0, seed=5, len_range=(20, 150))
    check_against_oracle(q, k, v, 0.125, True, seqlens, fp32=True, tag="grouped fp32")


@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, False)])
def test_grouped_query_large_grid(d, causal):
    # multi-query (H_kv = 1) and groups of 4 on the 8-wave kernel
    for H_kv in (1, 8):
        N = 8192 if causal else 2048
        q, k, v, _ = random_qkv_grouped(1, 32, H_kv, N, d, torch.bfloat16, 1.0, seed=70 + H_kv)
        check_listed_heads(q, k, v, 1.0 / math.sqrt(d), causal, None, [(0, 0), (0, 5), (0, 31)],
                           f"grouped large H_kv={H_kv} d={d}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H", [(2, 8), (1, 4)])
def test_head_size_256_large_grid(B, H, causal):
    """Head size 256 with 4096 keys: 256 workgroups run the 8-wave kernel with
    32-key tiles, 64 the one-wave-per-SIMD head-size-256 kernel; every row of
    three heads against the oracle, and bitwise repeatable."""
    N = 4096
    q, k, v, _ = random_qkv(B, H, N, 256, torch.bfloat16, 0.5, seed=90 + causal)
    check_listed_heads(q, k, v, 1.0 / 16.0, causal, None, [(0, 0), (B - 1, 3), (B - 1, H - 1)], f"d=256 B={B} H={H}")
    o1, l1 = gpu_forward(q, k, v, 1.0 / 16.0, causal, None)
    o2, l2 = gpu_forward(q, k, v, 1.0 / 16.0, causal, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_head_size_256_long_context_full_size():
    """The configuration bench.py times for head size 256 (B = 1, H = 16,
    N = 16384, causal, std 0.5): every row of all 16 heads against the oracle."""
    q, k, v, _ = random_qkv_grouped(1, 16, 16, 16384, 256, torch.bfloat16, 0.5, 8)
    say(f"[parity] d=256 long context full size {tuple(q.shape)}")
    o, lse = gpu_forward(q, k, v, 1.0 / 16.0, True, None)
    og, lg = np64(o), np64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    emax, emean, lmax, wh = full_size_stats(og, lg, q, k, v, 1.0 / 16.0, True)
    say(f"[parity] d=256 long context all heads: O max {emax:.3e} (head {wh}) mean {emean:.3e} LSE max {lmax:.3e}")
    assert emax <= BF16_MAX and emean <= BF16_MEAN and lmax <= BF16_LSE


def test_grouped_query_equals_repeated_heads():
    # the kernel's grouped path against its own plain path on repeated K/V: bitwise equal
    q, k, v, _ = random_qkv_grouped(2, 8, 2, 257, 128, torch.bfloat16, 1.0, seed=9)
    o1, l1 = gpu_forward(q, k, v, 0.0884, True, None)
    kr, vr = k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = gpu_forward(q, kr, vr, 0.0884, True, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


RAGGED_N = [1, 2, 3, 7, 8, 31, 33, 63, 64, 65, 100, 127, 129, 255, 256, 257, 300, 513, 1000]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths_bf16(d, causal):
    for n in RAGGED_N:
        q, k, v, _ = random_qkv(2, 2, n, d, torch.bfloat16, 1.0, seed=1000 + n)
        check_against_oracle(q, k, v, 1.0 / math.sqrt(d), causal, None, fp32=False, tag=f"ragged n={n} d={d}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_padding_lengths_bf16(d, causal):
    n = 300
    q, k, v, _ = random_qkv(6, 2, n, d, torch.bfloat16, 1.0, seed=7)
    seqlens = torch.tensor([0, 1, 63, 64, 65, n], dtype=torch.int32)
    check_against_oracle(q, k, v, 0.125, causal, seqlens, fp32=False, tag=f"padding d={d}")


@pytest.mark.parametrize("B", [64, 65])
def test_many_batch_lengths_bf16(B):
    """Per-batch key lengths on a grid that is resident at once: with at most 64
    batches the workgroups are assigned by batch length (longest first), over 64
    the plain order is used.  Repeated lengths (ties), empty and full batches,
    every row of every head."""
    H, N = 4, 512
    q, k, v, _ = random_qkv(B, H, N, 64, torch.bfloat16, 1.0, seed=70 + B)
    g = torch.Generator().manual_seed(B)
    lens = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int32)
    lens[0], lens[1], lens[2], lens[3] = 0, N, N, 257
    lens[B - 1] = lens[B - 2]
    for causal in (False, True):
        check_against_oracle(q, k, v, 0.125, causal, lens, fp32=False, tag=f"many batch lengths B={B} causal={causal}")


def test_padding_lengths_out_of_range_are_clamped():
    n = 130
    q, k, v, _ = random_qkv(3, 1, n, 64, torch.bfloat16, 1.0, seed=8)
    seqlens = torch.tensor([-5, 10_000, 77], dtype=torch.int32)
    o, lse = gpu_forward(q, k, v, 0.125, False, seqlens)
    o_ref, lse_ref = oracle.attention(np64(q), np64(k), np64(v), 0.125, False, np.array([0, n, 77]))
    assert np.abs(np64(o) - o_ref).max() <= BF16_MAX
    assert np.all(np64(lse)[0] == -np.inf) and np.all(np64(o)[0] == 0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp32_path(d):
    for n, causal, lens in [(128, False, None), (1, False, None), (77, True, None), (200, False, [0, 150]),
                            (333, True, [333, 90])]:
        B = 1 if lens is None else len(lens)
        q, k, v, _ = random_qkv(B, 2, n, d, torch.float32, 1.0, seed=n)
        seqlens = None if lens is None else torch.tensor(lens, dtype=torch.int32)
        check_against_oracle(q, k, v, 1.0 / math.sqrt(d), causal, seqlens, fp32=True, tag=f"fp32 n={n} d={d}")


def test_identity_values_expose_the_softmax():
    """V = identity (N = d = 64): O = P, compared with the oracle's softmax matrix."""
    n = 64
    q, k, _, _ = random_qkv(1, 2, n, 64, torch.bfloat16, 1.0, seed=21)
    v = torch.eye(n, dtype=torch.bfloat16).expand(1, 2, n, n).contiguous()
    for causal in (False, True):
        o, _ = gpu_forward(q, k, v, 0.125, causal, None)
        for h in range(2):
            p, _, _ = oracle.softmax_matrix(np64(q)[0, h], np64(k)[0, h], 0.125, np.arange(n), n, causal)
            og = np64(o)[0, h]
            assert np.abs(og - p).max() <= 2 ** -8
            if causal:
                assert np.all(og[np.triu_indices(n, 1)] == 0.0)
            assert np.abs(og.sum(axis=1) - 1).max() <= 2e-2


def test_equal_value_rows_and_zero_queries():
    n, d = 200, 64
    q, k, v, seqlens = random_qkv(2, 2, n, d, torch.bfloat16, 1.0, seed=22, len_range=(50, 200))
    u = v[:, :, :1].expand(2, 2, n, d).contiguous()
    for causal in (False, True):
        o, _ = gpu_forward(q, k, u, 0.125, causal, seqlens)
        assert torch.allclose(o.float().cpu(), u.float(), atol=0, rtol=2 ** -7)
        z = torch.zeros_like(q)
        o, lse = gpu_forward(z, k, v, 0.125, causal, seqlens)
        o_ref, lse_ref = oracle.attention(np64(z), np64(k), np64(v), 0.125, causal, seqlens.numpy())
        assert np.abs(np64(o) - o_ref).max() <= BF16_MAX
        assert np.abs(np64(lse) - lse_ref).max() <= 1e-5  # every P is exactly 1: l counts keys


def test_lse_optional_and_bitwise_determinism():
    inp = make_inputs(3)
    q, k, v = (x.to(DEV) for x in (inp["q"], inp["k"], inp["v"]))
    outs = []
    for _ in range(3):
        o, lse = binding.attention_forward(q, k, v, inp["scale"], True, None)
        outs.append((o.clone(), lse.clone()))
    o2, none = binding.attention_forward(q, k, v, inp["scale"], True, None, want_lse=False)
    torch.cuda.synchronize()
    assert none is None
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    assert torch.equal(o2, outs[0][0])


def test_guard_bands_untouched():
    n, d, B, H = 257, 128, 1, 3
    q, k, v, _ = random_qkv(B, H, n, d, torch.bfloat16, 1.0, seed=23)
    pad = 4096
    canary_o = torch.full((pad * 2 + B * H * n * d,), 12288.0, dtype=torch.bfloat16, device=DEV)
    canary_l = torch.full((pad * 2 + B * H * n,), -777.0, dtype=torch.float32, device=DEV)
    o = canary_o[pad:pad + B * H * n * d].view(B, H, n, d)
    lse = canary_l[pad:pad + B * H * n].view(B, H, n)
    for causal in (False, True):
        binding.attention_forward(q.to(DEV), k.to(DEV), v.to(DEV), 0.0884, causal, None, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(canary_o[:pad] == 12288.0) and torch.all(canary_o[-pad:] == 12288.0)
        assert torch.all(canary_l[:pad] == -777.0) and torch.all(canary_l[-pad:] == -777.0)
        assert torch.isfinite(o.float()).all()


def test_non_default_stream():
    inp = make_inputs(4)
    q, k, v = (x.to(DEV) for x in (inp["q"], inp["k"], inp["v"]))
    ref, _ = binding.attention_forward(q, k, v, inp["scale"], False, None)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, _ = binding.attention_forward(q, k, v, inp["scale"], False, None)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_device_side_error_codes():
    x = torch.zeros(64 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    p = x.data_ptr()
    st = binding.fa_fwd(p + 2, p, p, p, None, 1, 1, 64, 64, 0.125, 0, None, None)
    assert st == binding.FA_ERR_MISALIGNED
    st = binding.fa_fwd(p, p, p, p, None, 1, 1, 64, 96, 0.125, 0, None, None)
    assert st == binding.FA_ERR_UNSUPPORTED
    with pytest.raises(binding.FaError):
        binding.attention_forward(x[:64 * 64].view(1, 1, 64, 64), x[:64 * 64].view(1, 1, 64, 64),
                                  x[:64 * 64].view(1, 1, 64, 64), float("nan"))


def test_wrappers_refuse_host_outputs_and_wide_lengths():
    """Outputs in host memory, or key-padding lengths as int64, next to device
    inputs are refused before any launch (a kernel would write to a host
    address, or read int64 lengths as pairs of int32)."""
    q, k, v, _ = random_qkv(2, 2, 64, 64, torch.bfloat16, 1.0, seed=3)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    with pytest.raises(ValueError, match="out"):
        binding.attention_forward(qd, kd, vd, 0.125, out=torch.empty_like(q))
    with pytest.raises(ValueError, match="lse"):
        binding.attention_forward(qd, kd, vd, 0.125, lse=torch.empty(2, 2, 64))
    with pytest.raises(ValueError, match="seqlens"):
        binding.attention_forward(qd, kd, vd, 0.125, seqlens=torch.tensor([64, 50], device=DEV))
    with pytest.raises(ValueError, match="seqlens"):
        binding.attention_forward(qd, kd, vd, 0.125, seqlens=torch.tensor([64, 50], dtype=torch.int32))
    with pytest.raises(ValueError, match="workspace"):
        binding.decode_forward(qd[:, :, :1].contiguous(), kd, vd, 0.125, workspace=torch.empty(1 << 20, dtype=torch.uint8))


def test_clock_sample_reads_each_unit():
    """fa_clock_sample: the counters advance between two samples around
    back-to-back kernel launches, most compute units (of all 8 XCDs) pair up
    between the two samples, and cycles per 100 MHz tick give a core clock
    within the chip's range."""
    n_vals = 3 * binding.FA_CLOCK_SAMPLE_UNITS
    buf = torch.zeros(2 * n_vals, dtype=torch.int64, device=DEV)
    inp = make_inputs(4)
    q, k, v = (x.to(DEV) for x in (inp["q"], inp["k"], inp["v"]))
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *q.shape, inp["scale"], False, None, st)
    assert binding.fa_clock_sample(buf.data_ptr(), st) == binding.FA_OK
    for _ in range(20):
        assert binding.fa_fwd(*args) == binding.FA_OK
    assert binding.fa_clock_sample(buf.data_ptr() + n_vals * 8, st) == binding.FA_OK
    torch.cuda.synchronize()
    vals = buf.cpu().tolist()
    mhz = binding.clock_mhz_by_unit(vals[:n_vals], vals[n_vals:])
    xcds = sorted({key >> 16 for key in mhz})
    m = sorted(mhz.values())
    say(f"[clock] {len(m)} units paired on XCDs {xcds}: median {m[len(m) // 2]:.0f} MHz, "
        f"range {m[0]:.0f}..{m[-1]:.0f}")
    assert xcds == list(range(8)) and len(m) >= 128
    assert 100.0 <= m[len(m) // 2] <= 2600.0
