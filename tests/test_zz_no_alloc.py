"""fa_decode_noalloc (the decode step with the library's static scratch instead
of a caller workspace) against fa_decode with a workspace, through the C-ABI.

Both entry points run the same kernels with the same key splits, so the
outputs must be bitwise equal; each is also held to the decode tolerances
against the oracle.  Two calls in a row share the GPU's one scratch array: the
second, smaller call must not see anything of the first.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_57_amd import binding
from exact_io_aware_57_amd.inputs import random_decode
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_MAX, BF16_MEAN, BF16_LSE = 1e-2, 1e-3, 1e-3


def say(msg):
    print(msg, flush=True)


def np64(t):
    return t.detach().float().cpu().double().numpy()


def both(B, H, H_kv, Nq, Nk, d, causal, len_range, seed):
    q, k, v, sl = random_decode(B, H, H_kv, Nq, Nk, d, std=0.5, seed=seed, len_range=len_range)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if sl is None else sl.to(DEV)
    need = binding.fa_decode_workspace_size(B, H, H_kv, Nq, Nk, d, 0)
    assert 0 < need <= binding.FA_DECODE_NOALLOC_SCRATCH_BYTES
    say(f"[noalloc] B={B} H={H} H_kv={H_kv} Nq={Nq} Nk={Nk} d={d} causal={causal} lens={None if sl is None else sl.tolist()} "
        f"partials {need} bytes")
    o_ref, l_ref = binding.decode_forward(qd, kd, vd, scale, causal, sd)
    o, lse = torch.empty_like(qd), torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    st = binding.fa_decode_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv,
                                   Nq, Nk, d, scale, causal, None if sd is None else sd.data_ptr(), 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == binding.FA_OK, binding.fa_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    oo, ll = oracle.attention_decode(np64(q), np64(k), np64(v), scale, causal, None if sl is None else sl.numpy())
    og, lg = np64(o), np64(lse)
    err = np.abs(og - oo)
    err_r = np.abs(og - torch.from_numpy(oo).to(torch.bfloat16).double().numpy())
    fin = np.isfinite(ll)
    assert np.array_equal(np.isfinite(lg), fin)
    lerr = np.abs(lg[fin] - ll[fin]).max() if fin.any() else 0.0
    say(f"[noalloc] O max {err.max():.3e} mean vs bf16-rounded {err_r.mean():.3e} LSE max {lerr:.3e}")
    assert err.max() <= BF16_MAX and err_r.mean() <= BF16_MEAN and lerr <= BF16_LSE


def test_noalloc_matches_workspace_entry_two_calls():
    # the bench decode step (8 key splits, about 1 MiB of partials) ...
    both(8, 32, 8, 1, 32768, 128, True, None, seed=7)
    # ... then a smaller one with padding, grouped heads and several queries
    both(2, 4, 2, 3, 1000, 64, True, (1, 1000), seed=15)
