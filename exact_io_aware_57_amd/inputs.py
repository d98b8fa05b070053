"""Seeded synthetic inputs for the attention forward pass.

This module draws numbers and nothing else: it holds no part of the attention
arithmetic, so the HIP path and the CPU oracle can both take their inputs from
it without sharing any of the method.

Workloads.  The pages measure FlashAttention on BERT-large at sequence length
512, GPT-2 at 1K and Long-Range Arena at 1K-4K, and discuss context windows that
grow far beyond that (FlashAttention (UR), sections "Experimental results" and
"Industry impact"; FlashAttention-2 (HI), "Performance and efficiency").  No
dataset, weights or benchmark item is used: each workload below takes only the
shape of such a model's attention layer and fills Q, K, V with i.i.d. normal
values drawn from a seeded CPU ``torch.Generator`` in float32, then rounded to
bfloat16 (round to nearest even) for the bf16 workloads.  Key-padding lengths
are drawn from the same generator.
"""
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "random_qkv", "random_qkv_grouped", "random_seqlens"]


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp32" or "bf16": storage and input type of Q, K, V, O
    causal: bool
    std: float            # standard deviation of the i.i.d. normal entries
    scale: float          # the float32 softmax scale handed to the kernel
    len_range: Optional[Tuple[int, int]] = None   # key-padding lengths, inclusive

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def padded(self):
        return self.len_range is not None

    def describe(self):
        mask = "causal" if self.causal else "non-causal"
        if self.padded:
            mask += f", key padding U{{{self.len_range[0]}..{self.len_range[1]}}}"
        return f"{self.name}: B={self.B} H={self.H} N={self.N} d={self.d} {self.dtype} {mask}"


def _f32(x):
    return float(torch.tensor(x, dtype=torch.float32))


WORKLOADS = {
    1: Workload(1, "tiny", 1, 1, 128, 64, "fp32", False, 1.0, _f32(1.0 / 8.0)),
    2: Workload(2, "bert_large_shaped", 16, 16, 512, 64, "bf16", False, 1.0, _f32(1.0 / 8.0), (256, 512)),
    3: Workload(3, "gpt2_small_shaped", 8, 12, 1024, 64, "bf16", True, 1.0, _f32(1.0 / 8.0)),
    4: Workload(4, "long_sequence", 2, 8, 4096, 64, "bf16", False, 1.0, _f32(1.0 / 8.0)),
    5: Workload(5, "long_context", 1, 32, 16384, 128, "bf16", True, 0.5, _f32(1.0 / math.sqrt(128.0))),
}


def workload(index):
    return WORKLOADS[int(index)]


def random_seqlens(B, lo, hi, generator):
    """B key-padding lengths, uniform on the integers lo..hi inclusive, int32."""
    return torch.randint(lo, hi + 1, (B,), generator=generator, dtype=torch.int64).to(torch.int32)


def random_qkv(B, H, N, d, dtype=torch.bfloat16, std=1.0, seed=0, len_range=None):
    """Q, K, V as [B, H, N, d] CPU tensors of ``dtype`` (+ int32 seqlens or None).

    Entries are i.i.d. N(0, std^2), drawn in float32 from a CPU generator seeded
    with ``seed`` (in the order q, k, v, then the lengths) and rounded to
    ``dtype``.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        out.append(x.to(dtype).contiguous())
    seqlens = None
    if len_range is not None:
        seqlens = random_seqlens(B, len_range[0], len_range[1], g)
    return out[0], out[1], out[2], seqlens


def random_qkv_grouped(B, H, H_kv, N, d, dtype=torch.bfloat16, std=1.0, seed=0, len_range=None):
    """Q as [B, H, N, d] and K, V as [B, H_kv, N, d] CPU tensors (+ seqlens or None),
    drawn like ``random_qkv`` (q, k, v, then the lengths, from one seeded generator)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for shape in ((B, H, N, d), (B, H_kv, N, d), (B, H_kv, N, d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        out.append(x.to(dtype).contiguous())
    seqlens = None
    if len_range is not None:
        seqlens = random_seqlens(B, len_range[0], len_range[1], g)
    return out[0], out[1], out[2], seqlens


def random_decode(B, H, H_kv, Nq, Nk, d, dtype=torch.bfloat16, std=1.0, seed=0, len_range=None):
    """Decode inputs: Q [B, H, Nq, d] and the cache K, V [B, H_kv, Nk, d] as CPU
    tensors (+ per-batch cache lengths drawn from len_range, or None), all from
    one seeded generator in that order."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for shape in ((B, H, Nq, d), (B, H_kv, Nk, d), (B, H_kv, Nk, d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        out.append(x.to(dtype).contiguous())
    seqlens = None
    if len_range is not None:
        seqlens = random_seqlens(B, len_range[0], len_range[1], g)
    return out[0], out[1], out[2], seqlens


def random_qkv_fp8(B, H, H_kv, N, d, std=1.0, seed=0, len_range=None):
    """FP8 (e4m3) inputs with per-tensor scales: (q8, k8, v8, descale, seqlens).

    Q [B, H, N, d] and K, V [B, H_kv, N, d] are drawn like ``random_qkv_grouped``
    in float32, each tensor is divided by descale = max|x| / 448 so that its
    largest magnitude is the format's largest finite value, and rounded to e4m3
    by torch (round to nearest even).  q8, k8, v8 are uint8 CPU tensors of the
    codes; descale is a tuple of three floats, the tensor a code array stands
    for being descale * value(code)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    codes, descale = [], []
    for shape in ((B, H, N, d), (B, H_kv, N, d), (B, H_kv, N, d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        s = float(x.abs().max()) / 448.0
        s = s if s > 0 else 1.0
        codes.append((x / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).contiguous())
        descale.append(s)
    seqlens = None
    if len_range is not None:
        seqlens = random_seqlens(B, len_range[0], len_range[1], g)
    return codes[0], codes[1], codes[2], tuple(descale), seqlens


def make_inputs(index, seed=None):
    """Inputs of a numbered workload: dict(q, k, v, seqlens, scale, causal, wl).

    The default seed is the workload's index.
    """
    wl = workload(index)
    seed = wl.index if seed is None else seed
    q, k, v, seqlens = random_qkv(wl.B, wl.H, wl.N, wl.d, wl.torch_dtype, wl.std, seed, wl.len_range)
    return dict(q=q, k=k, v=v, seqlens=seqlens, scale=wl.scale, causal=wl.causal, wl=wl)
