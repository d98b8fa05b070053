"""CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code, table or helper with the
HIP library in ``exact_io_aware_57_amd/``.

What it computes is the plain definition the pages give for attention,
Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, with the full N x N score
matrix S materialised (FlashAttention (UR), section "The problem of standard
attention"; the same formula in FlashAttention (FA)).  The pages state that the
tiled, online-softmax method reaches exactly this result (FlashAttention (UR),
section "Online computation of softmax"; FlashAttention-2 (HI), introduction and
"Performance and efficiency"), so the definition, not the tiled algorithm, is the
oracle.  Everything is float64.

Modules
-------
attention : the definition in numpy float64 (``attention``, ``attention_rows``,
            ``softmax_matrix``, ``kv_head`` for grouped / multi-query
            attention, ``attention_decode`` for a few queries against a key
            cache, ``merge_partials`` for combining results over disjoint key
            sets, ``e4m3_decode`` and ``attention_fp8`` for FP8 inputs with
            per-tensor scales).  Every function is pinned by tests/test_oracle.py.
backward  : ``attention_backward``, the gradients dQ, dK, dV of the definition by
            the chain rule (the pages give no backward algorithm).
brute     : the same definition as scalar Python loops with ``math.exp`` and
            ``math.fsum`` and no max shift; a second, independent code path used
            only to pin ``attention`` on tiny inputs.
"""
from .attention import (  # noqa: F401
    allowed_mask, attention, attention_decode, attention_fp8, attention_rows, decode_allowed, e4m3_decode, kv_head,
    merge_partials, softmax_matrix,
)
from .backward import attention_backward  # noqa: F401
from .brute import attention_brute  # noqa: F401
