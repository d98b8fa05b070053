"""Every row of many heads against the oracle, with the heads spread over threads.

Test infrastructure.  numpy releases the interpreter lock inside its array
loops, so whole heads of a large problem are computed concurrently on the host
cores; BLAS runs one thread per worker so the workers do not oversubscribe
them.  The oracle itself is called unchanged, a block of query rows at a time.
Causal row blocks hand it only the keys up to the block's last row: the causal
mask drops every later key, so the result is the same as over all keys.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

MAX_WORKERS = 16   # at most the host share of one GPU machine


def host_workers():
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def oracle_head(q, k, v, scale, causal, valid_len=None, row_block=1024):
    """O [N, d] and LSE [N] (float64) of one head.

    q is [N, d], k and v are [N_k, d] (any float dtype; the oracle reads them as
    float64); valid_len is the head's key-padding length or None.
    """
    N = q.shape[0]
    o = np.empty((N, v.shape[1]))
    lse = np.empty(N)
    sl = None if valid_len is None else np.array([int(valid_len)])
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        kend = min(k.shape[0], r1) if causal else k.shape[0]
        o[r0:r1], lse[r0:r1] = oracle.attention_rows(q[None, None], k[None, None, :kend], v[None, None, :kend], scale,
                                                     causal, sl, 0, 0, np.arange(r0, r1))
    return o, lse


def map_heads(fn, items, workers=None):
    """[fn(item) for item in items], computed on a pool of host threads."""
    workers = workers or host_workers()
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl is optional
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))
    finally:
        if limit is not None:
            limit.restore_original_limits()
