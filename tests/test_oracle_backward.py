"""The backward oracle (``oracle.attention_backward``) against its pins (CPU only).

The gradients are pinned to things other than their own formula:

* central finite differences of the forward oracle, which is itself pinned
  (tests/oracle_pins.py), for the loss L = sum(O * G): the derivative of the
  definition, whatever formula computes it;
* torch's autograd through a plain float64 attention on the CPU (a library
  routine, used only here);
* identities of the definition: the key gradients of a head sum to zero (the
  output does not change when every key moves by the same vector), the value
  gradients sum to the output gradients of the rows that see a key, Q = 0 gives
  dK = 0, dO = 0 gives zero, the gradient is linear in dO, causal row 0 (one
  key) gets dQ = 0;
* the row blocking of the oracle does not change its result.

``test_backward_pins_catch_planted_mistake`` plants plausible mistakes in a copy
of the chain rule and requires a pin to fail for each.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_backward

SCALE = 0.7


def _inputs(B, H, H_kv, N, d, seed, padded):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H_kv, N, d))
    v = rng.normal(size=(B, H_kv, N, d))
    g = rng.normal(size=(B, H, N, d))
    seqlens = None
    if padded:
        seqlens = np.array([(N * (b + 1)) // (B + 1) + b for b in range(B)])
        seqlens[0] = 0 if B > 2 else seqlens[0]
    return q, k, v, g, seqlens


CASES = [  # (B, H, H_kv, N, d, causal, padded)
    (1, 1, 1, 1, 3, False, False),
    (2, 2, 2, 5, 3, False, False),
    (2, 2, 2, 5, 3, True, False),
    (3, 2, 1, 4, 2, False, True),
    (2, 4, 2, 5, 3, True, True),
]


def _fd_gradients(q, k, v, g, causal, seqlens, step=1e-5):
    """Central differences of L = sum(O * G) with O from the forward oracle."""
    def loss(q_, k_, v_):
        return float((attention(q_, k_, v_, SCALE, causal, seqlens)[0] * g).sum())

    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        gx = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + step
            lp = loss(*args)
            x[idx] = old - step
            lm = loss(*args)
            x[idx] = old
            gx[idx] = (lp - lm) / (2 * step)
        grads.append(gx)
    return grads


def pin_finite_differences(fn):
    for i, (B, H, H_kv, N, d, causal, padded) in enumerate(CASES):
        q, k, v, g, sl = _inputs(B, H, H_kv, N, d, 100 + i, padded)
        got = fn(q, k, v, g, SCALE, causal, sl)
        ref = _fd_gradients(q, k, v, g, causal, sl)
        for name, a, r in zip("qkv", got, ref):
            assert a.shape == r.shape, name
            np.testing.assert_allclose(a, r, rtol=1e-6, atol=1e-7, err_msg=f"d{name}, case {i}")


def _torch_gradients(q, k, v, g, causal, seqlens):
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    B, H, N, _ = q.shape
    rep = H // k.shape[1]
    kk, vv = kt.repeat_interleave(rep, dim=1), vt.repeat_interleave(rep, dim=1)
    s = SCALE * (qt @ kk.transpose(-1, -2))
    allowed = torch.ones(B, 1, N, N, dtype=torch.bool)
    if seqlens is not None:
        allowed &= (torch.arange(N)[None, :] < torch.tensor(seqlens)[:, None])[:, None, None, :]
    if causal:
        allowed &= torch.ones(N, N, dtype=torch.bool).tril()
    o = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=-1) @ vv
    (o * torch.tensor(g)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_torch_autograd(fn):
    # every row keeps at least one key here (torch's softmax of an empty row is NaN)
    for i, (B, H, H_kv, N, d, causal) in enumerate([(2, 4, 4, 33, 8, False), (2, 4, 2, 40, 8, True),
                                                    (1, 6, 1, 17, 5, False)]):
        q, k, v, g, _ = _inputs(B, H, H_kv, N, d, 200 + i, False)
        sl = np.array([N - 3 - b for b in range(B)]) if not causal else None
        got = fn(q, k, v, g, SCALE, causal, sl)
        ref = _torch_gradients(q, k, v, g, causal, sl)
        for name, a, r in zip("qkv", got, ref):
            np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-11, err_msg=f"d{name}, case {i}")


def pin_identities(fn):
    B, H, H_kv, N, d = 3, 4, 2, 30, 6
    for causal in (False, True):
        q, k, v, g, sl = _inputs(B, H, H_kv, N, d, 300 + causal, True)
        dq, dk, dv = fn(q, k, v, g, SCALE, causal, sl)
        # moving every key of a head by one vector leaves O unchanged
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-10)
        # the weights of a row that sees a key sum to one; every row sees key 0
        # (also when causal) unless its batch has no valid key
        L = np.clip(sl, 0, N)
        rows_see = np.repeat((L > 0)[:, None], N, axis=1)
        gs = (g * rows_see[:, None, :, None]).reshape(B, H_kv, H // H_kv, N, d).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), gs, atol=1e-10)
        # Q = 0: dK = scale dS^T Q = 0
        _, dk0, _ = fn(np.zeros_like(q), k, v, g, SCALE, causal, sl)
        assert np.all(dk0 == 0.0)
        # dO = 0: no gradient at all
        for x in fn(q, k, v, np.zeros_like(g), SCALE, causal, sl):
            assert np.all(x == 0.0)
        # linear in dO
        g2 = np.random.default_rng(7).normal(size=g.shape)
        a = fn(q, k, v, 2.5 * g + g2, SCALE, causal, sl)
        b1 = fn(q, k, v, g, SCALE, causal, sl)
        b2 = fn(q, k, v, g2, SCALE, causal, sl)
        for x, y, z in zip(a, b1, b2):
            np.testing.assert_allclose(x, 2.5 * y + z, atol=1e-10)
    # causal row 0 sees key 0 alone: its softmax is the constant 1
    q, k, v, g, _ = _inputs(2, 2, 2, 9, 4, 9, False)
    dq, _, _ = fn(q, k, v, g, SCALE, True, None)
    assert np.all(dq[:, :, 0] == 0.0)
    # rows past a batch's padding length still see the valid keys; a batch with no key has no gradient
    q, k, v, g, _ = _inputs(2, 2, 2, 9, 4, 10, False)
    dq, dk, dv = fn(q, k, v, g, SCALE, False, np.array([0, 4]))
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)
    assert np.all(dk[1, :, 4:] == 0) and np.all(dv[1, :, 4:] == 0) and np.all(dq[1, :, 8] != 0)


BACKWARD_PINS = [pin_finite_differences, pin_torch_autograd, pin_identities]


def oracle_bwd(q, k, v, g, scale, causal, seqlens):
    return attention_backward(q, k, v, g, scale, causal, seqlens)


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle_bwd)


def test_row_blocks_do_not_change_the_result():
    q, k, v, g, sl = _inputs(2, 4, 2, 70, 8, 11, True)
    for causal in (False, True):
        a = attention_backward(q, k, v, g, SCALE, causal, sl, row_block=1024)
        b = attention_backward(q, k, v, g, SCALE, causal, sl, row_block=9)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_backward_exported():
    assert oracle.attention_backward is attention_backward


# ---------------------------------------------------------------------------------
# Planted mistakes: a copy of the chain rule with one plausible error each.
# ---------------------------------------------------------------------------------
def _chain_rule_copy(q, k, v, g, scale, causal, seqlens, bug=None):
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = N if seqlens is None else min(max(int(seqlens[b]), 0), N)
        for h in range(H):
            gh = h % H_kv if bug == "interleaved_heads" else h // (H // H_kv)
            rows = np.arange(N)
            p, _, _ = oracle.softmax_matrix(q[b, h], k[b, gh], scale, rows, N if bug == "padding_ignored" else L,
                                            False if bug == "causal_ignored" else causal)
            dp = g[b, h] @ v[b, gh].T
            dsum = dp.sum(axis=1) if bug == "D_without_P" else (p * dp).sum(axis=1)
            ds = p * dp if bug == "no_D" else p * (dp - dsum[:, None])
            ds_k = ds.T if bug == "dK_untransposed" else ds
            dv_b = p @ g[b, h] if bug == "dV_untransposed" else p.T @ g[b, h]
            if bug == "gqa_overwrite":
                dv[b, gh] = dv_b
            else:
                dv[b, gh] += dv_b
            dq[b, h] = (1.0 if bug == "dQ_unscaled" else scale) * (ds @ k[b, gh])
            dk[b, gh] += scale * (ds_k.T @ q[b, h])
    return dq, dk, dv


BUGS = ["no_D", "D_without_P", "dK_untransposed", "dV_untransposed", "dQ_unscaled", "gqa_overwrite",
        "interleaved_heads", "causal_ignored", "padding_ignored"]


def test_unplanted_copy_passes_every_backward_pin():
    for pin in BACKWARD_PINS:
        pin(lambda *a: _chain_rule_copy(*a))


@pytest.mark.parametrize("bug", BUGS)
def test_backward_pins_catch_planted_mistake(bug):
    failed = []
    for pin in BACKWARD_PINS:
        try:
            pin(lambda *a: _chain_rule_copy(*a, bug=bug))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {bug!r}"
