"""The FP8 part of the oracle against its pins (CPU only).

``oracle.e4m3_decode`` is written from the definition of the OCP e4m3 format;
it is pinned to torch's float8_e4m3fn type (a library routine, used only here)
on all 256 codes, to values of the format fixed by its definition, and to
monotonicity.  ``oracle.attention_fp8`` is the pinned forward oracle applied to
the decoded, descaled tensors; it is pinned by agreement with that oracle on
small-integer inputs, whose codes are exact.  Planted mistakes in a copy of the
decoder (the other 8-bit layout's exponent bias, a wrong subnormal scale, a
dropped sign, a mantissa of four bits) must each fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_fp8, e4m3_decode
from exact_io_aware_57_amd.inputs import random_qkv_fp8


def torch_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).double().numpy()


def pin_library(fn):
    got, ref = fn(np.arange(256)), torch_values()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def pin_format_values(fn):
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875,
             0x40: 2.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert fn(np.array([c]))[0] == v, hex(c)
    assert np.signbit(fn(np.array([0x80]))[0]) and fn(np.array([0x80]))[0] == 0.0
    assert np.isnan(fn(np.array([0x7F]))[0]) and np.isnan(fn(np.array([0xFF]))[0])


def pin_monotone(fn):
    pos = fn(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(fn(np.arange(0x80, 0xFF)), -pos)


DECODE_PINS = [pin_library, pin_format_values, pin_monotone]


@pytest.mark.parametrize("pin", DECODE_PINS, ids=lambda p: p.__name__)
def test_decode_pin(pin):
    pin(e4m3_decode)


def _decoder_copy(codes, bug):
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = 1.0 if bug == "sign_dropped" else np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    frac = 16.0 if bug == "mantissa_over_16" else 8.0
    bias = 8.0 if bug == "bias_8" else 7.0
    sub = -7.0 if bug == "subnormal_2^-7" else -6.0
    mag = np.where(e == 0, m / frac * 2.0 ** sub, (1.0 + m / frac) * np.exp2(e - bias))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


@pytest.mark.parametrize("bug", ["sign_dropped", "mantissa_over_16", "bias_8", "subnormal_2^-7"])
def test_decode_pins_catch_planted_mistake(bug):
    failed = 0
    for pin in DECODE_PINS:
        try:
            pin(lambda c: _decoder_copy(c, bug))
        except AssertionError:
            failed += 1
    assert failed, bug


def test_unplanted_decoder_copy_passes():
    for pin in DECODE_PINS:
        pin(lambda c: _decoder_copy(c, None))


def test_attention_fp8_is_the_definition_on_exact_codes():
    """Small integers and halves are exact e4m3 codes: the FP8 oracle on their
    codes equals the forward oracle on the values themselves."""
    rng = np.random.default_rng(3)
    vals = np.array([-4.0, -2.0, -1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
    lut = {v: int(np.flatnonzero(torch_values() == v)[0]) for v in vals}
    shape = (2, 2, 37, 16)
    xs = [vals[rng.integers(0, len(vals), size=shape)] for _ in range(3)]
    codes = [np.vectorize(lut.get)(x) for x in xs]
    for causal in (False, True):
        o, lse = attention_fp8(*codes, 0.25, (0.5, 2.0, 3.0), causal, np.array([37, 20]))
        o_ref, lse_ref = attention(0.5 * xs[0], 2.0 * xs[1], 3.0 * xs[2], 0.25, causal, np.array([37, 20]))
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_fp8_inputs_are_seeded_and_within_range():
    a = random_qkv_fp8(2, 4, 2, 100, 64, seed=5, len_range=(10, 100))
    b = random_qkv_fp8(2, 4, 2, 100, 64, seed=5, len_range=(10, 100))
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y) and x.dtype == torch.uint8
    assert a[3] == b[3] and torch.equal(a[4], b[4])
    for codes, s in zip(a[:3], a[3]):
        v = e4m3_decode(codes.numpy())
        assert np.isfinite(v).all() and np.abs(v).max() == 448.0 and s > 0
    assert a[0].shape == (2, 4, 100, 64) and a[1].shape == (2, 2, 100, 64)


def test_oracle_exports_fp8():
    assert oracle.attention_fp8 is attention_fp8 and oracle.e4m3_decode is e4m3_decode
