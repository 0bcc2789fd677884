"""Pins of the oracle's FP8 E4M3 path (``oracle.fp8_e4m3_to_float``,
``oracle.attention_fp8``), and planted mistakes in the decoder that the pins
must catch.

The format is OCP FP8 E4M3 ("e4m3fn"): sign bit 7, exponent bits 6:3 with
bias 7, mantissa bits 2:0, subnormals at exponent 0, NaN at 0x7F/0xFF, no
infinities.  torch's float8_e4m3fn is an independent implementation of it.
"""
import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd.inputs import as_oracle_array, make_inputs, quantize_fp8

CODES = np.arange(256, dtype=np.uint8)


def pin_library(decode):
    got = decode(CODES)
    ref = torch.from_numpy(CODES).view(torch.float8_e4m3fn).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)[0][:8]


def pin_hand_values(decode):
    # (code, value) from the format's definition
    table = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
             (0x3C, 1.5), (0x77, 240.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9))]
    got = decode(np.array([c for c, _ in table], np.uint8))
    np.testing.assert_array_equal(got, np.array([v for _, v in table]))
    assert np.isnan(decode(np.array([0x7F, 0xFF], np.uint8))).all()


DECODE_PINS = [pin_library, pin_hand_values]


@pytest.mark.parametrize("pin", DECODE_PINS, ids=lambda f: f.__name__)
def test_fp8_decode_pin(pin):
    pin(oracle.fp8_e4m3_to_float)


MUTANTS = [
    ("bias_8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("subnormal_as_normal", "np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))",
     "(1.0 + m / 8.0) * np.exp2(e - 7.0)"),
    ("nan_as_480", "mag = np.where((e == 15) & (m == 7), np.nan, mag)", "mag = mag"),
    ("sign_dropped", "sign = np.where(c >> 7, -1.0, 1.0)", "sign = 1.0"),
    ("mantissa_over_16", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
    ("subnormal_scale", "m * 2.0 ** -9", "m * 2.0 ** -10"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_fp8_mutant(name, old, new):
    src = textwrap.dedent(inspect.getsource(oracle.fp8_e4m3_to_float))
    assert old in src, f"mutation anchor for {name} not found"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    failures = 0
    for pin in DECODE_PINS:
        try:
            pin(ns["fp8_e4m3_to_float"])
        except AssertionError:
            failures += 1
    assert failures, f"mutant {name} passed every pin"


def _case(seed, lens=(40, 17), D=16):
    q, k, v, cl = make_inputs(len(lens), 4, 2, D, 1, max(lens), "bf16", seed, cache_lens=list(lens))
    kc, vc = quantize_fp8(k, 1 / 16), quantize_fp8(v, 1 / 16)
    return as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy()


def test_attention_fp8_scales_enter_exactly(oracle_lib):
    q, kc, vc, lens = _case(31)
    s = 0.25
    # k_scale = 8 (a power of two): the same as keys multiplied by 8 in float32
    kf = oracle.fp8_e4m3_to_float(kc).astype(np.float32)
    vf = oracle.fp8_e4m3_to_float(vc).astype(np.float32)
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    ref = oracle.attention(qf, kf * np.float32(8), vf, lens, s, lib=oracle_lib)
    got = oracle.attention_fp8(q, kc, vc, lens, s, 8.0, 1.0, lib=oracle_lib)
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[1], ref[1], rtol=0, atol=1e-13)
    # v_scale multiplies the output and leaves lse alone
    got3 = oracle.attention_fp8(q, kc, vc, lens, s, 8.0, 3.0, lib=oracle_lib)
    np.testing.assert_allclose(got3[0], 3.0 * got[0], rtol=1e-15, atol=0)
    np.testing.assert_array_equal(got3[1], got[1])


def test_attention_fp8_single_key_closed_form(oracle_lib):
    q, kc, vc, lens = _case(32, lens=(1,), D=8)
    ks, vs, s = 0.0625, 0.5, 0.3
    out, lse = oracle.attention_fp8(q, kc, vc, lens, s, ks, vs, lib=oracle_lib)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k0 = oracle.fp8_e4m3_to_float(kc[0, :, 0, :]) * ks  # [Hkv, D]
    v0 = oracle.fp8_e4m3_to_float(vc[0, :, 0, :]) * vs
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(out[0, h, 0], v0[g], rtol=1e-15, atol=0)
        expect = float(np.float32(s)) * float(qf[0, h, 0] @ k0[g])
        assert math.isclose(lse[0, h, 0], expect, rel_tol=1e-14, abs_tol=1e-14)
