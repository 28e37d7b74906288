"""Pins of oracle.formats against the pages and against independent routines."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import loops
from oracle.formats import (E2M1_MAGNITUDES, E4M3_TABLE, bf16_from_f64, bf16_to_f32,
                            e2m1_decode, e2m1_encode_magnitude, e4m3_decode,
                            e4m3_encode_nonneg)


def test_e2m1_value_set_matches_pages():
    # src commit log, quantizer fix: bit 3 sign, bits 2:0 index {0,.5,1,1.5,2,3,4,6}
    for nib, val in read_golden("e2m1_values.txt"):
        nib, val = int(nib), float(val)
        got = e2m1_decode(np.array([nib]))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val)
        assert float(loops.e2m1_value(nib)) == abs(val) * (-1 if nib & 8 else 1)


def test_e4m3_decode_is_bit_reinterpretation():
    # a scale byte IS an E4M3 bit pattern (src commit log, `.view` vs `.to` fix);
    # torch's float8_e4m3fn reinterpretation is an independent decoder.
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = E4M3_TABLE
    nan = np.isnan(ref)
    assert (nan == np.isnan(ours)).all()
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert (ref[~nan] == ours[~nan]).all()
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert float(loops.e4m3_value(c)) == ours[c]


def test_e4m3_byte_0x3f_is_1_875_not_0_984():
    # The pages print "~0.984" for byte 0x3F; under E4M3FN it decodes to 1.875.
    # The invariant kept is the reinterpretation itself; the printed number is
    # rejected (no E4M3 code equals 0.984: the neighbours are 0.9375 and 1.0).
    assert e4m3_decode(np.array([0x3F]))[0] == 1.875
    assert e4m3_decode(np.array([0x37]))[0] == 0.9375
    assert e4m3_decode(np.array([0x38]))[0] == 1.0
    assert e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_encoder_matches_torch_conversion_dense_sweep():
    # torch's float -> float8_e4m3fn conversion rounds to nearest even; sweep all
    # float32 values between codes at a fine grid plus every exact midpoint.
    codes = E4M3_TABLE[:127]
    mids = (codes[:-1] + codes[1:]) / 2
    grid = np.linspace(0, 448, 200001)
    pts = np.concatenate([codes, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), grid])
    pts = np.clip(pts.astype(np.float32), 0, 448).astype(np.float64)
    ours = e4m3_encode_nonneg(pts)
    ref = torch.from_numpy(pts.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e4m3_encoder_ties_to_even_code():
    # midpoint of codes 0x38 (1.0) and 0x39 (1.125) -> 0x38; of 0x39 and 0x3A -> 0x3A
    assert e4m3_encode_nonneg(np.array([1.0625]))[0] == 0x38
    assert e4m3_encode_nonneg(np.array([1.1875]))[0] == 0x3A
    # below half the smallest subnormal (2^-9) -> 0; exactly half -> 0 (even)
    assert e4m3_encode_nonneg(np.array([2.0 ** -10]))[0] == 0
    assert e4m3_encode_nonneg(np.array([2.0 ** -10 * 1.0001]))[0] == 1


def test_e2m1_encoder_matches_brute_force_on_all_bf16_magnitudes():
    # every non-negative finite bf16 pattern as the scaled value v
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    v = bf16_to_f32(bits).astype(np.float64)
    ours = e2m1_encode_magnitude(v)
    # above 6 the nearest magnitude is 6 (index 7) by monotonicity; the float64
    # distances below are exact only for moderate v, so brute-force those
    assert (ours[v > 6] == 7).all()
    small = v <= 2.0 ** 20
    v, ours = v[small], ours[small]
    # brute force: distance to all 8 magnitudes, ties to the even index
    d = np.abs(v[:, None] - E2M1_MAGNITUDES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    ref = np.where(cand[:, ::2].any(axis=1),
                   2 * np.argmax(cand[:, ::2], axis=1),
                   2 * np.argmax(cand[:, 1::2], axis=1) + 1)
    assert (ours == ref).all()
    # and the exact-rational scan on a subsample
    for i in range(0, v.size, 97):
        assert loops.nearest_code(Fraction(float(v[i])), loops.E2M1_POS) == ours[i]


def test_e2m1_thresholds_follow_ties_to_even():
    v = np.array([0.25, 0.2500001, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.0001, 6.0, 1e9, np.inf])
    assert e2m1_encode_magnitude(v).tolist() == [0, 1, 2, 2, 4, 4, 6, 6, 7, 7, 7, 7]


def test_bf16_decode_encode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(bits)
    fin = np.isfinite(f)
    back = bf16_from_f64(f[fin].astype(np.float64))
    assert (back == bits[fin]).all()
    # torch's own bf16 view is an independent decoder
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (ref == f) | (np.isnan(ref) & np.isnan(f))
    assert same.all()


def test_bf16_rounding_single_step_from_f64():
    # values just above a bf16 midpoint in float64 that a float32 detour would
    # round onto the midpoint (double rounding) must round up
    one = 1.0
    half_ulp = 2.0 ** -8
    x = one + half_ulp + 2.0 ** -40
    assert bf16_from_f64(np.array([x]))[0] == 0x3F81
    assert bf16_from_f64(np.array([one + half_ulp]))[0] == 0x3F80      # tie -> even
    assert bf16_from_f64(np.array([one + 3 * half_ulp]))[0] == 0x3F82  # tie -> even
    # against torch's float32 -> bf16 cast on random float32 values (exact in f64)
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16_from_f64(f.astype(np.float64)) == ref).all()
    # and the exact-rational twin
    for x in f[:300]:
        assert loops.bf16_bits(loops.bf16(Fraction(float(x)))) == bf16_from_f64(np.array([x], np.float64))[0]


@pytest.mark.parametrize("x", [1e-3, 3.0, 1234.5, 2.0 ** -140, 1.7e38])
def test_f32_rounding_twin_agrees_with_numpy(x):
    a = np.float32(x)
    for d in (np.float32(2688.0), np.float32(7.0), np.float32(0.3)):
        assert loops.f32(Fraction(float(a)) / Fraction(float(d))) == float(a / d)
