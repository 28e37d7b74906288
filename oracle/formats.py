"""Number formats of NVFP4, written from their definitions (test infrastructure).

* bfloat16: IEEE-754 binary32 with the low 16 fraction bits dropped (8
  significant bits, 8 exponent bits, bias 127).
* E4M3FN (OCP FP8): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, NaN at S.1111.111, largest finite 448. The pages' global scale
  amax/(6*448) names this 448 (NVFP4 MegaMoE Debug Log, later revision, "input_scale red herring";
  NVFP4 MegaMoE Debug Log, Hypothesis 6 step 2). Scale bytes are bit patterns of this format:
  a stored byte is reinterpreted, never converted by value (src commit log,
  fix of the E4M3 unpack that used `.to` where `.view` was needed).
* E2M1 (FP4): sign-magnitude nibble, bit 3 the sign, bits 2:0 an index into the
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} (src commit log, quantizer fix items
  1 and 3).

Rounding is round-to-nearest with ties to the even code everywhere; the pages
only say "nearest", and this is the IEEE default.

Parity pins: tests/test_oracle_formats.py (all 256 E4M3 bytes against torch's
float8_e4m3fn reinterpretation, a dense sweep of the encoder against torch's
conversion, all 65,536 bf16 patterns through the decoder and encoder, the E2M1
encoder against brute-force nearest search).
"""
import math

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_to_f32(bits):
    """Decode bf16 bit patterns (uint16) to float32, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_from_f64(x):
    """Round float64 values to bf16 bit patterns, nearest-even, in one step.

    Rounding straight from the float64 value (rather than through float32)
    avoids double rounding. Normal bf16 numbers keep 8 significant bits; below
    2**-126 the spacing is fixed at 2**-133 (subnormals); magnitudes that round
    above the largest finite value become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = m * 2**e, m in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.rint(np.ldexp(a, -ulp_exp))   # exact scaling, then ties-to-even
        r = np.ldexp(q, ulp_exp)
    r = np.where(r > BF16_MAX, np.inf, r)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = bits | (sign.astype(np.uint16) << np.uint16(15))
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ----------------------------------------------------------------------------
# E4M3FN
# ----------------------------------------------------------------------------

def _e4m3_value(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
_E4M3_NONNEG = E4M3_TABLE[:127]              # codes 0x00..0x7E, ascending


def e4m3_decode(codes):
    """Value of each E4M3FN byte (bit reinterpretation), as float64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_nonneg(v):
    """Nearest E4M3FN code (ties to the even code) of values in [0, 448]."""
    v = np.asarray(v, dtype=np.float64)
    if v.size and (np.isnan(v).any() or v.min() < 0 or v.max() > E4M3_MAX):
        raise ValueError("e4m3_encode_nonneg expects values in [0, 448]")
    hi = np.minimum(np.searchsorted(_E4M3_NONNEG, v, side="left"), 126)
    lo = np.maximum(hi - 1, 0)
    dlo = v - _E4M3_NONNEG[lo]
    dhi = _E4M3_NONNEG[hi] - v
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)


# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([E2M1_MAGNITUDES, -E2M1_MAGNITUDES])   # index = nibble


def e2m1_decode(nibbles):
    """Value of each E2M1 nibble (0..15): bit 3 sign, bits 2:0 magnitude index."""
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def e2m1_encode_magnitude(v):
    """Magnitude index (0..7) of the E2M1 value nearest to v >= 0.

    Ties go to the even index; values above 6 saturate to 6 (index 7), which is
    also the nearest representable value.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.size and (np.isnan(v).any() or v.min() < 0):
        raise ValueError("e2m1_encode_magnitude expects non-negative values")
    hi = np.minimum(np.searchsorted(E2M1_MAGNITUDES, v, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    dlo = v - E2M1_MAGNITUDES[lo]
    dhi = E2M1_MAGNITUDES[hi] - v
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)
