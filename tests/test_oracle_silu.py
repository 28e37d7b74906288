"""Pin of stage 4's act = bf16(silu(g) * u) (reading: correctly rounded from the
exact value; silu(z) = z / (1 + e^-z)) against brute force at 80 significant
decimal digits (Python's decimal module, which rounds every operation
correctly at that precision).

The oracle evaluates in float64 and rounds once to bf16. That is the correct
rounding wherever the float64 value is not itself a bf16 rounding midpoint; it
is one where 1 + e^-g rounds to 1 (large gates), and there the oracle's rule
sends the midpoint toward zero. The cases below cover that regime
exhaustively (every bf16 gate from 32 to 1024 against every bf16 mantissa of
u), plus random gates of both signs and the range where the result is a bf16
subnormal.
"""
from decimal import Decimal, ROUND_HALF_EVEN, localcontext

import numpy as np

from oracle.formats import bf16_from_f64, bf16_to_f32
from oracle.moe import silu_mul_bf16

TWO = Decimal(2)


def _round_bf16_exact(d, tiny):
    """bf16 bits of the nearest-even rounding of the Decimal d (finite, in
    range), with an assertion that d is not within `tiny` (relative to the
    bf16 spacing) of a midpoint, i.e. the precision used decided it."""
    if d == 0:
        return 0x8000 if d.is_signed() else 0
    neg = d < 0
    a = -d if neg else d
    e = int(np.floor(np.log2(float(a)))) if float(a) > 0 else -200
    # correct the float estimate of floor(log2 a)
    while TWO ** e > a:
        e -= 1
    while TWO ** (e + 1) <= a:
        e += 1
    ulp_exp = max(e - 7, -133)
    scaled = a / TWO ** ulp_exp
    q = scaled.to_integral_value(rounding=ROUND_HALF_EVEN)
    frac = scaled - scaled.to_integral_value(rounding="ROUND_FLOOR")
    assert abs(frac - Decimal("0.5")) > tiny, "precision too low to decide the rounding"
    r = float(q) * 2.0 ** ulp_exp
    bits = int(bf16_from_f64(np.array([r]))[0])
    return bits | (0x8000 if neg else 0)


def _exact_act_bits(g_bits, u_bits):
    out = np.empty(len(g_bits), np.uint16)
    gf = bf16_to_f32(g_bits).astype(np.float64)
    uf = bf16_to_f32(u_bits).astype(np.float64)
    cache = {}
    for i, (g, u) in enumerate(zip(gf, uf)):
        # enough digits that e^-g itself is resolved next to 1 (large gates
        # move the value off g * u by a factor 1 - e^-g), plus 60 more
        prec = 80 + int(max(g, 0.0) / 2.302585)
        with localcontext() as c:
            c.prec = prec
            c.Emin = -10 ** 6
            c.Emax = 10 ** 6
            s = cache.get(g)
            if s is None:
                gd = Decimal(g)
                s = gd / (1 + (-gd).exp())
                cache[g] = s
            out[i] = _round_bf16_exact(s * Decimal(u), Decimal(10) ** (20 - prec))
    return out


def _all_mantissas(sign=0, exp_field=127):
    return np.array([(sign << 15) | (exp_field << 7) | m for m in range(128)], np.uint16)


def test_silu_mul_large_gates_exhaustive():
    # every bf16 gate in [32, 1024): 1 + e^-g rounds to 1 in float64 above
    # about 36.7, so silu(g) * u is g * u up to a factor within 2^-53 of 1,
    # and 1 in 256 of the products is a bf16 midpoint
    g = np.array([(e << 7) | m for e in range(127 + 5, 127 + 10) for m in range(128)], np.uint16)
    u = _all_mantissas()
    gg = np.repeat(g, u.size)
    uu = np.tile(u, g.size)
    # also negative u
    gg = np.concatenate([gg, gg[::7]])
    uu = np.concatenate([uu, uu[::7] | 0x8000])
    want = _exact_act_bits(gg, uu)
    got = silu_mul_bf16(gg, uu)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(bf16_to_f32(gg[i])), float(bf16_to_f32(uu[i])), hex(got[i]), hex(want[i]))
                           for i in bad[:5]]
    # the regime really contains midpoint products (where plain nearest-even
    # of g * u would be wrong)
    prod = bf16_to_f32(gg).astype(np.float64) * bf16_to_f32(uu).astype(np.float64)
    assert (bf16_from_f64(prod) != want).sum() > 100


def test_silu_mul_random_gates():
    rng = np.random.default_rng(11)
    # random finite bf16 gates in [-128, 128] of both signs, eight u each
    mag = rng.uniform(2.0 ** -20, 128.0, 3000) * rng.choice([-1.0, 1.0], 3000)
    g = bf16_from_f64(mag)
    u = bf16_from_f64(rng.standard_normal(3000 * 8) * 4.0)
    gg = np.repeat(g, 8)
    want = _exact_act_bits(gg, u)
    got = silu_mul_bf16(gg, u)
    assert (got == want).all(), np.nonzero(got != want)[0][:5]


def test_silu_mul_tiny_results():
    # gates from -130 to -87: silu(g) * u falls into and below the bf16
    # subnormal range (spacing 2^-133), and rounds to signed zero further down
    g = bf16_from_f64(np.linspace(-130.0, -87.0, 400))
    u = bf16_from_f64(np.array([1.0, -1.5, 3.0, 0.0078125]))
    gg = np.repeat(g, u.size)
    uu = np.tile(u, g.size)
    want = _exact_act_bits(gg, uu)
    got = silu_mul_bf16(gg, uu)
    assert (got == want).all(), np.nonzero(got != want)[0][:5]
    assert (want & 0x7FFF == 0).any() and ((want & 0x7F80) == 0).any()
