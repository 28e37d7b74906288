"""Pure-Python twin of the oracle, in exact rational arithmetic (test infrastructure).

Used only on tiny shapes to pin the vectorized NumPy oracle: the two must agree
bit for bit before any GPU result is compared with the oracle. It restates the
same definitions with independent code: float32 and bf16 rounding are done on
exact fractions with integer round-half-even; the E4M3 and E2M1 values are
computed from their bit fields by formula rather than read from a table; the
nearest-code searches scan every code; GEMM sums are exact integers.

Rounded results are returned as Python floats: every float32 and bf16 value is
exactly a float64, and floats keep the sign of zero, which the quantizer's sign
bit depends on.
"""
import math
from fractions import Fraction

FLT_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)
BF16_MAX_FR = Fraction((2 ** 8 - 1) * 2 ** 120)


def _floor_log2(a):
    """Largest e with 2**e <= a, for a Fraction a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_binary(x, sig_bits, min_exp, max_finite, negative_zero=False):
    """Round an exact rational to a binary format with `sig_bits` significant bits.

    min_exp is the exponent of the subnormal spacing. Ties to even. Returns a
    float (exact); a negative value that rounds to zero gives -0.0, and an
    exact zero gives -0.0 only when `negative_zero` says its sign is negative.
    """
    x = Fraction(x)
    if x == 0:
        return -0.0 if negative_zero else 0.0
    neg = x < 0
    a = -x if neg else x
    ulp_exp = max(_floor_log2(a) - (sig_bits - 1), min_exp)
    q = round(a / Fraction(2) ** ulp_exp)            # round-half-even on Fraction
    r = q * Fraction(2) ** ulp_exp
    val = math.inf if r > max_finite else float(r)
    return -val if neg else val


def f32(x, negative_zero=False):
    return _round_binary(x, 24, -149, FLT_MAX, negative_zero)


def bf16(x, negative_zero=False):
    return _round_binary(x, 8, -133, BF16_MAX_FR, negative_zero)


def bf16_value(bits):
    """Value of a bf16 bit pattern, from its fields (float, signed zero kept)."""
    neg = bool(bits & 0x8000)
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** -126
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    f = float(v)
    return -f if neg else f


def bf16_bits(v):
    """Bit pattern of an exact bf16 value given as a float."""
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a == math.inf:
        return sign | 0x7F80
    if a == 0:
        return sign
    a = Fraction(a)
    if a < Fraction(2) ** -126:
        m = a / Fraction(2) ** -133
        assert m.denominator == 1
        return sign | int(m)
    e = _floor_log2(a)
    m = (a / Fraction(2) ** e - 1) * 128
    assert m.denominator == 1
    return sign | ((e + 127) << 7) | int(m)


def e4m3_value(code):
    """E4M3FN value from its fields: (8*[e>0] + m) * 2**(max(e,1) - 10)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    assert not (e == 15 and m == 7), "NaN code"
    return s * Fraction(8 * (e > 0) + m) * Fraction(2) ** (max(e, 1) - 10)


def e2m1_value(nibble):
    """E2M1 value from its fields: bit 3 sign, bits 2:1 exponent, bit 0 mantissa."""
    s = -1 if nibble & 8 else 1
    e = (nibble >> 1) & 3
    m = nibble & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)


def nearest_code(v, values):
    """Index of the nearest value to v (scan), ties to the even index."""
    best = None
    for i, c in enumerate(values):
        d = abs(v - c)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


E4M3_POS = [e4m3_value(c) for c in range(127)]
E2M1_POS = [e2m1_value(n) for n in range(8)]


def quantize(rows_bits, gs=None):
    """Quantize rows of bf16 bit patterns, blocks of 16 along each row.

    gs: None for the tensor's own global scale fl32(amax / 2688), or a given
    (static) float32 global scale.
    Returns (q rows of bytes, sf rows of bytes, gs as a float).
    """
    ncols = len(rows_bits[0]) if rows_bits else 0
    assert ncols % 16 == 0
    rows = [[bf16_value(b) for b in r] for r in rows_bits]
    if gs is None:
        amax = max((abs(Fraction(v)) for r in rows for v in r), default=Fraction(0))
        gs = f32(amax / 2688)
    six_gs = f32(6 * Fraction(gs))
    q_rows, sf_rows = [], []
    for r in rows:
        sf_row, nibs = [], []
        for b0 in range(0, ncols, 16):
            blk = r[b0:b0 + 16]
            bmax = max(abs(Fraction(v)) for v in blk)
            if gs > 0:
                s = min(Fraction(f32(bmax / Fraction(six_gs))), Fraction(448))
            else:
                s = Fraction(0)
            code = nearest_code(s, E4M3_POS)
            sf_row.append(code)
            den = f32(e4m3_value(code) * Fraction(gs))
            for v in blk:
                if den == 0:
                    mag = 0
                else:
                    w = f32(abs(Fraction(v)) / Fraction(den))
                    mag = 7 if w == math.inf else nearest_code(Fraction(w), E2M1_POS)
                neg = math.copysign(1.0, v) < 0
                nibs.append((8 if neg else 0) | mag)
        q_rows.append([nibs[j] | (nibs[j + 1] << 4) for j in range(0, ncols, 2)])
        sf_rows.append(sf_row)
    return q_rows, sf_rows, gs


def deq_row_value(q_row, sf_row, c):
    """Dequantized element c of a row-packed operand (global scale excluded)."""
    byte = q_row[c // 2]
    nib = (byte >> 4) if c % 2 else (byte & 0xF)
    return e2m1_value(nib) * e4m3_value(sf_row[c // 16])


def deq_col_value(q, sf, k, n):
    """Dequantized element (k, n) of a K-packed (K/2, N) operand."""
    byte = q[k // 2][n]
    nib = (byte >> 4) if k % 2 else (byte & 0xF)
    return e2m1_value(nib) * e4m3_value(sf[k // 16][n])


def gemm(aq, asf, a_gs, bq, bsf, b_alpha, M, N, K):
    """Exact result (Fractions) of the block-scaled GEMM."""
    alpha = Fraction(a_gs) * Fraction(b_alpha)
    a = [[deq_row_value(aq[m], asf[m], k) for k in range(K)] for m in range(M)]
    b = [[deq_col_value(bq, bsf, k, n) for n in range(N)] for k in range(K)]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += a[m][k] * b[k][n]
            row.append(alpha * acc)
        out.append(row)
    return out


def _scaled_ints(vals):
    """Dequantized values are multiples of 2**-10; return them times 2**10."""
    out = []
    for v in vals:
        s = v * 1024
        assert s.denominator == 1
        out.append(int(s))
    return out


def moe_forward(x_bits, topk_ids, topk_weights, w13q, w13sf, w13_alpha,
                w2q, w2sf, w2_alpha):
    """Exact-arithmetic layer (tiny shapes only). Inputs are nested lists.

    Returns dict(y_bits, act_bits {(t, j): [bits]}, aq, asf, gs1, gs2). SiLU's
    exp is the only inexact step (math.exp on float64).
    """
    T = len(x_bits)
    H = len(x_bits[0])
    E = len(w13q)
    I = len(w2q[0]) * 2
    k = len(topk_ids[0])
    xq, xsf, gs1 = quantize(x_bits)
    w13 = [[_scaled_ints([deq_col_value(w13q[e], w13sf[e], kk, n) for n in range(2 * I)])
            for kk in range(H)] for e in range(E)]
    slots = [(t, j) for t in range(T) for j in range(k) if 0 <= topk_ids[t][j] < E]
    act = {}
    for (t, j) in slots:
        e = topk_ids[t][j]
        a = _scaled_ints([deq_row_value(xq[t], xsf[t], c) for c in range(H)])
        alpha = Fraction(gs1) * Fraction(w13_alpha[e]) / (1024 * 1024)
        gu = []
        for n in range(2 * I):
            acc = 0
            for kk in range(H):
                acc += a[kk] * w13[e][kk][n]
            gu.append(bf16(alpha * acc))
        bits = []
        for n in range(I):
            g, u = gu[n], gu[I + n]
            sil = g / (1.0 + math.exp(-g)) if g > -700.0 else -0.0 * g
            if g > 0 and 1.0 + math.exp(-g) == 1.0:
                # e^-g below 2^-53: the exact value g*u / (1 + e^-g) lies
                # strictly between g*u*(1 - 2^-52) and g*u, and no bf16
                # rounding boundary other than g*u itself lies there
                prod = Fraction(g) * Fraction(u) * (1 - Fraction(1, 1 << 60))
            else:
                prod = Fraction(sil) * Fraction(u)
            neg_zero = (math.copysign(1.0, sil) * math.copysign(1.0, u)) < 0
            bits.append(bf16_bits(bf16(prod, negative_zero=neg_zero)))
        act[(t, j)] = bits
    act_rows = [act[s] for s in slots]
    if act_rows:
        aq_rows, asf_rows, gs2 = quantize(act_rows)
    else:
        aq_rows, asf_rows, gs2 = [], [], 0.0
    w2 = [[_scaled_ints([deq_col_value(w2q[e], w2sf[e], kk, n) for n in range(H)])
           for kk in range(I)] for e in range(E)]
    y = [[Fraction(0)] * H for _ in range(T)]
    for i, (t, j) in enumerate(slots):
        e = topk_ids[t][j]
        a = _scaled_ints([deq_row_value(aq_rows[i], asf_rows[i], c) for c in range(I)])
        alpha = Fraction(gs2) * Fraction(w2_alpha[e]) / (1024 * 1024)
        wt = Fraction(topk_weights[t][j])
        for n in range(H):
            acc = 0
            for kk in range(I):
                acc += a[kk] * w2[e][kk][n]
            y[t][n] += wt * alpha * acc
    y_bits = [[bf16_bits(bf16(v)) for v in row] for row in y]
    return {"y_bits": y_bits, "act_bits": act, "gs1": gs1, "gs2": gs2,
            "aq": dict(zip(slots, aq_rows)), "asf": dict(zip(slots, asf_rows))}
