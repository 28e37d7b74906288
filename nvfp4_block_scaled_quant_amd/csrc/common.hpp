// Device-side building blocks shared by the NVFP4 kernels (gfx950 only).
//
// Number formats follow the "nvfp4-megamoe-kernel" pages: E2M1 nibbles are
// sign-magnitude (bit 3 sign, bits 2:0 index {0,.5,1,1.5,2,3,4,6}), two per
// byte with the even element low; scale bytes are OCP E4M3FN bit patterns
// (bias 7, max 448) per 16 elements (NVFP4 MegaMoE Debug Log Hypothesis 5/6, src commit log
// quantizer and `.view` fixes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kSixTimesE4M3Max = 2688.0f;   // 6 * 448, exact

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two float32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one hardware conversion on gfx950 (finite inputs give the same bits as
// f32_to_bf16_rne).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// float64 -> bf16 bits, nearest-even, in effect one rounding: rounding to
// float32 toward zero and setting the last bit when inexact (round to odd)
// keeps enough information for the second rounding to be exact.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
    const float t = __double2float_rz(v);
    uint32_t tb = __float_as_uint(t);
    if ((double)t != v) tb |= 1u;
    return f32_to_bf16_rne(__uint_as_float(tb));
}

// e^x in float64 (Cody-Waite reduction x = n ln2 + r, |r| <= ln2/2, with ln2
// split into a 32-bit head, so n * head is exact, and a tail; e^r from its
// Taylor series to degree 13, truncation below 2^-60 relative; then 2^n).
// About one ulp; inputs are clamped to [-800, 800], where the result is
// already 0 or infinity.
__device__ __forceinline__ double exp_f64(double x) {
    x = fmin(fmax(x, -800.0), 800.0);
    const double n = __builtin_rint(x * 1.4426950408889634);
    double r = __builtin_fma(-n, 0.6931471803691238, x);
    r = __builtin_fma(-n, 1.9082149292705877e-10, r);
    double p = 1.6059043836821613e-10;
    p = __builtin_fma(p, r, 2.08767569878681e-09);
    p = __builtin_fma(p, r, 2.505210838544172e-08);
    p = __builtin_fma(p, r, 2.755731922398589e-07);
    p = __builtin_fma(p, r, 2.7557319223985893e-06);
    p = __builtin_fma(p, r, 2.48015873015873e-05);
    p = __builtin_fma(p, r, 0.0001984126984126984);
    p = __builtin_fma(p, r, 0.001388888888888889);
    p = __builtin_fma(p, r, 0.008333333333333333);
    p = __builtin_fma(p, r, 0.041666666666666664);
    p = __builtin_fma(p, r, 0.16666666666666666);
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    return __builtin_ldexp(p, (int)n);
}

// e^x, accurate for x <= 87 (the result stays a normal float: e^87 < 2^126):
// the hardware base-2 exponential (1 ulp) of t = x log2(e) rounded to float,
// times 1 + r, r = (x log2(e) - t) ln 2. The residual x log2(e) - t is the
// exact rounding error of the product (one fma) plus x times the tail of
// log2(e); |r| < 2^-17, so its own rounding is far below an ulp of the result.
// Larger x give values at the top of the float range or +inf (beyond about
// 88.7); the callers send those gates to float64.
__device__ __forceinline__ float exp_split(float x) {
    const float t = x * 1.44269502f;                                           // log2(e), head
    const float r = __builtin_fmaf(__builtin_fmaf(x, 1.44269502f, -t), 0.693147182f,
                                   x * (1.925963e-8f * 0.693147182f));         // tail of log2(e), times ln 2
    const float p = __builtin_amdgcn_exp2f(t);
    return __builtin_fmaf(p, r, p);
}

// Whether the float32 value v of silu(g) * u (below) decides the correctly
// rounded bf16 result: g >= -87, v normal, and the 16 bits of v below bf16
// precision more than 16 from the rounding midpoint 0x8000, i.e.
// (low - 0x8000 + 16) mod 2^16 > 32. (v is within 5 ulps of the exact value
// by the error analysis below; measured on every finite bf16 gate from -87 up
// with eight u values: at most 2.66 ulps.)
__device__ __forceinline__ bool silu_f32_decides(float g, float v) {
    const uint32_t m = (__float_as_uint(v) + 0x8010u) & 0xFFFFu;
    return (g >= -87.0f) & __builtin_isnormal(v) & (m > 32u);
}

// float32 evaluation of silu(g) * u.
__device__ __forceinline__ float silu_mul_value(float g, float u) {
    // silu(g) = g / (1 + e^-g) for every g >= -87: e^-g <= e^87 is finite and
    // the reciprocal of 1 + e^-g (>= 1.6e-38) is still a normal float, so one
    // formula serves both signs. Error: the exponential about 2 ulps, the sum
    // half an ulp, the hardware reciprocal 1 ulp, the two products half an ulp
    // each: under 5 ulps, well inside the 16-ulp margin of silu_f32_decides.
    // Below g = -87 (and for non-finite g) v is wrong, zero or NaN, and those
    // gates always go to float64.
    const float e = exp_split(-g);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// The same value and whether it decides the correctly rounded bf16 result.
__device__ __forceinline__ float silu_mul_f32(float g, float u, bool& ok) {
    const float v = silu_mul_value(g, u);
    ok = silu_f32_decides(g, v);
    return v;
}

// The lanes of the wave whose (g, v) silu_f32_decides rejects, as a mask:
// one ballot per condition, so each is the compare's own lane mask. "v not
// normal" is one class test for the classes NaN (signaling 1, quiet 2),
// -inf (4), -subnormal (16), -0 (32), +0 (64), +subnormal (128), +inf (512).
// (The class test is written as the compare instruction itself: a ballot of
// __builtin_amdgcn_classf is lowered through a select and a second compare.)
__device__ __forceinline__ uint64_t silu_f32_redo_lanes(float g, float v) {
    const uint32_t m = (__float_as_uint(v) + 0x8010u) & 0xFFFFu;
    uint64_t not_normal;
    asm("v_cmp_class_f32_e64 %0, %1, %2" : "=s"(not_normal) : "v"(v), "s"(759u));
    return __builtin_amdgcn_ballot_w64(!(g >= -87.0f)) | not_normal | __builtin_amdgcn_ballot_w64(m <= 32u);
}

// The float64 evaluation. Where 1 + e^-g rounds to 1 (g above about 36.7)
// the float64 value is the plain product g * u (16 significant bits at most,
// exact), while the exact value is smaller in magnitude by a factor within
// 2^-53 of 1: a product that is a bf16 rounding midpoint must then round
// toward zero, so the value is first moved one float64 step toward zero (no
// other rounding boundary lies that close to a 16-bit product).
__device__ __forceinline__ uint32_t silu_mul_bf16_f64(float g, float u) {
    const double gd = g, ud = u;
    const double den = 1.0 + exp_f64(-gd);
    double v = (gd / den) * ud;
    if (den == 1.0 && v != 0.0 && __builtin_isfinite(v))
        v = __longlong_as_double(__double_as_longlong(v) - 1);
    return f64_to_bf16_rne(v);
}

// act = bf16(silu(g) * u) for bf16-valued g, u (the L1 epilogue), with
// silu(z) = z / (1 + e^-z), correctly rounded from the exact value.
// A float32 evaluation (relative error a few ulps) decides the rounding when
// it is far from a bf16 rounding midpoint; otherwise, and for g < -87 where
// e^g leaves the float32 normal range, the product is recomputed in float64
// (above). (Large gates make silu(g) * u the exact product g * u up to a tiny
// factor; about 1 in 256 of those products is a bf16 midpoint, which float32
// alone would round the wrong way.)
__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
    bool ok;
    const float v = silu_mul_f32(g, u, ok);
    if (__builtin_expect(ok, 1)) return f32_to_bf16_rne(v);
    return silu_mul_bf16_f64(g, u);
}

// Two of them as one packed pair (first in the low half): the float32 results
// are rounded together by the hardware pair conversion (nearest-even, the same
// rounding for normal values), and each element that float32 cannot decide is
// replaced by its float64 result (a branch per element, taken only by waves
// with such an element).
__device__ __forceinline__ uint32_t silu_mul_bf16x2(float g0, float u0, float g1, float u1) {
    bool ok0, ok1;
    const float v0 = silu_mul_f32(g0, u0, ok0);
    const float v1 = silu_mul_f32(g1, u1, ok1);
    uint32_t r = pack_bf16x2_rne(v0, v1);
    if (__builtin_expect(!ok0, 0)) r = (r & 0xFFFF0000u) | silu_mul_bf16_f64(g0, u0);
    if (__builtin_expect(!ok1, 0)) r = (r & 0xFFFFu) | (silu_mul_bf16_f64(g1, u1) << 16);
    return r;
}

// ---------------------------------------------------------------------------
// NVFP4 quantization arithmetic. Every operation is one IEEE float32 operation
// with round-to-nearest-even; divisions are the correctly rounded ones (the
// library is built with -fhip-fp32-correctly-rounded-divide-sqrt and
// -ffp-contract=off).
// ---------------------------------------------------------------------------
struct QuantScales {
    float gs;       // amax / 2688
    float six_gs;   // 6 * gs
};

__device__ __forceinline__ QuantScales make_scales(float amax) {
    QuantScales s;
    s.gs = amax / kSixTimesE4M3Max;
    s.six_gs = 6.0f * s.gs;
    return s;
}

// A global scale given by the caller (static activation scale): the rest of
// the rule is unchanged, so blocks beyond 6 * 448 * gs saturate (scale 448,
// magnitude 6).
__device__ __forceinline__ QuantScales scales_from_gs(float gs) {
    QuantScales s;
    s.gs = gs;
    s.six_gs = 6.0f * gs;
    return s;
}

// E4M3FN code nearest to s in [0, 448], ties to the even code.
// Subnormal range (s < 2^-6): spacing 2^-9, code = rint(s * 2^9).
// Normal range: with e = floor(log2 s) in [-6, 8], r = rint(s * 2^(3-e)) in
// [8, 16] and code = (e + 6) * 8 + r; r = 16 carries into the next binade.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    if (s < 0.015625f) {
        return (uint32_t)__builtin_rintf(s * 512.0f);
    }
    const int e = (int)((__float_as_uint(s) >> 23) & 0xFF) - 127;
    const float scaled = s * __uint_as_float((uint32_t)(127 + 3 - e) << 23);
    const uint32_t r = (uint32_t)__builtin_rintf(scaled);
    return (uint32_t)((e + 6) << 3) + r;
}

// E4M3FN code (0x00..0x7E) -> float32 value, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}

// Quantize one 16-element block given as 16 bf16 bit patterns in 8 words
// (element 2i in the low half of word i). Writes 8 packed bytes (2 words) and
// returns the scale byte.
__device__ __forceinline__ uint32_t quantize_block16(const uint32_t (&w)[8], const QuantScales& qs,
                                                     uint32_t (&packed)[2]) {
    uint32_t bmax_bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        bmax_bits = max(bmax_bits, max(lo, hi));
    }
    const float bmax = bf16_to_f32(bmax_bits);
    float s = 0.0f;
    if (qs.gs > 0.0f) {
        s = bmax / qs.six_gs;
        s = fminf(s, 448.0f);
    }
    const uint32_t code = e4m3_encode(s);
    const float den = e4m3_decode(code) * qs.gs;
    // v = fl32(|x| / den), the IEEE float32 quotient, formed as
    // fl32(fl64(|x| * r)) with r = fl64(1 / den) computed once per block.
    // Exact: the quotient of two floats is never a float32 rounding midpoint
    // and lies at least 2^-49 (relative) from one, while the float64 product
    // is within 2^-52 of it, so both round to the same float32 (normal
    // results; a subnormal quotient is far below the first E2M1 threshold
    // either way, and an overflowing one is infinite either way).
    const double rden = den > 0.0f ? 1.0 / (double)den : 0.0;
    // Magnitudes: the hardware float32 -> FP4 pair conversion of |x| / den
    // (scale 1). It rounds to the nearest of {0,.5,1,1.5,2,3,4,6} with ties to
    // the even code (the midpoints 0.25, 0.75, ..., 5 go to codes 0, 2, 2, 4,
    // 4, 6, 6) and saturates above 6: exactly the E2M1 rule (verified
    // bit-exact against the oracle on every bf16 pattern, at several scales). It writes the pair
    // (element 2i low, 2i + 1 high) into byte i % 4 of word i / 4. den == 0
    // gives rden = 0, v = 0 and magnitude 0. The sign bits are then copied
    // from the elements (bit 15 of each bf16) to bit 3 of each nibble.
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = (float)((double)bf16_to_f32(w[i] & 0x7FFFu) * rden);
        v[2 * i + 1] = (float)((double)bf16_to_f32((w[i] >> 16) & 0x7FFFu) * rden);
    }
    uint32_t p0 = 0, p1 = 0;   // the byte selector must be a literal
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, v[0], v[1], 1.0f, 0);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, v[2], v[3], 1.0f, 1);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, v[4], v[5], 1.0f, 2);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, v[6], v[7], 1.0f, 3);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, v[8], v[9], 1.0f, 0);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, v[10], v[11], 1.0f, 1);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, v[12], v[13], 1.0f, 2);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, v[14], v[15], 1.0f, 3);
    packed[0] = p0;
    packed[1] = p1;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        packed[i >> 2] |= (((w[i] >> 12) & 0x8u) | ((w[i] >> 24) & 0x80u)) << (8 * (i & 3));
    return code;
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// Byte transpose of a 4x4 block held in 4 words: in r[i] byte j = M[i][j];
// out c[j] byte i = M[i][j].
__device__ __forceinline__ void transpose4x4(const uint32_t (&r)[4], uint32_t (&c)[4]) {
    const uint32_t t01lo = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
    const uint32_t t01hi = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
    const uint32_t t23lo = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
    const uint32_t t23hi = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
    c[0] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);
    c[1] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);
    c[2] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
    c[3] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);
}

// ---------------------------------------------------------------------------
// Dequantization for the MFMA operands.
// The FP4 -> f16 conversion applies only the exponent of its float scale, so
// it is given 2^8, and the E4M3 scale enters as an f16 multiply: shifting an
// E4M3 byte left by 7 gives the f16 bit pattern of e4m3 * 2^-8 (bias 7 vs 15,
// the subnormal ranges line up). Every product e2m1 * e4m3 has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in f16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2_t scale_pair(uint32_t code) {
    const uint32_t b = code << 7;
    return __builtin_bit_cast(half2_t, b | (b << 16));
}

// 8 nibbles of `word` (element i in bits 4i..4i+3) -> 8 f16 values * scale.
__device__ __forceinline__ half8_t dequant8(uint32_t word, half2_t sp) {
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 0) * sp;
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 1) * sp;
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 2) * sp;
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 256.0f, 3) * sp;
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// The exact f16 values of one quantized 16-element block (8 packed bytes in
// two words, its scale byte) to 32 bytes at dst (16-byte aligned).
__device__ __forceinline__ void store_block_f16(uint8_t* __restrict__ dst, uint32_t p0, uint32_t p1,
                                                uint32_t code) {
    const half2_t sp = scale_pair(code);
    half8_t* d = reinterpret_cast<half8_t*>(dst);
    d[0] = dequant8(p0, sp);
    d[1] = dequant8(p1, sp);
}

// Block b of a row-major (rows, K) bf16 matrix (groups = K / 16 blocks per
// row) whose 16 elements v0, v1 (8 bf16 pairs) are already loaded: quantize
// it and store the packed bytes and scale (rows of pitch ldq / ldsf) and,
// when h is not null, its exact f16 values (rows of pitch_h(K) = 4 * ldq
// bytes). Each row's padding up to the pitches is written as zeros by the
// thread of its last block, so that a GEMM reading whole K steps sees zero
// data and scales there.
__device__ __forceinline__ void quantize_row_block_loaded(u32x4 v0, u32x4 v1, int64_t b,
                                                          int64_t groups, const QuantScales& qs,
                                                          uint8_t* __restrict__ q, int64_t ldq,
                                                          uint8_t* __restrict__ sf, int64_t ldsf,
                                                          uint8_t* __restrict__ h) {
    const uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    uint32_t packed[2];
    const uint32_t code = quantize_block16(w, qs, packed);
    u32x2 out;
    out[0] = packed[0];
    out[1] = packed[1];
    const int64_t r = b / groups, g = b - r * groups;
    *reinterpret_cast<u32x2*>(q + r * ldq + g * 8) = out;
    sf[r * ldsf + g] = (uint8_t)code;
    const int64_t ldh = 4 * ldq;
    if (h) store_block_f16(h + r * ldh + g * 32, packed[0], packed[1], code);
    if (g == groups - 1) {
        for (int64_t j = groups * 8; j < ldq; j += 8) *reinterpret_cast<u32x2*>(q + r * ldq + j) = (u32x2){0u, 0u};
        for (int64_t j = groups; j < ldsf; ++j) sf[r * ldsf + j] = 0;
        if (h)
            for (int64_t j = groups * 32; j < ldh; j += 16)
                *reinterpret_cast<u32x4*>(h + r * ldh + j) = (u32x4){0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void quantize_row_block(const uint16_t* __restrict__ x, int64_t b,
                                                   int64_t groups, const QuantScales& qs,
                                                   uint8_t* __restrict__ q, int64_t ldq,
                                                   uint8_t* __restrict__ sf, int64_t ldsf,
                                                   uint8_t* __restrict__ h) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 16);
    quantize_row_block_loaded(src[0], src[1], b, groups, qs, q, ldq, sf, ldsf, h);
}

}  // namespace nvfp4
