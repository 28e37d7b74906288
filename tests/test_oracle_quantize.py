"""Pins of the oracle's NVFP4 quantizer (O-Q) against what the pages fix."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import loops
from oracle.formats import (bf16_from_f64, bf16_to_f32, e2m1_decode, e4m3_decode)
from oracle.quantize import (dequantize_cols, global_scale,
                             quantize_bf16, quantize_f32, quantize_weight_bf16,
                             unpack_nibbles)


def _bf16(vals):
    return bf16_from_f64(np.asarray(vals, dtype=np.float64))


def _rand_bits(rng, shape, std=3.0):
    return _bf16(rng.standard_normal(shape) * std)


def test_global_scale_pairs_printed_on_pages():
    # NVFP4 MegaMoE Debug Log "Symptoms" (amax 3.86 -> igs 1.4e-3) and the later revision's
    # calibration arithmetic (2.86e-4 * 6 * 448 = 0.77)
    for amax, printed, digits in read_golden("global_scale_pairs.txt"):
        gs = float(global_scale(np.float32(float(amax))))
        assert float(f"{gs:.{int(digits) - 1}e}") == float(printed)


def test_nibble_order_fixture():
    for x0, x1, byte in read_golden("nibble_order.txt"):
        row = np.zeros((1, 16))
        row[0, 0], row[0, 1] = float(x0), float(x1)
        q, sf, gs = quantize_bf16(_bf16(row))
        assert q[0, 0] == int(byte, 16)
        assert sf[0, 0] == 0x7E


def test_amax_block_gets_scale_448_and_amax_element_code_7():
    # closed form: bmax = amax gives s = amax / (6 * amax / 2688) = 448 -> 0x7E,
    # and the amax element is v = amax / (448 gs) = 6 -> magnitude index 7
    rng = np.random.default_rng(11)
    for trial in range(50):
        rows, cols = rng.integers(1, 9), 16 * rng.integers(1, 9)
        x = _rand_bits(rng, (rows, cols), std=10.0 ** rng.uniform(-20, 20))
        q, sf, gs = quantize_bf16(x)
        xf = bf16_to_f32(x)
        r, c = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
        assert sf[r, c // 16] == 0x7E
        nib = unpack_nibbles(q, axis=1)[r, c]
        assert nib & 7 == 7


def test_block_scale_is_block_amax_over_six_gs():
    # each block's scale byte is E4M3(bmax / (6 gs)): the decoded scale is within
    # E4M3's half-spacing of that ratio (relative 2^-4 for normals)
    rng = np.random.default_rng(12)
    x = _rand_bits(rng, (64, 256))
    xf = bf16_to_f32(x).astype(np.float64)
    q, sf, gs = quantize_bf16(x)
    bmax = np.abs(xf).reshape(64, 16, 16).max(-1)
    ratio = bmax / (6.0 * float(gs))
    dec = e4m3_decode(sf)
    assert (np.abs(dec - ratio) <= ratio * 2.0 ** -4 * 1.0001 + 2.0 ** -10).all()


def test_sign_symmetry():
    # Q(-x) = Q(x) with bit 3 of every nibble flipped (the clamp(0,15) bug of the
    # src commit log, quantizer fix item 1, would break this)
    rng = np.random.default_rng(13)
    x = _rand_bits(rng, (17, 320))
    q1, sf1, gs1 = quantize_bf16(x)
    q2, sf2, gs2 = quantize_bf16(x ^ np.uint16(0x8000))
    assert gs1 == gs2 and (sf1 == sf2).all()
    assert (q2 == (q1 ^ 0x88)).all()


def test_power_of_two_invariance():
    # scaling x by 2^j scales gs by 2^j and leaves bytes and scales unchanged
    # (applying the global scale twice, the pages' igs double-count, breaks it)
    rng = np.random.default_rng(14)
    x = bf16_to_f32(_rand_bits(rng, (9, 128)))
    q, sf, gs = quantize_f32(x)
    for j in (-20, -3, 1, 7, 30):
        qj, sfj, gsj = quantize_f32(x * np.float32(2.0 ** j))
        assert (qj == q).all() and (sfj == sf).all()
        assert gsj == np.float32(gs * np.float32(2.0 ** j))


def test_round_trip_bound():
    # |x - sign * e2m1 * s_dec * gs| <= half an E2M1 spacing at the chosen value,
    # in units of den = s_dec * gs (plus one float32 rounding of the division);
    # saturated values (v > 6) are bounded by the E4M3 rounding of the scale.
    rng = np.random.default_rng(15)
    x = _rand_bits(rng, (40, 512))
    xf = bf16_to_f32(x).astype(np.float64)
    q, sf, gs = quantize_bf16(x)
    nib = unpack_nibbles(q, axis=1)
    den = np.repeat(e4m3_decode(sf), 16, axis=1) * float(np.float32(gs))
    rec = e2m1_decode(nib) * den
    v = np.abs(xf) / den
    mag = np.abs(e2m1_decode(nib))
    half_gap = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0))
    half_gap = np.where(v > 6, v - 6, half_gap)
    err = np.abs(xf - rec)
    assert (err <= half_gap * den * (1 + 2.0 ** -22) + np.abs(xf) * 2.0 ** -23).all()
    assert (v <= 6 * (1 + 2.0 ** -4) * (1 + 2.0 ** -20)).all()
    # the amax element reconstructs to 2688 gs, which is amax up to one rounding
    amax = np.abs(xf).max()
    assert abs(6 * 448 * float(gs) - amax) <= amax * 2.0 ** -23


def test_zero_tensor_zero_block_negative_zero():
    x = np.zeros((2, 32), dtype=np.uint16)
    x[1, 5] = 0x8000                      # -0.0
    q, sf, gs = quantize_bf16(x)
    assert gs == 0 and (sf == 0).all()
    nib = unpack_nibbles(q, axis=1)
    assert nib[1, 5] == 8 and nib.sum() == 8
    # a zero block next to a non-zero one: scale 0, magnitudes 0, signs kept
    x = _bf16([[1.0] * 16 + [0.0] * 15 + [-0.0]])
    q, sf, gs = quantize_bf16(x)
    assert sf[0, 1] == 0
    assert unpack_nibbles(q, axis=1)[0, 31] == 8
    # negative values rounding to magnitude 0 keep the sign bit
    x = _bf16([[6.0] + [-0.01] + [0.0] * 14])
    q, _, _ = quantize_bf16(x)
    assert unpack_nibbles(q, axis=1)[0, 1] == 8


def test_vectorized_matches_exact_twin():
    # the pure-Python exact-rational twin on random and adversarial inputs,
    # bit for bit (bytes, scale bytes, global scale bits)
    rng = np.random.default_rng(16)
    cases = [_rand_bits(rng, (3, 48)),
             _rand_bits(rng, (2, 32), std=1e-30),
             _rand_bits(rng, (2, 32), std=1e30),
             _bf16([[6.375, 1.0625, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 0.0, -0.0,
                     3.0, 2.9, 1e-5, -1e-5]]),
             rng.integers(0, 0x7F80, size=(2, 64)).astype(np.uint16)]
    for x in cases:
        q, sf, gs = quantize_bf16(x)
        lq, lsf, lgs = loops.quantize(x.tolist())
        assert (q == np.array(lq, dtype=np.uint8)).all()
        assert (sf == np.array(lsf, dtype=np.uint8)).all()
        assert float(gs) == lgs


def test_e4m3_midpoints_through_the_quantizer_match_twin():
    # a block whose amax is pinned to 2688 makes gs = 1 and 6 gs = 6 exactly, so
    # s = bmax / 6: sweep bmax over many bf16 values to hit E4M3 ties
    bits = np.arange(0x3A00, 0x4500, 7, dtype=np.uint16)     # ~[4.9e-4, 2048)
    n = bits.size
    x = np.zeros((n, 32), dtype=np.uint16)
    x[:, 16] = bits
    x[0, 0] = _bf16([2688.0])[0]
    q, sf, gs = quantize_bf16(x)
    assert gs == np.float32(1.0)
    lq, lsf, lgs = loops.quantize(x[::5].tolist())
    assert (sf[::5] == np.array(lsf)).all() and (q[::5] == np.array(lq)).all()


def test_unpack_is_inverse_of_pack_nonsquare():
    # unpack along K for a (K/2, N) tensor with K/2 != N; the pages' reshape bug
    # (NVFP4 MegaMoE Debug Log, "Weight nibble unpack reshape bug") interleaved along N instead
    rng = np.random.default_rng(17)
    nib = rng.integers(0, 16, size=(12, 5)).astype(np.uint8)     # (K, N)
    packed = nib[0::2] | (nib[1::2] << 4)                        # (K/2, N)
    assert (unpack_nibbles(packed, axis=0) == nib).all()
    nib_r = rng.integers(0, 16, size=(5, 12)).astype(np.uint8)   # (M, K)
    packed_r = nib_r[:, 0::2] | (nib_r[:, 1::2] << 4)
    assert (unpack_nibbles(packed_r, axis=1) == nib_r).all()


def test_weight_rule_blocks_along_k():
    # the weight rule is the activation rule on W transposed: amax over the whole
    # matrix, blocks of 16 consecutive K, byte [kh, n] = W[2kh, n] | W[2kh+1, n] << 4
    rng = np.random.default_rng(18)
    w = _rand_bits(rng, (64, 24), std=0.02)
    q, sf, alpha = quantize_weight_bf16(w)
    assert q.shape == (32, 24) and sf.shape == (4, 24)
    qt, sft, gst = quantize_bf16(np.ascontiguousarray(w.T))
    assert (q == qt.T).all() and (sf == sft.T).all() and alpha == gst
    deq = dequantize_cols(q, sf) * float(alpha)
    wf = bf16_to_f32(w).astype(np.float64)
    assert np.abs(deq - wf).max() <= np.abs(wf).max() * 0.25
    # one element moved to 2x the amax lands in its own (k-block, column) only
    w2 = w.copy()
    w2[37, 5] = _bf16([float(np.abs(wf).max()) * 2])[0]
    q2, sf2, _ = quantize_weight_bf16(w2)
    assert sf2[37 // 16, 5] == 0x7E
