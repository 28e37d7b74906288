"""Pins of the oracle's block-scaled GEMM (O-G): probes the pages describe,
exact brute force on tiny shapes, and the constant-scale case."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import loops
from oracle.formats import e2m1_decode, e4m3_decode
from oracle.gemm import gemm
from oracle.quantize import dequantize_cols, dequantize_rows, unpack_nibbles

ONE = 0x38          # E4M3 code of 1.0
NIB_ONE = 0x2       # E2M1 code of 1.0


def _rand_operands(rng, M, N, K, scale_codes=None):
    aq = rng.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
    bq = rng.integers(0, 256, size=(K // 2, N)).astype(np.uint8)
    codes = np.arange(0, 127) if scale_codes is None else np.asarray(scale_codes)
    asf = rng.choice(codes, size=(M, K // 16)).astype(np.uint8)
    bsf = rng.choice(codes, size=(K // 16, N)).astype(np.uint8)
    return aq, asf, bq, bsf


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 32), (16, 16, 64), (7, 2, 48)])
def test_brute_force_exact_tiny(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    aq, asf, bq, bsf = _rand_operands(rng, M, N, K)
    a_gs, b_alpha = np.float32(1.7e-3), np.float32(3.1e-5)
    ours = gemm(aq, asf, a_gs, bq, bsf, b_alpha)
    exact = loops.gemm(aq.tolist(), asf.tolist(), float(a_gs), bq.tolist(), bsf.tolist(),
                       float(b_alpha), M, N, K)
    ex = np.array([[float(v) for v in r] for r in exact])
    # magnitude bound for the float64 summation's own rounding
    absum = (np.abs(dequantize_rows(aq, asf)) @ np.abs(dequantize_cols(bq, bsf))
             * float(a_gs) * float(b_alpha))
    assert (np.abs(ours - ex) <= absum * 2.0 ** -50).all()


def test_brute_force_equal_exponent_scales_bit_exact():
    # scales confined to one binade keep every float64 partial sum exact
    rng = np.random.default_rng(5)
    M, N, K = 9, 11, 64
    aq, asf, bq, bsf = _rand_operands(rng, M, N, K, scale_codes=np.arange(0x38, 0x40))
    ours = gemm(aq, asf, np.float32(1.0), bq, bsf, np.float32(1.0))
    exact = loops.gemm(aq.tolist(), asf.tolist(), 1.0, bq.tolist(), bsf.tolist(), 1.0, M, N, K)
    assert (ours == np.array([[float(v) for v in r] for r in exact])).all()


def test_constant_scale_case():
    # all scale bytes 1.0 (src commit log, constant-scale test): the result is the
    # plain product of the E2M1 values times alpha
    rng = np.random.default_rng(6)
    M, N, K = 5, 7, 96
    aq, _, bq, _ = _rand_operands(rng, M, N, K)
    asf = np.full((M, K // 16), ONE, np.uint8)
    bsf = np.full((K // 16, N), ONE, np.uint8)
    a = e2m1_decode(unpack_nibbles(aq, 1))
    b = e2m1_decode(unpack_nibbles(bq, 0))
    assert (gemm(aq, asf, np.float32(0.5), bq, bsf, np.float32(4.0)) == 2.0 * (a @ b)).all()


@pytest.mark.parametrize("side", ["A", "B"])
def test_single_scale_probe_moves_only_its_row_or_column(side):
    # src commit log, SFA probes: SFA[0,0]=2.0 must move row 0, and so must
    # SFA[0,3]; every K-group g of a row is probed, and the change is exactly
    # alpha * (s' - s) * sum_{k in group g} e2m1(a[m,k]) * deq(B)[k, n]
    rng = np.random.default_rng(7)
    M, N, K = 4, 6, 80
    aq, asf, bq, bsf = _rand_operands(rng, M, N, K, scale_codes=np.arange(0x30, 0x48))
    alpha = np.float32(1.0)
    base = gemm(aq, asf, alpha, bq, bsf, alpha)
    for g in range(K // 16):
        if side == "A":
            m = g % M
            asf2 = asf.copy()
            asf2[m, g] = 0x40                                        # 2.0
            out = gemm(aq, asf2, alpha, bq, bsf, alpha)
            d = e4m3_decode(asf2[m, g]) - e4m3_decode(asf[m, g])
            a_nib = e2m1_decode(unpack_nibbles(aq, 1))[m, 16 * g:16 * g + 16]
            pred = d * a_nib @ dequantize_cols(bq, bsf)[16 * g:16 * g + 16]
            others = np.arange(M) != m
            assert (out[others] == base[others]).all()
            assert np.allclose(out[m] - base[m], pred, rtol=1e-12, atol=1e-12)
            if abs(d) > 0 and np.abs(pred).max() > 0:
                assert np.abs(out[m] - base[m]).max() > 0
        else:
            n = g % N
            bsf2 = bsf.copy()
            bsf2[g, n] = 0x40
            out = gemm(aq, asf, alpha, bq, bsf2, alpha)
            d = e4m3_decode(bsf2[g, n]) - e4m3_decode(bsf[g, n])
            b_nib = e2m1_decode(unpack_nibbles(bq, 0))[16 * g:16 * g + 16, n]
            pred = dequantize_rows(aq, asf)[:, 16 * g:16 * g + 16] @ (d * b_nib)
            others = np.arange(N) != n
            assert (out[:, others] == base[:, others]).all()
            assert np.allclose(out[:, n] - base[:, n], pred, rtol=1e-12, atol=1e-12)


def test_one_hot_k_probes_read_single_b_rows():
    # one-hot A rows: row m has a single 1.0 at k = 16 g + i, so C[m] is exactly
    # alpha * deq(B)[k] (K-group g <-> k in [16g, 16g+16); the B nibble order is
    # checked independently of A's)
    rng = np.random.default_rng(8)
    K, N = 64, 10
    ks = [0, 1, 15, 16, 17, 31, 32, 47, 48, 63]
    M = len(ks)
    aq = np.zeros((M, K // 2), np.uint8)
    asf = np.full((M, K // 16), ONE, np.uint8)
    for m, k in enumerate(ks):
        aq[m, k // 2] = NIB_ONE << (4 * (k % 2))
    _, _, bq, bsf = _rand_operands(rng, M, N, K)
    out = gemm(aq, asf, np.float32(1.0), bq, bsf, np.float32(1.0))
    b = dequantize_cols(bq, bsf)
    for m, k in enumerate(ks):
        assert (out[m] == b[k]).all()


def test_power_of_two_alpha_scales_exactly():
    rng = np.random.default_rng(9)
    aq, asf, bq, bsf = _rand_operands(rng, 3, 4, 32)
    c1 = gemm(aq, asf, np.float32(0.75), bq, bsf, np.float32(1e-3))
    c2 = gemm(aq, asf, np.float32(1.5), bq, bsf, np.float32(1e-3))
    assert (c2 == 2 * c1).all()
