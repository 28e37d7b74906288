"""GPU block-scaled GEMM (nvfp4_gemm) against the oracle's fp64 GEMM."""
import numpy as np
import pytest

import workloads as W
from conftest import to_dev, to_host
from helpers import check_bf16_output
from oracle.formats import bf16_from_f64
from oracle.gemm import gemm as ref_gemm
from oracle.quantize import quantize_bf16, quantize_weight_bf16

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed, a_std=3.0):
    rng = np.random.default_rng(seed)
    a = bf16_from_f64(rng.standard_normal((M, K)) * a_std)
    b = bf16_from_f64(rng.standard_normal((K, N)) * 0.02)
    aq, asf, ags = quantize_bf16(a)
    bq, bsf, balpha = quantize_weight_bf16(b)
    return aq, asf, np.float32(ags), bq, bsf, np.float32(balpha)


def _run(nv, aq, asf, ags, bq, bsf, balpha):
    # canonical B (K/2, N) -> the packed (N, K/2) layout, on the device
    bq_t, bsf_t = nv.prepack_weights(to_dev(bq)[None], to_dev(bsf)[None])
    out = nv.gemm(to_dev(aq), to_dev(asf), to_dev(np.array([ags], np.float32)), bq_t[0],
                  bsf_t[0], to_dev(np.array([balpha], np.float32)))
    return to_host(out)


# K not a multiple of 128 (144, 208, 80, 16, 7168 + 16): the A rows' f16 form
# and the packed weights are padded with zeros to whole 128-element steps. Shapes
# whose 256-row tiles would fill less than half the GPU run 128-row tiles
# (with K chunks, or, at 1280 x 6144, 240 tiles and no chunks)
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 32, 384), (17, 272, 640), (256, 256, 256),
                                   (300, 512, 1024), (257, 48, 7168), (64, 6144, 128),
                                   (513, 784, 896), (160, 256, 512), (100, 512, 256),
                                   (420, 384, 1024), (5, 48, 144), (33, 272, 7184),
                                   (300, 256, 16), (64, 96, 80), (17, 64, 208), (2048, 512, 256),
                                   (64, 256, 32768), (8, 16, 65536 + 16), (1280, 6144, 1024)])
def test_gemm_random(nv, M, N, K):
    ops = _operands(M, N, K, seed=M + N + K)
    out = _run(nv, *ops)
    ref = ref_gemm(*ops)
    st = check_bf16_output(out, ref, f"gemm {M}x{N}x{K}")
    assert st["cos"] >= 0.9999


def test_gemm_dense_config(nv):
    # the dense config: A 256 x 7168 from bf16 N(0,1)*3, B 7168 x 6144 from N(0,0.02)
    a, b = W.dense_gemm_inputs(W.DENSE)
    aq, asf, ags = quantize_bf16(a)
    bq, bsf, balpha = quantize_weight_bf16(b)
    ops = (aq, asf, np.float32(ags), bq, bsf, np.float32(balpha))
    out = _run(nv, *ops)
    ref = ref_gemm(*ops)
    st = check_bf16_output(out, ref, "dense config")
    print("dense config", st)
    assert st["cos"] >= 0.9999


def test_gemm_constant_scale_bit_exact(nv):
    # all scale bytes 1.0 and small K: float32 sums are exact, so the GPU must
    # equal the correctly rounded oracle bit for bit (src commit log,
    # constant-scale test)
    rng = np.random.default_rng(1)
    M, N, K = 40, 64, 128
    aq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    bq = rng.integers(0, 256, (K // 2, N)).astype(np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    bsf = np.full((K // 16, N), 0x38, np.uint8)
    ops = (aq, asf, np.float32(1.0), bq, bsf, np.float32(1.0))
    out = _run(nv, *ops)
    assert (out == bf16_from_f64(ref_gemm(*ops))).all()


def test_gemm_single_scale_probes(nv):
    # src commit log: SFA[0,0] = 2.0 moved row 0 but SFA[0,3] = 2.0 did not.
    # Here every K-group of an A row and of a B column is probed: the change
    # lands on its own row (column) only and matches the oracle.
    rng = np.random.default_rng(2)
    M, N, K = 20, 48, 256
    aq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    bq = rng.integers(0, 256, (K // 2, N)).astype(np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    bsf = np.full((K // 16, N), 0x38, np.uint8)
    base = _run(nv, aq, asf, np.float32(1.0), bq, bsf, np.float32(1.0))
    for g in range(K // 16):
        m = g % M
        asf2 = asf.copy()
        asf2[m, g] = 0x40
        out = _run(nv, aq, asf2, np.float32(1.0), bq, bsf, np.float32(1.0))
        others = np.arange(M) != m
        assert (out[others] == base[others]).all(), f"A group {g} leaked into other rows"
        assert (out[m] == bf16_from_f64(ref_gemm(aq, asf2, 1.0, bq, bsf, 1.0)[m])).all()
        n = (5 * g) % N
        bsf2 = bsf.copy()
        bsf2[g, n] = 0x40
        out = _run(nv, aq, asf, np.float32(1.0), bq, bsf2, np.float32(1.0))
        oc = np.arange(N) != n
        assert (out[:, oc] == base[:, oc]).all(), f"B group {g} leaked into other columns"
        assert (out[:, n] == bf16_from_f64(ref_gemm(aq, asf, 1.0, bq, bsf2, 1.0)[:, n])).all()


def test_gemm_one_hot_k_probes_at_real_shape(nv):
    # NVFP4 MegaMoE Debug Log Hypothesis 8: the probes passed at test shapes but the real shape
    # M=1, N=6144, K=7168 was never probed. One-hot A rows read single K rows of
    # deq(B) (checks B's nibble order independently of A's) at that shape.
    rng = np.random.default_rng(3)
    K, N = 7168, 6144
    ks = [0, 1, 15, 16, 17, 127, 128, 129, 3583, 3584, 7167]
    M = len(ks)
    aq = np.zeros((M, K // 2), np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    for m, k in enumerate(ks):
        aq[m, k // 2] = 0x2 << (4 * (k % 2))
    b = bf16_from_f64(rng.standard_normal((K, N)) * 0.02)
    bq, bsf, balpha = quantize_weight_bf16(b)
    out = _run(nv, aq, asf, np.float32(1.0), bq, bsf, np.float32(1.0))
    ref = ref_gemm(aq, asf, 1.0, bq, bsf, 1.0)
    assert (out == bf16_from_f64(ref)).all()
