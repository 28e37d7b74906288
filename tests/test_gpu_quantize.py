"""GPU quantizers (nvfp4_quantize, nvfp4_quantize_weights) against the oracle:
bytes, scale bytes and global-scale bits must match exactly."""
import numpy as np
import pytest

import workloads as W
from conftest import to_dev, to_host
from oracle.formats import bf16_from_f64
from oracle.quantize import quantize_bf16, quantize_weight_bf16

pytestmark = pytest.mark.gpu


def _bf16(v):
    return bf16_from_f64(np.asarray(v, np.float64))


def _check_rows(nv, x_bits, label):
    q, sf, gs = nv.quantize(to_dev(x_bits))
    rq, rsf, rgs = quantize_bf16(x_bits)
    q, sf, gs = to_host(q), to_host(sf), to_host(gs)
    assert gs.view(np.uint32)[0] == np.float32(rgs).view(np.uint32), f"{label}: gs"
    bad_sf = np.argwhere(sf != rsf)
    assert bad_sf.size == 0, f"{label}: {len(bad_sf)} scale bytes differ, first {bad_sf[:3]}"
    bad_q = np.argwhere(q != rq)
    assert bad_q.size == 0, f"{label}: {len(bad_q)} packed bytes differ, first {bad_q[:3]}"


@pytest.mark.parametrize("M,K,std", [(1, 16, 3.0), (3, 48, 3.0), (17, 272, 1.0), (32, 256, 3.0),
                                     (256, 7168, 3.0), (1000, 144, 1e-3), (5, 64, 1e30),
                                     (7, 32, 1e-38)])
def test_quantize_random(nv, M, K, std):
    rng = np.random.default_rng(M * 7 + K)
    _check_rows(nv, _bf16(rng.standard_normal((M, K)) * std), f"M{M} K{K} std{std}")


def test_quantize_tiny_and_prefill_recipes(nv):
    _check_rows(nv, W.activations(W.TINY), "tiny x")
    cfg = W.small_layer("p", T=512, H=7168, I=16, E=1, topk=1, seed=40, outlier_frac=1e-3)
    _check_rows(nv, W.activations(cfg), "prefill-recipe x")


def test_quantize_all_bf16_patterns_as_elements(nv):
    # every finite bf16 pattern appears as an element; the amax is pinned so
    # that gs = 1 and scales and nibbles run through every decision boundary
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    fin = (bits & 0x7F80) != 0x7F80
    vals = bits[fin]
    vals = vals[bf16_to_abs(vals) <= 2688.0]
    n = (vals.size + 15) // 16 * 16
    x = np.zeros(n, np.uint16)
    x[:vals.size] = vals
    x = x.reshape(-1, 16)
    x = np.concatenate([x, _bf16([[2688.0] + [0.0] * 15])], axis=0)
    _check_rows(nv, x, "all bf16 patterns")


def bf16_to_abs(bits):
    from oracle.formats import bf16_to_f32
    return np.abs(bf16_to_f32(bits))


def test_quantize_e4m3_tie_sweep(nv):
    # amax pinned to 2688 (gs = 1): block maxima sweep bf16 values so that
    # bmax / 6 lands on every E4M3 midpoint region
    bits = np.arange(0x3000, 0x4528, dtype=np.uint16)
    x = np.zeros((bits.size + 1, 16), np.uint16)
    x[:-1, 3] = bits
    x[:-1, 4] = bits ^ np.uint16(0x8000)
    x[:-1, 5] = (bits >> 1).astype(np.uint16)
    x[-1, 0] = _bf16([2688.0])[0]
    _check_rows(nv, x, "e4m3 tie sweep")


def test_quantize_edge_cases(nv):
    _check_rows(nv, np.zeros((4, 32), np.uint16), "all zero")
    z = np.zeros((2, 32), np.uint16)
    z[1, 7] = 0x8000
    _check_rows(nv, z, "negative zero")
    _check_rows(nv, _bf16([[1.0] * 16 + [0.0] * 15 + [-0.0]]), "zero block")
    _check_rows(nv, _bf16([[6.0, -0.01] + [0.0] * 14]), "negative to zero")
    rng = np.random.default_rng(3)
    tiny = _bf16(rng.standard_normal((3, 64)) * 1e-39)      # bf16 subnormals
    _check_rows(nv, tiny, "subnormal inputs")


def test_quantize_empty(nv):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, sf, gs = nv.quantize(x)
    assert q.shape == (0, 32) and sf.shape == (0, 4)
    assert to_host(gs)[0] == 0.0


@pytest.mark.parametrize("E,K,N", [(1, 16, 16), (3, 64, 48), (2, 272, 40), (4, 256, 256)])
def test_quantize_weights_small(nv, E, K, N):
    rng = np.random.default_rng(E * 100 + K + N)
    w = _bf16(rng.standard_normal((E, K, N)) * 0.02)
    q, sf, alpha = (to_host(t) for t in nv.quantize_weights(to_dev(w)))
    for e in range(E):
        rq, rsf, ra = quantize_weight_bf16(w[e])
        assert (q[e] == rq).all() and (sf[e] == rsf).all()
        assert alpha[e].view(np.uint32) == np.float32(ra).view(np.uint32)


def test_quantize_weights_full_expert(nv):
    # one expert of the layer's real shape: w13 (7168, 6144) and w2 (3072, 7168)
    w13, w2 = W.expert_weights_bf16(W.DECODE, 5)
    for w in (w13, w2):
        q, sf, alpha = (to_host(t) for t in nv.quantize_weights(to_dev(w[None])))
        rq, rsf, ra = quantize_weight_bf16(w)
        assert alpha[0].view(np.uint32) == np.float32(ra).view(np.uint32)
        assert (sf[0] == rsf).all()
        assert (q[0] == rq).all()


def _padded_rows(a, pitch):
    # canonical (E, R, C) -> C rows of `pitch` bytes each, zero padded
    E, R, C = a.shape
    rows = np.zeros((E, C, pitch), np.uint8)
    rows[:, :, :R] = a.transpose(0, 2, 1)
    return rows


def _packed_data(q, ldq):
    # 16-row blocks whose 32-byte half steps are stored together
    E, _, C = q.shape
    return _padded_rows(q, ldq).reshape(E, C // 16, 16, ldq // 32, 32).transpose(0, 1, 3, 2, 4)


def _packed_scales(sf, ldwsf):
    # a row's scale groups g = 32 quad + 8 u + 2 pair + b (step 4 quad + u of
    # the quad, pair of groups, byte) are stored per 16-row block as
    # [quad][row][pair][u][b]
    E, _, C = sf.shape
    rows = _padded_rows(sf, ldwsf).reshape(E, C // 16, 16, ldwsf // 32, 4, 4, 2)
    return rows.transpose(0, 1, 3, 2, 5, 4, 6).reshape(E, C // 16, ldwsf // 32, 16, 32)


@pytest.mark.parametrize("E,K,N", [(1, 16, 16), (3, 272, 48), (2, 256, 208), (1, 7168, 96),
                                   (4, 400, 128)])
def test_prepack_weights_layout(nv, E, K, N):
    # pure data movement: byte-exact against NumPy's transpose and reshape,
    # padding bytes zero
    rng = np.random.default_rng(E + K + N)
    q = rng.integers(0, 256, (E, K // 2, N)).astype(np.uint8)
    sf = rng.integers(0, 256, (E, K // 16, N)).astype(np.uint8)
    q_t, sf_t = (to_host(t) for t in nv.prepack_weights(to_dev(q), to_dev(sf)))
    ldq, _, ldwsf = nv.operand_pitches(K)
    assert q_t.shape == (E, N // 16, ldq // 32, 16, 32)
    assert sf_t.shape == (E, N // 16, ldwsf // 32, 16, 32)
    assert (q_t == _packed_data(q, ldq)).all()
    assert (sf_t == _packed_scales(sf, ldwsf)).all()
    # spot checks of the scale layout by its index formula
    for e, g, c in [(0, 0, 0), (E - 1, K // 16 - 1, N - 1), (0, min(9, K // 16 - 1), min(17, N - 1))]:
        st, pair, b = g // 8, (g % 8) // 2, g % 2
        flat = sf_t[e].reshape(-1)
        off = (c // 16) * 16 * ldwsf + (st // 4) * 512 + (c % 16) * 32 + pair * 8 + (st % 4) * 2 + b
        assert flat[off] == sf[e, g, c]
