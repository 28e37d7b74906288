"""A layer whose output has a closed form, worked out by hand from the rule
(NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline", Hypothesis 6; the readings of
the SiLU, requantization and combine steps listed with the oracle), as an
end-to-end pin of the oracle that does not re-run its own code.

Inputs, all constant so that every quantization is exact:
  x = 3.0 everywhere (T tokens of H = 256);
  expert 0: gate weights 0.5, up weights 0.25, w2 weights 2^-10;
  expert 1: gate weights 0.5, up weights 0.125, w2 weights 2^-10;
  every token routed to (expert 0, expert 1) with weights (0.25, 0.75).

By hand:
  * x: gs1 = 3/2688, every block scale 448 (E4M3 0x7E), every code 6; the
    dequantized x is exactly 3 (6 * 448 * gs1).
  * w13 of expert e (one global scale per expert, the gate amax 0.5): gate
    blocks scale 448, up blocks scale 224 (e = 0) or 112 (e = 1), codes 6:
    exact.
  * L1: gate = H * 3 * 0.5 = 384, up = H * 3 * u_e = 192 or 96 (bf16 exact).
  * SiLU: 1 + e^-384 is 1 in float64, so act = bf16(384 * up) taken from just
    below the product: 73728 (expert 0) and 36864 (expert 1), both bf16 exact
    and not rounding midpoints.
  * requant: gs2 = 73728 / 2688 over all act rows; expert 0 rows get scale
    448, expert 1 rows 224, codes 6: exact.
  * L2 of expert e: o = I * act_e * 2^-10 = 9216 and 4608 (I = 128).
  * combine: y = 0.25 * 9216 + 0.75 * 4608 = 5760 (1.40625 * 2^12, bf16
    exact). Swapping the two routing weights would give 8064; dropping an
    alpha, or a global scale, would change it by orders of magnitude.
"""
import numpy as np

from oracle.formats import bf16_from_f64, bf16_to_f32
from oracle.moe import moe_forward
from oracle.quantize import quantize_weight_bf16

T, H, I, E, K = 4, 256, 128, 2, 2


def _bf16(value, shape):
    return bf16_from_f64(np.full(shape, value, dtype=np.float64))


def _layer():
    x = _bf16(3.0, (T, H))
    w13q = np.zeros((E, H // 2, 2 * I), np.uint8)
    w13sf = np.zeros((E, H // 16, 2 * I), np.uint8)
    w2q = np.zeros((E, I // 2, H), np.uint8)
    w2sf = np.zeros((E, I // 16, H), np.uint8)
    w13a = np.zeros(E, np.float32)
    w2a = np.zeros(E, np.float32)
    for e, up in enumerate((0.25, 0.125)):
        w13 = np.concatenate([np.full((H, I), 0.5), np.full((H, I), up)], axis=1)
        w13q[e], w13sf[e], w13a[e] = quantize_weight_bf16(bf16_from_f64(w13))
        w2q[e], w2sf[e], w2a[e] = quantize_weight_bf16(_bf16(2.0 ** -10, (I, H)))
    ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    wts = np.tile(np.array([[0.25, 0.75]], np.float32), (T, 1))
    return x, ids, wts, w13q, w13sf, w13a, w2q, w2sf, w2a


def test_layer_closed_form():
    r = moe_forward(*_layer(), keep=True)
    assert np.float32(r["gs1"]) == np.float32(3.0) / np.float32(2688.0)
    assert (r["xsf"] == 0x7E).all() and (r["xq"] == 0x77).all()      # scale 448, codes 6 | 6 << 4
    act = bf16_to_f32(r["act_bits"]).astype(np.float64)
    assert (act[:, 0] == 73728.0).all() and (act[:, 1] == 36864.0).all()
    assert np.float32(r["gs2"]) == np.float32(73728.0) / np.float32(2688.0)
    y = bf16_to_f32(r["y_bits"]).astype(np.float64)
    assert (y == 5760.0).all(), np.unique(y)
    # the unrounded value differs from 5760 only by the float32 roundings of
    # the global scales (relative 2^-23 at most)
    assert np.abs(r["y"] - 5760.0).max() <= 5760.0 * 2.0 ** -22


def test_layer_closed_form_swapped_weights():
    x, ids, wts, *w = _layer()
    y = bf16_to_f32(moe_forward(x, ids, wts[:, ::-1].copy(), *w)["y_bits"]).astype(np.float64)
    assert (y == 8064.0).all(), np.unique(y)                          # 0.75 * 9216 + 0.25 * 4608
