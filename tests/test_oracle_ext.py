"""Pins of the oracle's extensions beyond the five stages: the static activation
scale, per-half weight global scales and the top-k router."""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import loops
from oracle.formats import bf16_from_f64, bf16_to_f32
from oracle.moe import moe_forward
from oracle.quantize import (global_scale, quantize_bf16, quantize_bf16_static,
                             quantize_weight_bf16, quantize_weight_bf16_parts)
from oracle.router import route_topk


def _bf16(vals):
    return bf16_from_f64(np.asarray(vals, dtype=np.float64))


# ---------------------------------------------------------------- static scale

def test_static_scale_equal_to_dynamic_reproduces_dynamic_rule():
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((6, 96)) * 3.0)
    q, sf, gs = quantize_bf16(x)
    q2, sf2, gs2 = quantize_bf16_static(x, gs)
    assert (q == q2).all() and (sf == sf2).all() and gs2 == gs


@pytest.mark.parametrize("frac", [0.9, 0.5, 0.1, 0.01])
def test_static_scale_saturates_like_clamped_input(frac):
    # A static scale gs = fl32(c / 2688) below the tensor's own amax / 2688
    # saturates: every block whose amax exceeds c gets scale byte 0x7E and its
    # larger elements magnitude 6, exactly as the dynamic rule does on x
    # clamped to [-c, c] (whose amax is c). This ties the static path to the
    # pinned dynamic rule.
    rng = np.random.default_rng(int(frac * 1000))
    x = _bf16(rng.standard_normal((8, 128)) * 4.0)
    xf = bf16_to_f32(x).astype(np.float64)
    c = float(bf16_to_f32(_bf16([np.abs(xf).max() * frac]))[0])
    gs = global_scale(np.float32(c))
    xc = _bf16(np.clip(xf, -c, c))
    assert np.abs(bf16_to_f32(xc)).max() == c
    q, sf, gs_s = quantize_bf16_static(x, gs)
    qc, sfc, gsc = quantize_bf16(xc)
    assert gs_s == gsc == gs
    assert (q == qc).all() and (sf == sfc).all()
    if frac < 1:
        assert (sf == 0x7E).any()


@pytest.mark.parametrize("gs_factor", [1e-3, 0.3, 1.0, 7.0, 1e4])
def test_static_scale_matches_exact_twin(gs_factor):
    rng = np.random.default_rng(int(gs_factor * 10) + 3)
    x = _bf16(rng.standard_normal((3, 64)) * 2.0)
    x[0, :16] = 0                                      # an all-zero block
    gs = np.float32(global_scale(np.float32(np.abs(bf16_to_f32(x)).max())) * gs_factor)
    q, sf, _ = quantize_bf16_static(x, gs)
    tq, tsf, tgs = loops.quantize(x.tolist(), gs=float(gs))
    assert tgs == float(gs)
    assert (q == np.array(tq, np.uint8)).all() and (sf == np.array(tsf, np.uint8)).all()


def test_static_scale_zero_gives_zero_codes_with_signs():
    x = _bf16([[1.0, -2.0, 0.0, -0.0] * 4])
    q, sf, gs = quantize_bf16_static(x, np.float32(0.0))
    assert (sf == 0).all() and gs == 0
    nib = np.stack([q & 0xF, q >> 4], axis=-1).reshape(1, -1)
    assert ((nib & 7) == 0).all()
    assert (nib[0] >> 3).tolist() == [0, 1, 0, 1] * 4


# ---------------------------------------------------------- per-half weights

def test_weight_parts_one_is_the_per_matrix_rule():
    w = W.normal_bf16((64, 48), 0.02, 5, 1)
    q, sf, a = quantize_weight_bf16(w)
    q1, sf1, a1 = quantize_weight_bf16_parts(w, 1)
    assert (q == q1).all() and (sf == sf1).all() and a1.tolist() == [a]


def test_weight_parts_share_scale_when_halves_share_amax():
    # if both halves hold the same amax, per-half scales equal the per-matrix
    # scale and the bytes are identical
    w = W.normal_bf16((64, 32), 0.02, 6, 1).copy()
    wf = bf16_to_f32(w)
    i, j = np.unravel_index(np.abs(wf).argmax(), wf.shape)
    other = (j + 16) % 32
    w[i, other] = w[i, j] ^ np.uint16(0x8000)          # same magnitude, other half
    q, sf, a = quantize_weight_bf16(w)
    q2, sf2, a2 = quantize_weight_bf16_parts(w, 2)
    assert a2[0] == a2[1] == a
    assert (q == q2).all() and (sf == sf2).all()


def test_weight_parts_are_independent_of_the_other_half():
    # scaling the up half by 2^-6 scales only its alpha by 2^-6; bytes unchanged
    w = W.normal_bf16((64, 32), 0.02, 7, 1)
    wf = bf16_to_f32(w).astype(np.float64)
    w2 = _bf16(np.concatenate([wf[:, :16], wf[:, 16:] * 2.0 ** -6], axis=1))
    q, sf, a = quantize_weight_bf16_parts(w, 2)
    q2, sf2, a2 = quantize_weight_bf16_parts(w2, 2)
    assert (q == q2).all() and (sf == sf2).all()
    assert a2[0] == a[0] and a2[1] == np.float32(a[1] * 2.0 ** -6)


def _tiny_layer(parts=1, up_scale=1.0):
    cfg = W.TINY
    x = W.activations(cfg)
    ids, wts = W.routing(cfg)
    w13q, w13sf, w13a, w2q, w2sf, w2a = [], [], [], [], [], []
    for e in range(cfg.E):
        w13, w2 = W.expert_weights_bf16(cfg, e)
        if up_scale != 1.0:
            f = bf16_to_f32(w13).astype(np.float64)
            f[:, cfg.I:] *= up_scale
            w13 = _bf16(f)
        q, sf, a = quantize_weight_bf16_parts(w13, parts) if parts > 1 else quantize_weight_bf16(w13)
        w13q.append(q); w13sf.append(sf); w13a.append(a)
        q, sf, a = quantize_weight_bf16(w2)
        w2q.append(q); w2sf.append(sf); w2a.append(a)
    return (x, ids, wts, np.stack(w13q), np.stack(w13sf), np.array(w13a, np.float32),
            np.stack(w2q), np.stack(w2sf), np.array(w2a, np.float32))


def test_layer_with_equal_half_alphas_is_the_per_expert_layer():
    L = _tiny_layer()
    ref = moe_forward(*L, keep=True)
    a2 = np.stack([L[5], L[5]], axis=1)
    out = moe_forward(*L[:5], a2, *L[6:], keep=True)
    assert (out["y_bits"] == ref["y_bits"]).all()
    assert (out["gu"] == ref["gu"]).all()


def test_layer_up_half_alpha_scales_only_up_columns():
    L = _tiny_layer()
    I = W.TINY.I
    a2 = np.stack([L[5], L[5] * np.float32(4.0)], axis=1)
    ref = moe_forward(*L, keep=True)
    out = moe_forward(*L[:5], a2, *L[6:], keep=True)
    v = ref["valid"]
    assert (out["gu"][v][:, :I] == ref["gu"][v][:, :I]).all()
    assert (out["gu"][v][:, I:] == 4.0 * ref["gu"][v][:, I:]).all()


def test_per_half_scales_reduce_up_error_when_halves_differ():
    # with the up half 2^-18 as large as gate, one shared scale pushes the up
    # half's block scales to the bottom of the E4M3 subnormals (one or two
    # significant bits, many flushed to 0); per-half scales keep the up
    # half's round-trip error where it is without the 2^-18
    cfg = W.TINY
    w13, _ = W.expert_weights_bf16(cfg, 0)
    f = bf16_to_f32(w13).astype(np.float64)
    f[:, cfg.I:] *= 2.0 ** -18
    w = _bf16(f)
    wf = bf16_to_f32(w).astype(np.float64)
    from oracle.quantize import dequantize_cols

    def up_err(q, sf, alphas):
        d = dequantize_cols(q, sf)
        d[:, :cfg.I] *= alphas[0]
        d[:, cfg.I:] *= alphas[-1]
        up = wf[:, cfg.I:]
        return np.linalg.norm(d[:, cfg.I:] - up) / np.linalg.norm(up)

    q, sf, a = quantize_weight_bf16(w)
    q2, sf2, a2 = quantize_weight_bf16_parts(w, 2)
    assert up_err(q2, sf2, a2) < 0.25 * up_err(q, sf, [a])
    q3, sf3, _ = quantize_weight_bf16_parts(w13, 2)
    assert (q3 == q2).all() and (sf3 == sf2).all()


# -------------------------------------------------------------------- router

def test_router_brute_force_tiny():
    rng = np.random.default_rng(3)
    for trial in range(40):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        # few distinct values so that ties occur
        lg = rng.integers(-3, 3, size=(1, E)).astype(np.float32) * np.float32(0.5)
        ids, w = route_topk(lg, k)
        best = None
        for comb in itertools.combinations(range(E), k):
            s = sum(float(lg[0, c]) for c in comb)
            if best is None or s > best[0] or (s == best[0] and list(comb) < best[1]):
                best = (s, list(comb))
        assert sorted(ids[0].tolist()) == best[1]
        vals = lg[0, ids[0]]
        assert (np.diff(vals) <= 0).all()
        for a, b in zip(ids[0][:-1], ids[0][1:]):
            if lg[0, a] == lg[0, b]:
                assert a < b
        assert abs(w.sum() - 1.0) < 1e-15


def test_router_k1_weight_is_one_and_equal_logits_uniform():
    lg = np.random.default_rng(4).standard_normal((16, 10)).astype(np.float32)
    ids, w = route_topk(lg, 1)
    assert (w == 1.0).all() and (ids[:, 0] == lg.argmax(axis=1)).all()
    ids, w = route_topk(np.full((3, 12), 0.7, np.float32), 4)
    assert (ids == np.arange(4)).all()
    assert np.allclose(w, 0.25, rtol=0, atol=1e-16)


def test_router_weights_shift_invariant():
    lg = np.random.default_rng(5).standard_normal((32, 48)).astype(np.float32)
    ids, w = route_topk(lg, 8)
    ids2, w2 = route_topk(lg + np.float32(8.0), 8)
    assert (ids == ids2).all()
    assert np.allclose(w, w2, rtol=1e-6, atol=0)       # only the float32 shift rounds


def test_router_matches_library_topk_softmax():
    # special case that reduces to library routines: torch.topk + softmax on
    # distinct logits (float64)
    lg = np.random.default_rng(6).standard_normal((256, 48)).astype(np.float32)
    ids, w = route_topk(lg, 8)
    v, i = torch.topk(torch.from_numpy(lg.astype(np.float64)), 8, dim=1)
    assert (ids == i.numpy()).all()
    assert np.allclose(w, torch.softmax(v, dim=1).numpy(), rtol=1e-14, atol=0)
