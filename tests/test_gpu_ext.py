"""GPU extensions against the oracle: static activation scale, per-half weight
global scales, and the top-k router (all through the C ABI)."""
import numpy as np
import pytest

import workloads as W
from conftest import to_dev, to_host
from helpers import make_layer
from oracle.formats import bf16_from_f64, bf16_to_f32
from oracle.quantize import (global_scale, quantize_bf16_static, quantize_weight_bf16,
                             quantize_weight_bf16_parts)
from oracle.router import route_topk
from test_gpu_moe import compare_layer

pytestmark = pytest.mark.gpu


def _x(shape, seed, std=3.0):
    return bf16_from_f64(np.random.default_rng(seed).standard_normal(shape) * std)


# ---------------------------------------------------------------- static scale

@pytest.mark.parametrize("M,K", [(1, 16), (37, 272), (256, 7168), (4096, 512)])
@pytest.mark.parametrize("factor", [0.0, 0.05, 0.5, 1.0, 3.0])
def test_quantize_static_bit_exact(nv, M, K, factor):
    import torch
    x = _x((M, K), M + K)
    amax = float(np.abs(bf16_to_f32(x)).max())
    gs = np.float32(global_scale(np.float32(amax)) * np.float32(factor))
    q, sf = nv.quantize_static(to_dev(x), to_dev(np.array([gs], np.float32)))
    torch.cuda.synchronize()
    rq, rsf, _ = quantize_bf16_static(x, gs)
    assert (to_host(sf) == rsf).all()
    assert (to_host(q) == rq).all()
    if 0 < factor < 1:
        assert (rsf == 0x7E).any()           # saturated blocks are exercised


# ------------------------------------------------------- per-part weight scales

@pytest.mark.parametrize("E,K,N,parts", [(3, 256, 288, 2), (2, 7168, 6144, 2), (4, 128, 96, 3),
                                         (2, 512, 64, 1)])
def test_quantize_weights_parts_bit_exact(nv, E, K, N, parts):
    import torch
    w = np.stack([W.normal_bf16((K, N), 0.02, 70 + e, 1) for e in range(E)])
    if parts > 1:
        # make the parts' ranges differ by powers of two
        f = bf16_to_f32(w).astype(np.float64)
        for p in range(parts):
            f[:, :, p * (N // parts):(p + 1) * (N // parts)] *= 2.0 ** (-3 * p)
        w = bf16_from_f64(f)
    q, sf, a = nv.quantize_weights_parts(to_dev(w), parts)
    torch.cuda.synchronize()
    q, sf, a = to_host(q), to_host(sf), to_host(a)
    for e in range(E):
        rq, rsf, ra = quantize_weight_bf16_parts(w[e], parts)
        assert (sf[e] == rsf).all() and (q[e] == rq).all()
        assert (a[e].view(np.uint32) == ra.view(np.uint32)).all()
    if parts == 1:
        q1, sf1, a1 = nv.quantize_weights(to_dev(w))
        assert (to_host(q1) == q).all() and (to_host(sf1) == sf).all()
        assert (to_host(a1) == a[:, 0]).all()


# ------------------------------------------------- layer with per-half scales

@pytest.mark.parametrize("T,H,I,E,k", [(32, 256, 128, 4, 2), (300, 512, 256, 6, 3),
                                       (8, 1024, 512, 8, 4)])
def test_layer_per_half_alphas(nv, T, H, I, E, k):
    # up half at 2^-4 of gate: the two global scales differ by 16x
    cfg = W.small_layer(f"ph{T}", T=T, H=H, I=I, E=E, topk=k, seed=T + 7 * I)
    L = make_layer(cfg, w13_parts=2, up_scale=2.0 ** -4)
    assert L["w13a"].shape == (E, 2)
    assert (L["w13a"][:, 0] > 8 * L["w13a"][:, 1]).all()
    compare_layer(nv, L, f"per-half T{T} H{H} I{I} E{E} k{k}")


def test_layer_per_half_equal_alphas_match_per_expert(nv):
    # (E, 2) alphas with equal halves give bit-identical output to (E,) alphas
    from helpers import run_gpu_layer
    cfg = W.small_layer("pheq", T=200, H=512, I=256, E=4, topk=2, seed=31)
    L = make_layer(cfg)
    g1 = run_gpu_layer(nv, L)
    L2 = dict(L)
    L2["w13a"] = np.stack([L["w13a"], L["w13a"]], axis=1)
    g2 = run_gpu_layer(nv, L2)
    assert (g1["y"] == g2["y"]).all() and (g1["act"] == g2["act"]).all()


# ---------------------------------------------- layer with a static x scale

@pytest.mark.parametrize("T,factor", [(32, 0.5), (32, 2.0), (300, 0.25), (300, 1.0), (8, 0.1)])
def test_layer_static_x_scale(nv, T, factor):
    cfg = W.small_layer(f"st{T}", T=T, H=512, I=256, E=6, topk=3, seed=T + 40)
    L = make_layer(cfg)
    amax = float(np.abs(bf16_to_f32(L["x"])).max())
    L["x_gs"] = np.float32(global_scale(np.float32(amax)) * np.float32(factor))
    g, r, _ = compare_layer(nv, L, f"static x scale T{T} x{factor}")
    assert g["gs1"] == L["x_gs"]
    if factor < 1:
        assert (r["xsf"] == 0x7E).any()


# ---------------------------------------------------------------------- router

def _check_router(nv, logits, k):
    import torch
    ids, w = nv.route_topk(to_dev(logits), k)
    torch.cuda.synchronize()
    ids, w = to_host(ids), to_host(w)
    rid, rw = route_topk(logits, k)
    assert (ids == rid).all(), np.argwhere(ids != rid)[:5]
    # float32 exp and sum against float64: |d| = l_0 - l_j up to ~30 here,
    # relative error below (|d| + 2 + k + 1) * 2^-24 < 4e-6
    assert np.allclose(w, rw, rtol=4e-6, atol=1e-9), float(np.abs(w - rw).max())
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=2e-6)
    return ids, w


def test_router_prefill_routing(nv):
    # the layer configs' router: logits N(0,1), top-8 of 48 (4096 tokens) and
    # the skewed bias (8192 tokens)
    for cfg in (W.PREFILL, W.SKEWED):
        rng = np.random.default_rng(cfg.seed_x)
        logits = (rng.standard_normal((cfg.T, cfg.E)) + W.zipf_bias(cfg)[None, :]).astype(np.float32)
        ids, _ = _check_router(nv, logits, cfg.topk)
        if cfg.zipf_s > 0:
            assert (np.bincount(ids.ravel(), minlength=cfg.E) == 0).sum() >= 4


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 7, 7), (33, 64, 3), (100, 65, 10),
                                   (17, 512, 1), (9, 512, 64), (3, 300, 100)])
def test_router_shapes(nv, T, E, k):
    logits = np.random.default_rng(T * E + k).standard_normal((T, E)).astype(np.float32) * 3
    _check_router(nv, logits, k)


def test_router_ties_take_smaller_index(nv):
    # few distinct values: many exact ties, broken toward the smaller expert
    rng = np.random.default_rng(5)
    logits = (rng.integers(-2, 3, size=(257, 40)) * 0.5).astype(np.float32)
    logits[0] = 1.0                                     # all equal
    ids, w = _check_router(nv, logits, 6)
    assert ids[0].tolist() == list(range(6))
    assert np.allclose(w[0], 1 / 6, rtol=1e-6)


def test_router_output_drives_the_layer(nv):
    # router on the device, its ids and weights fed to the layer: the layer's
    # result equals the oracle layer run on the oracle router's output
    import torch
    cfg = W.small_layer("rt", T=64, H=256, I=128, E=8, topk=2, seed=77)
    L = make_layer(cfg)
    logits = np.random.default_rng(77).standard_normal((cfg.T, cfg.E)).astype(np.float32)
    ids, w = nv.route_topk(to_dev(logits), cfg.topk)
    torch.cuda.synchronize()
    rid, rw = route_topk(logits, cfg.topk)
    assert (to_host(ids) == rid).all()
    L["ids"] = to_host(ids)
    L["wts"] = to_host(w)
    compare_layer(nv, L, "router -> layer")
