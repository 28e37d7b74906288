"""The allocation-free layer entry point (nvfp4_moe_forward_noalloc, static
per-GPU scratch) against nvfp4_moe_forward with a caller workspace: y must be
bit-identical, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's intermediates), on both GEMM paths."""
import numpy as np
import pytest

import workloads as W
from conftest import to_dev, to_host
from helpers import gpu_packed_weights, make_layer

pytestmark = pytest.mark.gpu


def _layer(nv, cfg):
    L = make_layer(cfg)
    return L, gpu_packed_weights(nv, L), {k: to_dev(L[k]) for k in ("x", "ids", "wts")}


def _both(nv, d, pw):
    """y of the workspace entry point, then of the allocation-free one."""
    import torch
    args = (d["x"], d["ids"], d["wts"], pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"],
            pw["w2a"])
    y_ws = to_host(nv.moe_forward(*args))
    y = torch.full_like(d["x"], float("nan"))
    nv.moe_forward_noalloc(*args, y=y)
    torch.cuda.synchronize()
    return y_ws, to_host(y)


def test_noalloc_matches_workspace_entry_point(nv):
    # first a tiled-GEMM batch (800 slots on 8 experts), then a smaller
    # weight-streaming one (12 slots on 4 experts) and a one-token call
    big = W.small_layer("na1", T=200, H=512, I=256, E=8, topk=4, seed=31)
    small = W.small_layer("na2", T=6, H=256, I=128, E=4, topk=2, seed=32)
    one = W.small_layer("na3", T=1, H=256, I=128, E=4, topk=2, seed=33)
    for cfg in (big, small, one):
        L, pw, d = _layer(nv, cfg)
        assert nv.moe_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk) <= nv.MOE_SCRATCH_BYTES
        y_ws, y_na = _both(nv, d, pw)
        assert (y_na == y_ws).all(), f"{cfg.name}: allocation-free y differs"
        assert np.isfinite(y_na.view(np.int16).astype(np.float32)).all()


def test_noalloc_options_and_repeat(nv):
    # per-half alphas through the options; the same call twice gives the same y
    import torch
    cfg = W.small_layer("na4", T=40, H=256, I=128, E=4, topk=2, seed=34)
    L = make_layer(cfg, w13_parts=2)
    pw = gpu_packed_weights(nv, L)
    d = {k: to_dev(L[k]) for k in ("x", "ids", "wts")}
    args = (d["x"], d["ids"], d["wts"], pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"],
            pw["w2a"])
    assert pw["w13a"].dim() == 2
    y_ws = to_host(nv.moe_forward(*args))
    y1 = to_host(nv.moe_forward_noalloc(*args))
    y2 = to_host(nv.moe_forward_noalloc(*args))
    torch.cuda.synchronize()
    assert (y1 == y_ws).all() and (y2 == y_ws).all()


def test_noalloc_rejects_oversized_problem(nv):
    import torch
    cfg = W.small_layer("na5", T=4, H=256, I=128, E=4, topk=2, seed=35)
    L, pw, d = _layer(nv, cfg)
    T = 30000        # 30000 x 2 slots x (I = 128) needs more than the scratch
    x = torch.zeros((T, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, 2), dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    assert nv.moe_workspace_size(T, 256, 128, 4, 2) > nv.MOE_SCRATCH_BYTES
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.moe_forward_noalloc(x, ids, wts, pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"],
                               pw["w2a"])
    assert e.value.status == 6


def test_noalloc_in_a_hip_graph(nv):
    # the use it is for: the layer captured into a HIP graph (no allocation or
    # workspace inside the captured call). Every replay, with eager calls and
    # synchronizations between them, must give the eager result bit for bit.
    import torch
    for cfg in (W.small_layer("nag1", T=6, H=256, I=128, E=4, topk=2, seed=36),
                W.small_layer("nag2", T=120, H=256, I=128, E=4, topk=2, seed=37)):
        L, pw, d = _layer(nv, cfg)
        args = (d["x"], d["ids"], d["wts"], pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"],
                pw["w2a"])
        y_ref = to_host(nv.moe_forward(*args))
        y = torch.empty_like(d["x"])
        nv.moe_forward_noalloc(*args, y=y)          # first call on the device: set-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            nv.moe_forward_noalloc(*args, y=y)
        for rep in range(3):
            y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert (to_host(y) == y_ref).all(), f"{cfg.name}: replay {rep} differs"
            assert (to_host(nv.moe_forward(*args)) == y_ref).all()     # eager work between replays
            torch.cuda.synchronize()
