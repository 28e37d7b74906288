"""The Python binding's checks of caller-given outputs and workspaces: a wrong
shape, dtype or a host tensor is rejected before any kernel is launched, and
correct caller-given outputs give the same bytes as allocated ones."""
import numpy as np
import pytest

import workloads as W
from conftest import to_dev, to_host
from helpers import gpu_packed_weights, make_layer

pytestmark = pytest.mark.gpu


def _x(M, K, seed=3):
    from oracle.formats import bf16_from_f64
    return to_dev(bf16_from_f64(np.random.default_rng(seed).standard_normal((M, K)) * 2.0))


def test_quantize_rejects_bad_outputs(nv):
    import torch
    x = _x(8, 64)
    u8 = dict(dtype=torch.uint8, device=x.device)
    with pytest.raises(ValueError):
        nv.quantize(x, q=torch.empty((8, 16), **u8))                 # needs (8, 32)
    with pytest.raises(ValueError):
        nv.quantize(x, sf=torch.empty((8, 2), **u8))                 # needs (8, 4)
    with pytest.raises(TypeError):
        nv.quantize(x, q=torch.empty((8, 32), dtype=torch.int8, device=x.device))
    with pytest.raises(ValueError):
        nv.quantize(x, gs=torch.empty((2,), dtype=torch.float32, device=x.device))
    with pytest.raises(TypeError):
        nv.quantize(x, workspace=torch.empty((1024,), dtype=torch.uint8))   # host memory
    with pytest.raises(ValueError):
        nv.quantize_static(x, torch.empty((0,), dtype=torch.float32, device=x.device))
    with pytest.raises(ValueError):
        nv.quantize_static(x, torch.ones((1,), dtype=torch.float32, device=x.device),
                           q=torch.empty((4, 32), **u8))


def test_quantize_caller_outputs_match(nv):
    import torch
    x = _x(40, 272, seed=9)
    q0, sf0, gs0 = nv.quantize(x)
    q = torch.full((40, 136), 0xAB, dtype=torch.uint8, device=x.device)
    sf = torch.full((40, 17), 0xCD, dtype=torch.uint8, device=x.device)
    gs = torch.full((1,), -1.0, dtype=torch.float32, device=x.device)
    # a workspace of another dtype: its size in bytes is what the library sees
    ws = torch.empty((64,), dtype=torch.float32, device=x.device)
    q1, sf1, gs1 = nv.quantize(x, q=q, sf=sf, gs=gs, workspace=ws)
    torch.cuda.synchronize()
    assert q1 is q and sf1 is sf and gs1 is gs
    assert (to_host(q1) == to_host(q0)).all() and (to_host(sf1) == to_host(sf0)).all()
    assert to_host(gs1)[0] == to_host(gs0)[0]


def test_route_topk_rejects_bad_outputs(nv):
    import torch
    logits = torch.zeros((5, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        nv.route_topk(logits, 2, ids=torch.empty((5, 3), dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        nv.route_topk(logits, 2, weights=torch.empty((5, 2), dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        nv.route_topk(logits, 0)


def test_gemm_rejects_bad_output(nv):
    import torch
    K, N, M = 256, 64, 16
    from oracle.formats import bf16_from_f64
    w = to_dev(bf16_from_f64(np.random.default_rng(1).standard_normal((1, K, N)) * 0.02))
    wq, wsf, wa = nv.quantize_weights(w)
    bq, bsf = nv.prepack_weights(wq, wsf)
    ldq, ldsf, _ = nv.operand_pitches(K)
    aq = torch.zeros((M, ldq), dtype=torch.uint8, device="cuda")
    asf = torch.zeros((M, K // 16), dtype=torch.uint8, device="cuda")
    a_gs = torch.ones((1,), dtype=torch.float32, device="cuda")
    # aq (M, ldq) holds K = 2 * ldq = 256 elements here (ldq = K / 2 at K = 256)
    assert ldq == K // 2
    with pytest.raises(ValueError):
        nv.gemm(aq, asf, a_gs, bq[0], bsf[0], wa, out=torch.empty((M, N + 16), dtype=torch.bfloat16,
                                                               device="cuda"))
    with pytest.raises(ValueError):
        nv.gemm(aq, asf, torch.empty((0,), dtype=torch.float32, device="cuda"), bq[0], bsf[0], wa)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    assert nv.gemm(aq, asf, a_gs, bq[0], bsf[0], wa, out=out) is out
    torch.cuda.synchronize()
    assert (out.float() == 0).all()                      # zero activations


def test_moe_forward_rejects_bad_outputs(nv):
    import torch
    cfg = W.small_layer("bind", T=16, H=256, I=128, E=4, topk=2, seed=5)
    L = make_layer(cfg)
    args = [to_dev(L[k]) for k in ("x", "ids", "wts")]
    pw = gpu_packed_weights(nv, L)
    w = [pw[k] for k in ("w13", "w13_sf", "w13a", "w2", "w2_sf", "w2a")]
    x = args[0]
    with pytest.raises(ValueError):
        nv.moe_forward(*args, *w, y=torch.empty((16, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):
        nv.moe_forward(*args, *w, workspace=torch.empty((16,), dtype=torch.uint8))   # host memory
    nws = nv.moe_workspace_size(16, 256, 128, 4, 2)
    y0 = nv.moe_forward(*args, *w)
    y = torch.empty((16, 256), dtype=torch.bfloat16, device=x.device)
    ws = torch.empty(((nws + 3) // 4,), dtype=torch.int32, device=x.device)
    assert nv.moe_forward(*args, *w, y=y, workspace=ws) is y
    torch.cuda.synchronize()
    assert (to_host(y) == to_host(y0)).all()
