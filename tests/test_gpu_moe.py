"""GPU expert layer (nvfp4_moe_forward) against the oracle, stage by stage."""
import numpy as np
import pytest

import workloads as W
from helpers import (bf16_ulp_distance, check_bf16_output, cosine, make_layer,
                     run_gpu_layer, run_oracle_layer)

pytestmark = pytest.mark.gpu


def compare_layer(nv, L, label, min_act_exact=0.995, pool=None):
    """Stage-by-stage parity of one layer call, each stage against the
    oracle's step applied to the GPU's own inputs of that stage (teacher
    forcing), plus the free-running layer against the full oracle:

    1. xq, xsf, gs1 bit-exact with the oracle's quantization of x;
    2. routing tables exact;
    3. gate_up (the L1 output, from the tap) within the GEMM bound of the
       oracle's unrounded L1 of the same slot (each half on its own scale);
    4. act bit-exact with the oracle's SiLU*up of the GPU's gate_up, and the
       requantized aq, asf, gs2 bit-exact with the oracle's quantization of
       the GPU's act rows;
    5. y of every token within the bound (2e-3 before the final rounding,
       plus faithful rounding) of the oracle's L2 and combine run on the GPU's
       aq, asf and gs2.
    Free-running: act against the oracle's own act (at most 2 ulps or 2^-12 of
    the act amax apart, mostly identical) and y against the full oracle
    (cosine >= 0.9999).

    The layer runs twice, without and then with the gate/up tap; y must be
    identical.
    """
    from oracle.formats import bf16_to_f32
    from oracle.moe import l2_combine, silu_mul_bf16
    from oracle.quantize import quantize_bf16
    g = run_gpu_layer(nv, L, repeat=2)
    assert (g["ys"][0] == g["ys"][1]).all(), f"{label}: the gate/up tap changed y"
    r = run_oracle_layer(L, pool=pool)
    T, k = L["ids"].shape
    E = L["w13q"].shape[0]
    I = L["w2q"].shape[1] * 2
    S = T * k
    ids = L["ids"].astype(np.int64)
    valid = (ids >= 0) & (ids < E)

    # stage 1: quantized x, bit-exact
    assert g["gs1"].view(np.uint32) == np.float32(r["gs1"]).view(np.uint32), f"{label}: gs1"
    assert (g["xsf"] == r["xsf"]).all(), f"{label}: xsf"
    assert (g["xq"] == r["xq"]).all(), f"{label}: xq"

    # stage 2: routing tables
    cnt = np.bincount(ids[valid], minlength=E)
    assert (g["counts"] == cnt).all(), f"{label}: counts"
    assert (g["offsets"] == np.concatenate([[0], np.cumsum(cnt)])).all(), f"{label}: offsets"
    nvalid = int(valid.sum())
    order = np.argsort(np.where(valid.ravel(), ids.ravel(), E), kind="stable")[:nvalid]
    assert (g["sorted_slot"][:nvalid] == order).all(), f"{label}: sorted order"
    slot_row = np.full(S, -1)
    slot_row[order] = np.arange(nvalid)
    assert (g["slot_row"] == slot_row).all(), f"{label}: slot_row"
    t_of, j_of = np.divmod(order, k)
    st = {}

    gpu_act = g["act"][:nvalid]
    if nvalid:
        # stage 3: gate_up against the oracle's unrounded L1 of the same slot
        gu = g["gu"][:nvalid]
        gu_ref = r["gu"][t_of, j_of]
        for half, cols in (("gate", slice(0, I)), ("up", slice(I, 2 * I))):
            sh = check_bf16_output(gu[:, cols], gu_ref[:, cols], f"{label}: {half}", min_exact=0.99)
            st[f"{half}_exact"] = sh["exact"]

        # stage 4: act from the GPU's own gate/up, bit-exact
        act_tf = silu_mul_bf16(gu[:, :I], gu[:, I:])
        bad = np.argwhere(gpu_act != act_tf)
        assert bad.size == 0, f"{label}: act differs from SiLU*up of the GPU's gate/up at {bad[:3]}"
        # requantization of the GPU's act rows, bit-exact (one gs2 over them)
        q_tf, sf_tf, gs2_tf = quantize_bf16(gpu_act)
        assert g["gs2"].view(np.uint32) == np.float32(gs2_tf).view(np.uint32), f"{label}: gs2"
        assert (g["asf"][:nvalid] == sf_tf).all(), f"{label}: asf"
        assert (g["aq"][:nvalid] == q_tf).all(), f"{label}: aq"

        # free-running act against the oracle's own act of the same slot: a
        # gate/up sum within float32 noise of a bf16 midpoint may round the
        # other way (stage 3 allows it), and act then follows with the slope
        # of silu: a few ulps for g > 0, many for very negative g, where act
        # is tiny next to the tensor's amax. Bound: 2 ulps or 2^-12 of the
        # act amax, whichever is larger.
        ref_act = r["act_bits"][t_of, j_of]
        same = gpu_act == ref_act
        ga = bf16_to_f32(gpu_act).astype(np.float64)
        ra = bf16_to_f32(ref_act).astype(np.float64)
        ulp = bf16_ulp_distance(gpu_act, ref_act)
        ok = (ulp <= 2) | (np.abs(ga - ra) <= np.abs(ra).max() * 2.0 ** -12)
        assert ok.all(), f"{label}: free-running act beyond bound at {np.argwhere(~ok)[:3]}"
        st["act_exact_free"] = float(same.mean())
        st["act_max_ulp_free"] = int(ulp.max())
        assert st["act_exact_free"] >= min_act_exact, f"{label}: act exact rate {st['act_exact_free']}"
        st["aq_rows_same_free"] = float(((g["aq"][:nvalid] == r["aq"][t_of, j_of]).all(axis=1) &
                                         (g["asf"][:nvalid] == r["asf"][t_of, j_of]).all(axis=1)).mean())
    else:
        assert g["gs2"] == 0, f"{label}: gs2 of an empty act"

    # stage 5: the oracle's L2 and combine on the GPU's requantized rows
    aq_tj = np.zeros((T, k, I // 2), np.uint8)
    asf_tj = np.zeros((T, k, I // 16), np.uint8)
    aq_tj[t_of, j_of] = g["aq"][:nvalid]
    asf_tj[t_of, j_of] = g["asf"][:nvalid]
    y_tf, _ = l2_combine(aq_tj, asf_tj, g["gs2"], ids, L["wts"], L["w2q"], L["w2sf"], L["w2a"], pool=pool)
    sy = check_bf16_output(g["y"], y_tf, f"{label}: y", min_exact=0.98)
    sy.pop("beyond_rounding_rows", None)
    st.update({f"y_{key}": v for key, v in sy.items()})

    # free-running: y against the full oracle
    yg = bf16_to_f32(g["y"]).astype(np.float64)
    st["cos"] = cosine(yg, r["y"])
    ymax = np.abs(r["y"]).max()
    st["max_rel_free"] = float(np.abs(yg - r["y"]).max() / ymax) if ymax > 0 else 0.0
    assert st["cos"] >= 0.9999, f"{label}: free-running cosine {st['cos']}"
    print(label, st)
    return g, r, st


def test_tiny_config(nv):
    compare_layer(nv, make_layer(W.TINY), "tiny")


@pytest.mark.parametrize("T,H,I,E,k", [(77, 272, 144, 6, 3), (1, 256, 128, 4, 2),
                                       (700, 512, 256, 2, 1), (130, 128, 16, 5, 5),
                                       (64, 1040, 400, 8, 2)])
def test_ragged_shapes(nv, T, H, I, E, k):
    cfg = W.small_layer(f"r{T}", T=T, H=H, I=I, E=E, topk=k, seed=T + H + I)
    compare_layer(nv, make_layer(cfg), f"ragged T{T} H{H} I{I} E{E} k{k}")


# shapes where slots per expert average at most 16 take the weight-streaming
# path (16-row tiles): single rows, experts spanning several tiles, K tails;
# K of 8, 12 and 16 whole 128-element steps (two to four groups of four:
# waves start at different groups and wrap around) and of 6 and 9 steps
# (a partial last group)
@pytest.mark.parametrize("T,H,I,E,k", [(8, 256, 128, 8, 4), (60, 512, 256, 8, 2),
                                       (20, 272, 144, 4, 2), (3, 1040, 400, 16, 5),
                                       (33, 128, 16, 3, 1), (12, 1024, 1536, 8, 2),
                                       (5, 2048, 768, 6, 3)])
def test_small_batch_shapes(nv, T, H, I, E, k):
    assert T * k <= 16 * E
    cfg = W.small_layer(f"s{T}", T=T, H=H, I=I, E=E, topk=k, seed=3 * T + H + I)
    compare_layer(nv, make_layer(cfg), f"small-batch T{T} H{H} I{I} E{E} k{k}")


# small batches whose H or I is beyond what the weight-streaming kernels'
# LDS holds (K up to 17,024) take the tiled GEMMs
@pytest.mark.parametrize("T,H,I,E,k", [(4, 17040, 32, 2, 1), (5, 64, 17040, 2, 2)])
def test_small_batch_beyond_streaming_lds(nv, T, H, I, E, k):
    cfg = W.small_layer(f"bigK{H}x{I}", T=T, H=H, I=I, E=E, topk=k, seed=H + I)
    compare_layer(nv, make_layer(cfg), f"small batch, big K: T{T} H{H} I{I}")


# batches above one routing chunk (4096 slots) are routed by one work-group
# per chunk after a counting pre-pass: one slot past a chunk, three chunks
# with skipped ids on the chunk boundaries, and enough slots (264,000) for the
# chunk to grow past 4096 (52 chunks of 5120)
@pytest.mark.parametrize("T,H,I,E,k,skip", [(4097, 128, 16, 5, 1, False), (1100, 256, 128, 16, 8, True),
                                            (33000, 128, 16, 8, 8, False)])
def test_routing_chunks(nv, T, H, I, E, k, skip):
    cfg = W.small_layer(f"chunks{T}", T=T, H=H, I=I, E=E, topk=k, seed=T + E)
    L = make_layer(cfg)
    if skip:
        ids = L["ids"].copy().ravel()
        for b in (4095, 4096, 8191, 8192, 8799):
            ids[b] = -1 if b % 2 else E + 3
        L["ids"] = ids.reshape(T, k)
    g, _, _ = compare_layer(nv, L, f"routing chunks T{T} k{k}")
    assert g["counts"].sum() == ((L["ids"] >= 0) & (L["ids"] < E)).sum()


# the largest expert count the routing supports (512), on the weight-streaming
# path (8,000 slots <= 16 per expert) and the tiled one with chunked routing
# (48,000 slots, top-16), and top-k equal to E (every token to every expert)
@pytest.mark.parametrize("T,H,I,E,k", [(1000, 128, 64, 512, 8), (3000, 128, 32, 512, 16),
                                       (200, 256, 128, 32, 32)])
def test_max_experts_and_topk(nv, T, H, I, E, k):
    cfg = W.small_layer(f"maxE{E}k{k}", T=T, H=H, I=I, E=E, topk=k, seed=E + k)
    g, _, _ = compare_layer(nv, make_layer(cfg), f"max experts T{T} E{E} k{k}")
    assert g["counts"].sum() == T * k


def test_skipped_ids_and_empty_experts(nv):
    cfg = W.small_layer("skip", T=90, H=256, I=128, E=6, topk=3, seed=9)
    L = make_layer(cfg)
    ids = L["ids"].copy()
    ids[ids == 2] = -1                 # expert 2 left empty
    ids[5, :] = [-1, 6, 99]            # a token with every slot skipped
    ids[7, 1] = -5
    L["ids"] = ids
    g, r, _ = compare_layer(nv, L, "skipped ids")
    from oracle.formats import bf16_to_f32
    assert (bf16_to_f32(g["y"][5]) == 0).all()
    assert g["counts"][2] == 0


def test_skewed_routing_small(nv):
    cfg = W.small_layer("skew", T=300, H=256, I=128, E=16, topk=4, seed=50, zipf_s=1.2,
                        alpha_loguniform=True, outlier_frac=1e-3)
    L = make_layer(cfg)
    cnt = np.bincount(L["ids"].ravel(), minlength=16)
    assert (cnt == 0).sum() >= 1 or cnt.max() >= 0.1 * cnt.sum()
    compare_layer(nv, L, "skewed small")


def test_all_slots_skipped(nv):
    cfg = W.small_layer("none", T=10, H=128, I=64, E=3, topk=2, seed=4)
    L = make_layer(cfg)
    L["ids"] = np.full_like(L["ids"], -1)
    g = run_gpu_layer(nv, L)
    assert (g["y"] & 0x7FFF == 0).all()
    assert g["gs2"] == 0


def test_repeat_is_bit_identical(nv):
    cfg = W.small_layer("rep", T=200, H=512, I=256, E=8, topk=4, seed=12)
    g = run_gpu_layer(nv, make_layer(cfg), repeat=3)
    assert all((y == g["ys"][0]).all() for y in g["ys"])


def test_layer_closed_form(nv):
    # the constant layer of test_oracle_closed_form: y = 5760 everywhere, by
    # hand; the GPU gets it exactly (and the intermediates the hand values)
    from oracle.formats import bf16_to_f32
    from test_oracle_closed_form import _layer
    x, ids, wts, w13q, w13sf, w13a, w2q, w2sf, w2a = _layer()
    L = dict(x=x, ids=ids, wts=wts, w13q=w13q, w13sf=w13sf, w13a=w13a, w2q=w2q, w2sf=w2sf, w2a=w2a)
    g = run_gpu_layer(nv, L)
    assert (bf16_to_f32(g["y"]) == 5760.0).all(), np.unique(bf16_to_f32(g["y"]))
    act = bf16_to_f32(g["act"]).astype(np.float64)
    slot = g["sorted_slot"][:act.shape[0]]
    assert (act[slot % 2 == 0] == 73728.0).all() and (act[slot % 2 == 1] == 36864.0).all()
    assert g["gs2"] == np.float32(73728.0) / np.float32(2688.0)


def test_concurrent_streams(nv):
    # the library keeps no per-call state outside the workspace: two layers,
    # each with its own workspace, issued on two streams (default priority)
    # so that their kernels may overlap, give what they give one at a time
    import torch
    from conftest import to_dev, to_host
    from helpers import gpu_packed_weights
    runs = []
    for name, T, seed in (("cs1", 700, 61), ("cs2", 40, 62)):     # tiled and weight-streaming paths
        L = make_layer(W.small_layer(name, T=T, H=512, I=256, E=8, topk=4, seed=seed))
        pw = gpu_packed_weights(nv, L)
        d = {k: to_dev(L[k]) for k in ("x", "ids", "wts")}
        args = (d["x"], d["ids"], d["wts"], pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"], pw["w2a"])
        ref = to_host(nv.moe_forward(*args))
        ws = torch.empty((nv.moe_workspace_size(T, 512, 256, 8, 4),), dtype=torch.uint8, device="cuda")
        runs.append((args, ref, ws))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for rep in range(4):
        for i, (args, ref, ws) in enumerate(runs):
            with torch.cuda.stream(streams[i]):
                outs[i].append(nv.moe_forward(*args, workspace=ws))
    torch.cuda.synchronize()
    for i, (args, ref, ws) in enumerate(runs):
        for y in outs[i]:
            assert (to_host(y) == ref).all(), f"stream {i}"


@pytest.mark.parametrize("static", [False, True])
def test_repeat_is_bit_identical_large_x(nv, static):
    # x above 128K elements: amax pass, then the quantization in the routing
    # launch beside the routing work-group; repeated calls agree bit for bit
    cfg = W.small_layer("repx", T=300, H=512, I=256, E=8, topk=4, seed=13)
    assert cfg.T * cfg.H > 1 << 17
    L = make_layer(cfg)
    if static:
        from oracle.formats import bf16_to_f32
        from oracle.quantize import global_scale
        L["x_gs"] = np.float32(global_scale(np.float32(np.abs(bf16_to_f32(L["x"])).max())) * np.float32(0.5))
    g = run_gpu_layer(nv, L, repeat=3)
    assert all((y == g["ys"][0]).all() for y in g["ys"])


# ---- degenerate and boundary cases -------------------------------------------

def test_empty_batch(nv):
    # T = 0: nothing to do, y is (0, H)
    import torch
    cfg = W.small_layer("empty", T=4, H=256, I=128, E=4, topk=2, seed=21)
    L = make_layer(cfg)
    from helpers import gpu_packed_weights
    pw = gpu_packed_weights(nv, L)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    wts = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    y = nv.moe_forward(x, ids, wts, pw["w13"], pw["w13_sf"], pw["w13a"], pw["w2"], pw["w2_sf"], pw["w2a"])
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 256)


def test_all_zero_input(nv):
    # x == 0: gs1 = 0, every scale byte and nibble 0, act = 0, gs2 = 0, y = +0
    cfg = W.small_layer("zero", T=40, H=256, I=128, E=4, topk=2, seed=22)
    L = make_layer(cfg)
    L["x"] = np.zeros_like(L["x"])
    g = run_gpu_layer(nv, L)
    r = run_oracle_layer(L)
    assert g["gs1"] == 0 and g["gs2"] == 0
    assert not g["xq"].any() and not g["xsf"].any()
    assert (g["y"] == 0).all()
    assert (r["y"] == 0).all()


def test_one_token_every_expert(nv):
    # top-k = E: the single token visits every expert once (weight streaming)
    cfg = W.small_layer("allexp", T=1, H=512, I=256, E=8, topk=8, seed=23)
    compare_layer(nv, make_layer(cfg), "one token, top-k = E")


def test_single_expert(nv):
    # E = 1, top-1: one expert, two 256-row tiles (256 + 44)
    cfg = W.small_layer("oneexp", T=300, H=256, I=128, E=1, topk=1, seed=24)
    compare_layer(nv, make_layer(cfg), "single expert")


def test_tile_boundaries(nv):
    # experts with exactly 256 and 257 slots: a full tile, and a full tile plus
    # a one-row tile
    cfg = W.small_layer("tiles", T=513, H=256, I=128, E=2, topk=1, seed=25)
    L = make_layer(cfg)
    ids = np.zeros((513, 1), np.int32)
    ids[256:] = 1
    L["ids"] = ids
    g, _, _ = compare_layer(nv, L, "tile boundaries")
    assert list(g["counts"]) == [256, 257]


@pytest.mark.parametrize("T", [32, 33])
def test_path_switch_boundary(nv, T):
    # S = 16 * E takes the weight-streaming kernels, one more slot the tiled GEMM
    cfg = W.small_layer(f"switch{T}", T=T, H=512, I=256, E=4, topk=2, seed=26 + T)
    compare_layer(nv, make_layer(cfg), f"path switch T={T}")


def test_tile_row_block_variants(nv):
    # the GEMM sizes each tile to 64-row multiples of its row count: experts
    # with 427 (256 + 171), 150, 64 and 65 slots take tiles of 4, 3, 1 and 2
    # row blocks per wave
    counts = [427, 150, 64, 65]
    T = sum(counts)
    cfg = W.small_layer("mi", T=T, H=512, I=256, E=4, topk=1, seed=27)
    L = make_layer(cfg)
    L["ids"] = np.repeat(np.arange(4, dtype=np.int32), counts)[np.random.default_rng(27).permutation(T)][:, None]
    g, _, _ = compare_layer(nv, L, "tile row-block variants")
    assert list(g["counts"]) == counts


def _exact_gate_up_layer(T, E, I, seed):
    """A layer whose gate and up values are single exact products on both
    sides: x has one nonzero per row (column 0, so each gate/up element is
    x̂[t, 0] · ŵ[0, n]), gs1 = 1 (x amax 2688) and every w13 alpha = 2^-10
    (w13 amax 2.625), so the float32 accumulation and the alpha scaling are
    exact and g, u reach the SiLU bit-identical to the oracle's. act must
    then match bit for bit: this pins the correctly rounded SiLU·up."""
    from oracle.formats import bf16_from_f64
    from oracle.quantize import quantize_weight_bf16
    rng = np.random.default_rng(seed)
    H = 16
    xv = np.zeros((T, H))
    xv[:, 0] = rng.choice([-1.0, 1.0], T) * 2.0 ** rng.uniform(-3, 6, T)
    xv[0, 0] = 2688.0
    L = dict(x=bf16_from_f64(xv),
             ids=(np.arange(T) % E).astype(np.int32)[:, None],
             wts=np.ones((T, 1), np.float32))
    w13q = np.zeros((E, H // 2, 2 * I), np.uint8)
    w13sf = np.zeros((E, H // 16, 2 * I), np.uint8)
    w2q = np.zeros((E, I // 2, H), np.uint8)
    w2sf = np.zeros((E, I // 16, H), np.uint8)
    w13a = np.zeros(E, np.float32)
    w2a = np.zeros(E, np.float32)
    for e in range(E):
        w13 = rng.uniform(-1.0, 1.0, (H, 2 * I)) * 2.625
        w13[0, 0] = 2.625
        w13q[e], w13sf[e], w13a[e] = quantize_weight_bf16(bf16_from_f64(w13))
        w2q[e], w2sf[e], w2a[e] = quantize_weight_bf16(bf16_from_f64(rng.standard_normal((I, H)) * 0.02))
    assert (w13a == np.float32(2.0 ** -10)).all()
    L.update(w13q=w13q, w13sf=w13sf, w13a=w13a, w2q=w2q, w2sf=w2sf, w2a=w2a)
    return L


@pytest.mark.parametrize("T,E,I", [(256, 1, 256), (512, 2, 320), (96, 8, 256)])
def test_silu_up_bit_exact_on_exact_gate_up(nv, T, E, I):
    # (256, 1): 256-row MFMA tiles; (512, 2): two experts, partial N tile;
    # (96, 8): 12 slots per expert, the weight-streaming path
    L = _exact_gate_up_layer(T, E, I, seed=T + E)
    g, r, _ = compare_layer(nv, L, f"exact gate/up T{T} E{E} I{I}", min_act_exact=1.0)
    assert g["gs1"] == np.float32(1.0)
    gu = r["gu"][:, 0, :]
    gate = gu[:, :I]
    # the inputs reach the float64 fallback's regions: gates below -87 and
    # gates so large that silu(g) * u rounds like the plain product g * u
    assert (gate < -87).any() and (gate > 17).any()
