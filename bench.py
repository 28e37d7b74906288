"""Benchmark of the NVFP4 expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one nvfp4_moe_forward (quantize x, route, L1 grouped GEMM with fused
SiLU*up, requantize, L2 grouped GEMM, weighted combine) over the prefill batch:
4096 tokens, hidden 7168, intermediate 3072, 48 local experts, top-8, x bf16
N(0,1)*3 with 0.1% outliers at +-40, router logits N(0,1), softmax-renormalized
top-8 weights, weights bf16 N(0, 0.02) quantized with the NVFP4 weight rule by
the library's own nvfp4_quantize_weights. Inputs are synthetic and resident in
HBM before the timed region starts.

The JSON line reports tokens/s (value), effective TFLOP/s (6 * slots * H * I per
step), per-stage device times from HIP events recorded by the library on its
stream, the L1 and L2 GEMMs' MFMA roofline fractions, and beside them the other
configurations of the recipe: the skewed prefill batch (8192 tokens), the dense
single-expert GEMM (256 x 7168 x 6144), the decode batch (8 tokens, weight HBM
GB/s, cycling through eight seeded routings), and the CPU oracle timed on the
whole prefill workload on this host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_MFMA_TFLOPS = 2500.0     # MI355X dense f16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "l1_gemm_prefill_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode batch (profiling runs)")
    ap.add_argument("--only", choices=("prefill", "skewed", "dense", "decode", "vendor-gemm"), default=None,
                    help="run one measurement and print its JSON (profiling runs)")
    ap.add_argument("--no-graph", action="store_true", help="decode: skip the HIP-graph timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for PMC byte-counter scaling)")
    return ap.parse_args()


def gemm_source_hash():
    """Hash of the GEMM kernel's sources (and of the routing kernel, which
    orders its tiles) with comments and blank space removed:
    the stored PMC traffic is reported only while this matches, i.e. until the
    code (not its commentary) changes."""
    import re
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp", "launch.hpp", "route.hip"):     # route.hip: the tile order
        with open(os.path.join(ROOT, "nvfp4_block_scaled_quant_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def make_weights(nv, cfg):
    """Per-expert bf16 weights from the workload recipe, quantized on the GPU
    (canonical layout) and prepacked once into the layout the GEMMs read."""
    import torch
    import workloads as W
    E, H, I = cfg.E, cfg.H, cfg.I
    s13, s13f = nv.packed_shapes(E, H, 2 * I)
    s2, s2f = nv.packed_shapes(E, I, H)
    w13 = torch.empty(s13, dtype=torch.uint8, device="cuda")
    w13sf = torch.empty(s13f, dtype=torch.uint8, device="cuda")
    w2 = torch.empty(s2, dtype=torch.uint8, device="cuda")
    w2sf = torch.empty(s2f, dtype=torch.uint8, device="cuda")
    w13a = torch.empty((E,), dtype=torch.float32, device="cuda")
    w2a = torch.empty((E,), dtype=torch.float32, device="cuda")
    for e in range(E):
        w13_bf16, w2_bf16 = W.expert_weights_bf16(cfg, e)
        q, sf, a = nv.quantize_weights(to_dev(w13_bf16)[None])
        q_t, sf_t = nv.prepack_weights(q, sf)
        w13[e], w13sf[e], w13a[e] = q_t[0], sf_t[0], a[0]
        q, sf, a = nv.quantize_weights(to_dev(w2_bf16)[None])
        q_t, sf_t = nv.prepack_weights(q, sf)
        w2[e], w2sf[e], w2a[e] = q_t[0], sf_t[0], a[0]
    if cfg.alpha_loguniform:
        a13, a2 = W.alphas_loguniform(cfg)
        w13a.copy_(torch.from_numpy(a13))
        w2a.copy_(torch.from_numpy(a2))
    torch.cuda.synchronize()
    return w13, w13sf, w13a, w2, w2sf, w2a


def time_layer(nv, cfg, weights, steps, warmup, events_in_loop=True, variant=None, routings=1):
    """Run warmup + timed steps; return (ms per step, per-stage ms, S_valid,
    the ids of every routing used, whether y is finite).

    routings: how many seeded routings (logit draws of the config's recipe
    with seeds seed_x, seed_x + 1, ...) the steps cycle through, so that a
    small batch does not touch the same experts in every step.

    variant: None (the layer as specified), "static_x" (nvfp4_moe_forward_ex
    with a static gs1, set to the value the dynamic rule gives for this x, so
    the numbers are the same and only the amax pass is gone) or "per_half"
    (w13 alphas of shape (E, 2), both halves equal to the per-expert alpha).

    events_in_loop: the stage events are recorded in every timed step (the
    per-stage device times then cover exactly the timed region). Otherwise
    the timed loop runs without them, and the stage times come from ten
    extra steps afterwards: for short steps the event records themselves are
    a visible part of the step time."""
    import numpy as np
    import torch
    import workloads as W
    import dataclasses
    x = to_dev(W.activations(cfg))
    routes = [W.routing(dataclasses.replace(cfg, seed_x=cfg.seed_x + r)) for r in range(routings)]
    ids_np = np.stack([r[0] for r in routes])
    dev_routes = [(to_dev(i), to_dev(w)) for i, w in routes]
    s_valid = int(((ids_np[0] >= 0) & (ids_np[0] < cfg.E)).sum())
    ws = torch.empty((nv.moe_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk),),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    x_gs = None
    if variant == "static_x":
        x_gs = nv.quantize(x)[2]
    elif variant == "per_half":
        w13, w13sf, w13a, w2, w2sf, w2a = weights
        weights = (w13, w13sf, torch.stack([w13a, w13a], dim=1).contiguous(), w2, w2sf, w2a)

    def step(i, ev=None):
        ids, wts = dev_routes[i % routings]
        nv.moe_forward(x, ids, wts, *weights, y=y, workspace=ws, stage_events=ev, x_gs=x_gs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    events = [nv.StageEvents() for _ in range(steps if events_in_loop else min(steps, 10))]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, events[i] if events_in_loop else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not events_in_loop:
        for i, ev in enumerate(events):
            step(i, ev)
        torch.cuda.synchronize()
    per = [ev.elapsed_ms() for ev in events]
    stage_ms = {k: float(np.mean([p[k] for p in per])) for k in per[0]}
    # device time of each step with events: first event to last
    step_ms = [float(sum(p.values())) for p in per]
    ok = bool(torch.isfinite(y.float()).all().item())
    return (t1 - t0) * 1e3 / steps, stage_ms, s_valid, ids_np, ok, step_ms


def time_router(nv, cfg, launches=200):
    """Microseconds per nvfp4_route_topk launch on the config's logits (T, E),
    top-k, timed with events on torch's current stream (the one the binding
    launches on)."""
    import numpy as np
    import torch
    import workloads as W
    rng = np.random.default_rng(cfg.seed_x)
    logits = to_dev((rng.standard_normal((cfg.T, cfg.E)) + W.zipf_bias(cfg)[None, :]).astype(np.float32))
    ids = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device="cuda")
    wts = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device="cuda")
    for _ in range(10):
        nv.route_topk(logits, cfg.topk, ids, wts)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        nv.route_topk(logits, cfg.topk, ids, wts)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / launches


def decode_bytes(cfg, ids_np):
    """Algorithmic HBM bytes of one decode step, averaged over the routings in
    ids_np (R, T, topk): every touched expert's w13 and w2 bytes and scales,
    plus x, y, the routing arrays and the intermediates. Returns (bytes, mean
    number of touched experts)."""
    import numpy as np
    H, I, E = cfg.H, cfg.I, cfg.E
    per_expert = (H // 2) * 2 * I + (H // 16) * 2 * I + (I // 2) * H + (I // 16) * H
    touched = float(np.mean([len(np.unique(r[(r >= 0) & (r < E)])) for r in ids_np]))
    S = cfg.T * cfg.topk
    act = S * I * 2 * 2 + S * (I // 2 + I // 16) * 2 + S * H * 4 * 2
    return touched * per_expert + cfg.T * H * 2 * 2 + act, touched


def time_decode(nv, weights, steps, routings=8, graph=True):
    """The decode batch (8 tokens, top-8 of 48) cycling through `routings`
    seeded routings, so that consecutive steps touch different expert sets;
    bytes are the routings' mean algorithmic weight bytes."""
    import workloads as W
    dcfg = W.DECODE
    dms, dstage, _, dids, dfin, _ = time_layer(nv, dcfg, weights, steps, 5, events_in_loop=False,
                                            routings=routings)
    nbytes, touched = decode_bytes(dcfg, dids)
    g_us = time_decode_graph(nv, weights, routings=routings) if graph else None
    return {"workload": "decode", "tokens": dcfg.T, "routings": routings, "us_per_step": dms * 1e3,
            "graph_us_per_step": g_us, "graph_GBps": nbytes / (g_us * 1e-6) / 1e9 if g_us else None,
            "graph_hbm_frac": nbytes / (g_us * 1e-6) / 1e9 / PEAK_HBM_GBPS if g_us else None,
            "touched_experts_mean": touched, "algorithmic_bytes_mean": nbytes,
            "GBps": nbytes / (dms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "stage_us": {k: v * 1e3 for k, v in dstage.items()},
            "finite": dfin}


def time_decode_graph(nv, weights, replays=50, routings=8):
    """The decode batch captured in one HIP graph: the eight seeded routings'
    nvfp4_moe_forward_noalloc calls (the allocation-free entry point,
    workspace in the library's static scratch) one after another, as a decode
    loop would capture a run of layers; the graph is replayed `replays`
    times and timed with events on torch's current stream. Returns
    microseconds per layer call."""
    import dataclasses
    import torch
    import workloads as W
    dcfg = W.DECODE
    x = to_dev(W.activations(dcfg))
    y = torch.empty((dcfg.T, dcfg.H), dtype=torch.bfloat16, device="cuda")
    routes = [tuple(to_dev(a) for a in W.routing(dataclasses.replace(dcfg, seed_x=dcfg.seed_x + r)))
              for r in range(routings)]
    nv.moe_forward_noalloc(x, *routes[0], *weights, y=y)      # set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for ids, wts in routes:
            nv.moe_forward_noalloc(x, ids, wts, *weights, y=y)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * routings)


def time_skewed(nv, weights, steps, warmup):
    """The skewed prefill batch (8192 tokens, Zipf-biased top-8 routing that
    leaves experts empty, log-uniform per-expert alphas in [1e-4, 1e-2]) on the
    same quantized weights with the config's alphas."""
    import torch
    import workloads as W
    scfg = W.SKEWED
    w13, w13sf, _, w2, w2sf, _ = weights
    a13, a2 = W.alphas_loguniform(scfg)
    sw = (w13, w13sf, torch.from_numpy(a13).cuda(), w2, w2sf, torch.from_numpy(a2).cuda())
    ms, stage, s_valid, ids_np, fin, step_ms = time_layer(nv, scfg, sw, steps, warmup)
    import numpy as np
    counts = np.bincount(ids_np[0].ravel(), minlength=scfg.E)
    l1_flops = 2.0 * s_valid * scfg.H * 2 * scfg.I
    return {"workload": "skewed prefill", "tokens": scfg.T, "slots": s_valid, "ms_per_step": ms,
            "tokens_per_s": scfg.T / (ms * 1e-3),
            "eff_tflops": 6.0 * s_valid * scfg.H * scfg.I / (ms * 1e-3) / 1e12,
            "l1_f16_peak_frac": l1_flops / (stage["l1"] * 1e-3) / 1e12 / PEAK_F16_MFMA_TFLOPS,
            "l2_f16_peak_frac": l1_flops / 2 / (stage["l2"] * 1e-3) / 1e12 / PEAK_F16_MFMA_TFLOPS,
            "stage_ms": stage,
            "step_ms_device": {"median": float(np.median(step_ms)), "min": float(np.min(step_ms))},
            "empty_experts": int((counts == 0).sum()),
            "hottest_expert_slot_share": float(counts.max() / counts.sum()), "finite": fin}


def time_dense_gemm(nv, launches=50):
    """The single-expert dense GEMM (M 256, K 7168, N 6144): A quantized from
    bf16 N(0,1)*3, B from N(0,0.02) by the library, prepacked; each timed
    nvfp4_gemm call converts A to its f16 form and runs the GEMM. Timed with
    events on torch's current stream (the binding launches there)."""
    import torch
    import workloads as W
    cfg = W.DENSE
    a, b = W.dense_gemm_inputs(cfg)
    aq, asf, ags = nv.quantize(to_dev(a))
    bq, bsf, balpha = nv.quantize_weights(to_dev(b)[None])
    bq_t, bsf_t = nv.prepack_weights(bq, bsf)
    out = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((nv._lib.nvfp4_gemm_workspace(cfg.M, cfg.N, cfg.K),), dtype=torch.uint8, device="cuda")
    for _ in range(10):
        nv.gemm(aq, asf, ags, bq_t[0], bsf_t[0], balpha, out=out, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        nv.gemm(aq, asf, ags, bq_t[0], bsf_t[0], balpha, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    flop = 2.0 * cfg.M * cfg.N * cfg.K
    wbytes = cfg.K * cfg.N // 2 + cfg.K // 16 * cfg.N
    return {"workload": "dense GEMM M 256 x K 7168 x N 6144", "us_per_call": us,
            "tflops": flop / (us * 1e-6) / 1e12, "f16_peak_frac": flop / (us * 1e-6) / 1e12 / PEAK_F16_MFMA_TFLOPS,
            "weight_GBps": wbytes / (us * 1e-6) / 1e9,
            "note": "the 24.8 MB weight operand stays resident in the last-level cache across calls"}


def _oracle_expert_weights(args):
    """Worker: one expert's weights quantized with the oracle's rule."""
    import workloads as W
    from oracle.quantize import quantize_weight_bf16
    cfg, e = args
    w13, w2 = W.expert_weights_bf16(cfg, e)
    return e, quantize_weight_bf16(w13), quantize_weight_bf16(w2)


def cpu_baseline(cfg, experts=tuple(range(48))):
    """The oracle's layer forward timed on the prefill workload: all T tokens'
    x and the slots routed to `experts` (by default all 48, i.e. the whole
    workload; the other slots would be skipped), with those experts' weights
    quantized by the oracle beforehand (untimed, in spawned worker processes).
    Reported as token-equivalents per second: sample slots / topk / seconds."""
    import multiprocessing as mp
    import numpy as np
    import workloads as W
    from oracle.moe import moe_forward
    x = W.activations(cfg)
    ids, wts = W.routing(cfg)
    keep = np.isin(ids, experts)
    ids_s = np.where(keep, ids, -1).astype(np.int32)
    E, H, I = cfg.E, cfg.H, cfg.I
    w13q = np.zeros((E, H // 2, 2 * I), np.uint8)
    w13sf = np.zeros((E, H // 16, 2 * I), np.uint8)
    w2q = np.zeros((E, I // 2, H), np.uint8)
    w2sf = np.zeros((E, I // 16, H), np.uint8)
    w13a = np.zeros(E, np.float32)
    w2a = np.zeros(E, np.float32)
    nproc = max(1, min(len(experts), 16, len(os.sched_getaffinity(0))))
    with mp.get_context("spawn").Pool(nproc) as pool:
        for e, (q1, s1, a1), (q2, s2, a2) in pool.imap_unordered(
                _oracle_expert_weights, [(cfg, e) for e in experts]):
            w13q[e], w13sf[e], w13a[e] = q1, s1, a1
            w2q[e], w2sf[e], w2a[e] = q2, s2, a2
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    t0 = time.perf_counter()
    moe_forward(x, ids_s, wts, w13q, w13sf, w13a, w2q, w2sf, w2a)
    dt = time.perf_counter() - t0
    slots = int(keep.sum())
    cores = len(os.sched_getaffinity(0))
    return {"value": slots / cfg.topk / dt, "unit": "tokens/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle", "seconds": dt,
            "sample": (f"prefill workload (T={cfg.T}, H={H}, I={I}, E={E}, top-{cfg.topk}): all "
                       f"tokens' x quantized, the {slots} slots routed to experts "
                       f"{experts[0]}..{experts[-1]} run through L1/SiLU/requant/L2/combine"
                       f"{' (the whole workload)' if len(experts) == E else ''}; value = slots/topk "
                       f"per second (token-equivalents); float64 BLAS matmuls multithreaded, the "
                       f"rest single-threaded NumPy; the oracle's weight quantization is not timed")}


def calibrate_copy():
    """Device copies of 1 GiB and of 256 MiB (three each), whose PMC byte
    counters give the scaling of FETCH_SIZE and WRITE_SIZE to bytes."""
    import torch
    for n in (1 << 30, 1 << 28):
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 3}))
        del a, b


def _vendor_rate(a, b, flop, reps):
    import torch
    c = torch.matmul(a, b)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del c
    tf = flop / (us * 1e-6) / 1e12
    return {"us_per_call": us, "tflops": tf, "f16_peak_frac": tf / PEAK_F16_MFMA_TFLOPS}


def _exact_f16(nv, x_bf16):
    """The exact f16 values code * E4M3 scale of the NVFP4 quantization of the
    rows of x (global scale left out, as in the GEMMs' f16 operands)."""
    import torch
    q, sf, _ = nv.quantize(x_bf16)
    lut = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6], device=q.device)
    codes = torch.stack([lut[(q & 15).long()], lut[(q >> 4).long()]], dim=-1).reshape(x_bf16.shape[0], -1)
    return (codes * sf.view(torch.float8_e4m3fn).float().repeat_interleave(16, dim=1)).half()


def vendor_f16_gemm(nv, reps=20):
    """torch.matmul (hipBLASLt) f16 GEMMs as context for the L1/L2 fractions,
    not the peak: (1) n x n x n on normal-distributed f16 data; (2) the L1
    GEMM's flops as one dense GEMM (M = T * topk rows of the quantized layer
    input, each token's row repeated topk times; N = 2I; K = H; one expert's
    quantized w13 as B, K-major like the packed weights) on the exact f16
    values of the NVFP4 operands. The operand values change the power the
    matrix cores draw and so the clock the chip holds under its power limit."""
    import torch
    import workloads as W
    cfg = W.PREFILL
    out = {}
    g = torch.Generator(device="cuda").manual_seed(5)
    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.float16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.float16, generator=g)
    out["square_normal"] = {"shape": f"{n} x {n} x {n}, normal f16 data, f32 accumulate",
                            **_vendor_rate(a, b, 2.0 * n ** 3, reps)}
    del a, b
    x = to_dev(W.activations(cfg))
    a = _exact_f16(nv, x).repeat_interleave(cfg.topk, dim=0).contiguous()
    w13_bf16, _ = W.expert_weights_bf16(cfg, 0)
    bt = _exact_f16(nv, to_dev(w13_bf16).t().contiguous())             # (2I, H): B, K-major
    M, K, N = a.shape[0], a.shape[1], bt.shape[0]
    out["l1_shape_nvfp4_values"] = {
        "shape": f"{M} x {N} x {K} (M x N x K), exact f16 values of NVFP4 operands, B K-major, f32 accumulate",
        **_vendor_rate(a, bt.t(), 2.0 * M * N * K, reps)}
    del a, bt, x
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the layer is measured on one GPU's share of experts; --gpus {args.gpus} "
              f"is not supported (only --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import nvfp4_block_scaled_quant_amd as nv
    import workloads as W
    if args.only == "vendor-gemm":
        print(json.dumps(vendor_f16_gemm(nv)), flush=True)
        return

    cfg = W.PREFILL
    t_setup = time.perf_counter()
    weights = make_weights(nv, cfg)
    setup_s = time.perf_counter() - t_setup
    if args.decode_only or args.only == "decode":
        print(json.dumps(time_decode(nv, weights, args.decode_steps, graph=not args.no_graph)), flush=True)
        return
    if args.only == "skewed":
        print(json.dumps(time_skewed(nv, weights, args.steps, args.warmup)), flush=True)
        return
    if args.only == "dense":
        print(json.dumps(time_dense_gemm(nv)), flush=True)
        return
    if args.only == "prefill":
        ms, stage_ms, _, _, _, _ = time_layer(nv, cfg, weights, args.steps, args.warmup)
        print(json.dumps({"workload": "prefill", "ms_per_step": ms, "stage_ms": stage_ms}), flush=True)
        return
    ms, stage_ms, s_valid, ids_np, finite, step_ms = time_layer(nv, cfg, weights, args.steps, args.warmup)
    flops = 6.0 * s_valid * cfg.H * cfg.I
    l1_flops = 2.0 * s_valid * cfg.H * 2 * cfg.I
    l1_tflops = l1_flops / (stage_ms["l1"] * 1e-3) / 1e12
    l2_tflops = (l1_flops / 2) / (stage_ms["l2"] * 1e-3) / 1e12

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("gemm_source_hash") == gemm_source_hash():
            traffic = tr.get("hbm_bytes_per_launch")

    out = {
        "metric": "NVFP4 MoE layer tokens/s + eff. TFLOP/s (prefill); weight HBM GB/s (decode)",
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3/16) operands, f16 MFMA, f32 accumulate, bf16 out",
        "data": "synthetic",
        "config": {"workload": "prefill", "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "topk": cfg.topk,
                   "slots": s_valid, "parallelism": "single GPU, one GPU's expert share"},
        "eff_tflops": flops / (ms * 1e-3) / 1e12,
        "f16_peak_frac_layer": flops / (ms * 1e-3) / 1e12 / PEAK_F16_MFMA_TFLOPS,
        "stage_ms": stage_ms,
        "step_ms_device": {"median": float(np.median(step_ms)), "min": float(np.min(step_ms)),
                           "note": "per timed step, first to last stage event on the library's stream"},
        "l2_gemm": {"kernel": "L2 grouped GEMM (gemm_kernel<2>)", "achieved_tflops": l2_tflops,
                    "f16_peak_frac": l2_tflops / PEAK_F16_MFMA_TFLOPS},
        "roofline": {"bound": "mfma", "kernel": "L1 grouped GEMM (gemm_kernel<1>)",
                     "achieved": l1_tflops, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": l1_tflops / PEAK_F16_MFMA_TFLOPS, "traffic": traffic,
                     "algorithmic_flop_per_launch": l1_flops,
                     "fp4_peak_frac": l1_tflops / 10100.0},
        "finite": finite,
        "setup_s": setup_s,
        "note": "the source pages publish no throughput figures, only correctness traces on "
                "their own (NVIDIA) hardware",
    }
    # extensions beyond the five stages, measured on the same prefill batch
    ext = {"router_us": {c.name: time_router(nv, c) for c in (W.PREFILL, W.SKEWED)}}
    for variant in ("static_x", "per_half"):
        vms, vstage, _, _, vfin, _ = time_layer(nv, cfg, weights, 10, 3, variant=variant)
        ext[variant] = {"ms_per_step": vms, "stage_ms": vstage, "finite": vfin}
    out["extensions"] = ext
    # the other configurations of the workload recipe, each measured the same way
    out["skewed"] = time_skewed(nv, weights, args.steps, 3)
    out["dense_gemm"] = time_dense_gemm(nv)
    out["vendor_f16_gemm"] = vendor_f16_gemm(nv)
    if not args.no_decode:
        out["decode"] = time_decode(nv, weights, args.decode_steps)
    del weights
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
