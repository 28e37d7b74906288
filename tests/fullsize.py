"""Process-pool helpers for the full-size parity tests (test infrastructure).

The oracle is single-threaded NumPy apart from BLAS; at the layer's real size
(48 experts of 7168 x 6144 and 3072 x 7168 weights) its per-expert work is
spread over worker processes. Workers run only oracle and input-generator code
on the CPU (spawned, never forked from a process that holds a GPU context).
"""
import multiprocessing as mp
import os

import numpy as np


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def make_pool():
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    return mp.get_context("spawn").Pool(n, initializer=_init_worker)


def _quant_expert(args):
    import workloads as W
    from oracle.quantize import quantize_weight_bf16
    cfg, e = args
    w13, w2 = W.expert_weights_bf16(cfg, e)
    return e, quantize_weight_bf16(w13), quantize_weight_bf16(w2)


def oracle_weights(cfg, pool, experts=None):
    """All experts' weights quantized with the oracle's rule, in parallel."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w13q = np.zeros((E, H // 2, 2 * I), np.uint8)
    w13sf = np.zeros((E, H // 16, 2 * I), np.uint8)
    w2q = np.zeros((E, I // 2, H), np.uint8)
    w2sf = np.zeros((E, I // 16, H), np.uint8)
    w13a = np.zeros(E, np.float32)
    w2a = np.zeros(E, np.float32)
    todo = list(range(E)) if experts is None else list(experts)
    for e, (q1, s1, a1), (q2, s2, a2) in pool.imap_unordered(_quant_expert, [(cfg, e) for e in todo]):
        w13q[e], w13sf[e], w13a[e] = q1, s1, a1
        w2q[e], w2sf[e], w2a[e] = q2, s2, a2
    return dict(w13q=w13q, w13sf=w13sf, w13a=w13a, w2q=w2q, w2sf=w2sf, w2a=w2a)


def layer_inputs(cfg, weights):
    import workloads as W
    L = dict(weights)
    L["x"] = W.activations(cfg)
    L["ids"], L["wts"] = W.routing(cfg)
    if cfg.alpha_loguniform:
        L["w13a"], L["w2a"] = W.alphas_loguniform(cfg)
    return L
