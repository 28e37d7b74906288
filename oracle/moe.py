"""The five-stage NVFP4 mixture-of-experts expert layer (test infrastructure).

Stages as the pages list them (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline"):

1. ``stage_activation(hidden)``: quantize x with the NVFP4 rule (oracle.quantize),
   one global scale gs1 over all of x;
2. token-to-expert permutation: one slot per (token t, choice j) whose expert id
   lies in [0, E); ids outside that range are skipped (the pages do not define
   them; this is the reading taken);
3. L1 GEMM of each slot's quantized row against w13[e] = [gate; up] with
   alpha = gs1 * w13_alpha[e]; gate is the first I output columns, up the last I
   (src commit log, gate/up interleave removal);
4. act = SiLU(gate) * up, then ``stage_activation(act)``: one global scale gs2
   over the activations of all valid slots;
5. L2 GEMM with alpha = gs2 * w2_alpha[e], then the routing-weighted scatter
   of the L2 rows back to their tokens:
   y[t] = sum_j topk_weights[t, j] * out[t, j] in j order.

Rounding points (the pages print bf16-looking intermediates and a bf16
output; these are the readings taken): gate_up is rounded to bf16 before SiLU
(R1); act is rounded to bf16 once (R2); nothing between the L2 sum and y is
rounded except the single final bf16 rounding of y (R3). Everything else here
is float64, and SiLU(z) = z / (1 + exp(-z)).

Parity: each stage is pinned through the modules it calls (formats, quantize,
gemm). The pages never reach a correct layer output, so no published value
pins the layer end to end; instead a layer worked out by hand
(tests/test_oracle_closed_form.py: constant inputs, every quantization exact,
y = 5760) pins it, and the composition is checked by the invariants in
tests/test_oracle_moe.py (gate/up split, per-expert alpha, skipped slots,
slot-order independence, the pure-Python twin on the tiny layer).
"""
import numpy as np

from .formats import bf16_from_f64, bf16_to_f32
from .quantize import (dequantize_cols, dequantize_rows, quantize_bf16,
                       quantize_bf16_static, quantize_f32)


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_mul_bf16(g_bits, u_bits):
    """act = bf16(silu(g) * u) for bf16 inputs g, u (R2), rounded to nearest
    even from the exact value.

    The float64 value silu(g) * u decides the rounding, with one exception:
    where 1 + exp(-g) rounds to 1 in float64 (g above about 36.7) it is the
    plain product g * u (at most 16 significant bits, exact), while the exact
    value g * u / (1 + e^-g) is smaller in magnitude by a factor within 2^-53
    of 1. If that product is a bf16 rounding midpoint the exact value lies just
    inside it, so it must round toward zero; elsewhere the tiny factor cannot
    move the result across a rounding boundary. The float64 value is therefore
    moved one float64 step toward zero in that case before the rounding.
    """
    g = bf16_to_f32(g_bits).astype(np.float64)
    u = bf16_to_f32(u_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        den = 1.0 + np.exp(-g)
    v = g / den * u
    exact_product = (den == 1.0) & (v != 0) & np.isfinite(v)
    v = np.where(exact_product, np.nextafter(v, 0.0), v)
    return bf16_from_f64(v)


def slots_by_expert(topk_ids, num_experts):
    """For each expert, the (token, choice) pairs routed to it, in (t, j) order."""
    ids = np.asarray(topk_ids)
    out = []
    for e in range(num_experts):
        t_idx, j_idx = np.nonzero(ids == e)
        out.append((t_idx, j_idx))
    return out


def _l1_expert(task):
    """L1 rows of one expert and the SiLU half of stage 4 (R1, R2)."""
    xq_rows, xsf_rows, w13q_e, w13sf_e, alpha, I, keep = task
    a = dequantize_rows(xq_rows, xsf_rows)
    b = dequantize_cols(w13q_e, w13sf_e)
    ab = a @ b
    # alpha: one value for all 2I columns, or (gate, up) one per half
    ag, au = (alpha, alpha) if np.ndim(alpha) == 0 else (alpha[0], alpha[1])
    gu_f64 = np.concatenate([ag * ab[:, :I], au * ab[:, I:]], axis=1)
    gu = bf16_from_f64(gu_f64)                                       # R1
    return silu_mul_bf16(gu[:, :I], gu[:, I:]), (gu_f64 if keep else None)   # R2


def _l2_expert(task):
    """Weighted L2 rows of one expert, float64."""
    aq_rows, asf_rows, w2q_e, w2sf_e, alpha, w = task
    a = dequantize_rows(aq_rows, asf_rows)
    b = dequantize_cols(w2q_e, w2sf_e)
    return w[:, None] * (alpha * (a @ b))


def _map(fn, tasks, pool):
    """Per-expert work, in order; `pool` (anything with .map) spreads it."""
    return pool.map(fn, tasks) if pool is not None else [fn(t) for t in tasks]


def moe_forward(x_bits, topk_ids, topk_weights, w13q, w13sf, w13_alpha,
                w2q, w2sf, w2_alpha, keep=False, pool=None, x_gs=None):
    """Reference layer output.

    Shapes: x_bits (T, H) uint16 bf16 bits; topk_ids (T, k) int; topk_weights
    (T, k) float32; w13q (E, H/2, 2I) uint8; w13sf (E, H/16, 2I) uint8;
    w13_alpha (E,) float32, or (E, 2) for per-half weight global scales (gate,
    up: column part p of w13[e] is scaled by gs1 * w13_alpha[e, p]);
    w2q (E, I/2, H); w2sf (E, I/16, H); w2_alpha (E,).

    x_gs: None for the dynamic activation scale gs1 = amax(x) / 2688, or a
    float32 static scale used as gs1 (oracle.quantize.quantize_f32_static).

    Returns a dict with y (float64, unrounded), y_bits (bf16) and, when keep is
    set, the per-slot intermediates indexed [t, j]: gu (float64, unrounded),
    act_bits (bf16, T x k x I), aq, asf, contrib (weighted L2 rows, float64),
    valid mask, plus xq, xsf, gs1, gs2.

    `pool` (e.g. a multiprocessing pool) only distributes the per-expert GEMMs;
    the arithmetic is the same with or without it.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(topk_ids).astype(np.int64)
    T, H = x_bits.shape
    k = ids.shape[1] if ids.ndim == 2 else 0
    E = w13q.shape[0]
    I = w2q.shape[1] * 2

    # stage 1
    if x_gs is None:
        xq, xsf, gs1 = quantize_bf16(x_bits)
    else:
        xq, xsf, gs1 = quantize_bf16_static(x_bits, x_gs)

    # stage 2
    groups = slots_by_expert(ids, E)
    valid = (ids >= 0) & (ids < E)

    # stage 3 + the SiLU half of stage 4
    act_bits = np.zeros((T, k, I), dtype=np.uint16)
    gu_keep = np.zeros((T, k, 2 * I), dtype=np.float64) if keep else None
    w13a = np.asarray(w13_alpha, dtype=np.float32).astype(np.float64)
    tasks = [(xq[t_idx], xsf[t_idx], w13q[e], w13sf[e],
              np.float64(gs1) * w13a[e], I, keep)
             for e, (t_idx, j_idx) in enumerate(groups) if t_idx.size]
    placed = [(t_idx, j_idx) for t_idx, j_idx in groups if t_idx.size]
    for (t_idx, j_idx), (act_e, gu_e) in zip(placed, _map(_l1_expert, tasks, pool)):
        act_bits[t_idx, j_idx] = act_e
        if keep:
            gu_keep[t_idx, j_idx] = gu_e

    # the requantization half of stage 4: one gs2 over all valid slots
    t_all, j_all = np.nonzero(valid)
    aq = np.zeros((T, k, I // 2), dtype=np.uint8)
    asf = np.zeros((T, k, I // 16), dtype=np.uint8)
    if t_all.size:
        q_v, sf_v, gs2 = quantize_bf16(act_bits[t_all, j_all])
        aq[t_all, j_all] = q_v
        asf[t_all, j_all] = sf_v
    else:
        gs2 = np.float32(0.0)

    # stage 5: L2 and the weighted combine, float64 until the final rounding
    y, contrib = l2_combine(aq, asf, gs2, ids, topk_weights, w2q, w2sf, w2_alpha, pool=pool)
    out = {"y": y, "y_bits": bf16_from_f64(y), "gs1": gs1, "gs2": np.float32(gs2)}
    if keep:
        out.update(xq=xq, xsf=xsf, gu=gu_keep, act_bits=act_bits, aq=aq, asf=asf,
                   valid=valid, contrib=contrib)
    return out


def l2_combine(aq, asf, gs2, topk_ids, topk_weights, w2q, w2sf, w2_alpha, pool=None):
    """Stage 5 on given requantized activations: the L2 GEMM of each valid
    slot's row against w2[e] with alpha = gs2 * w2_alpha[e], then y[t] = sum
    over j, in j order, of topk_weights[t, j] times that row (float64, left
    unrounded). aq (T, k, I/2) and asf (T, k, I/16) are indexed by (token,
    choice); rows of skipped slots are not read.

    Returns (y (T, H) float64, contrib (T, k, H) float64 weighted L2 rows).
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    E = w2q.shape[0]
    H = w2q.shape[2]
    groups = slots_by_expert(ids, E)
    placed = [(t_idx, j_idx) for t_idx, j_idx in groups if t_idx.size]
    contrib = np.zeros((T, k, H), dtype=np.float64)
    tasks = [(aq[t_idx, j_idx], asf[t_idx, j_idx], w2q[e], w2sf[e],
              np.float64(np.float32(gs2)) * np.float64(np.float32(w2_alpha[e])), wts[t_idx, j_idx])
             for e, (t_idx, j_idx) in enumerate(groups) if t_idx.size]
    for (t_idx, j_idx), rows in zip(placed, _map(_l2_expert, tasks, pool)):
        contrib[t_idx, j_idx] = rows
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(k):                                               # j order
        y += contrib[:, j, :]
    return y, contrib


def quantize_act_rows(act_bits):
    """Stage-4 quantization on its own: rows of bf16 activations."""
    return quantize_bf16(act_bits)


__all__ = ["moe_forward", "silu", "silu_mul_bf16", "slots_by_expert", "l2_combine",
           "quantize_act_rows", "quantize_f32"]
