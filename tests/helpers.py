"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerance reading (the target tolerance: GEMM and layer outputs within a max relative
error of 2e-3 of the oracle's fp64 accumulation, cosine >= 0.9999). A bf16
output carries its own rounding of up to half an ulp, which is up to 2^-8 ~
3.9e-3 of an element just above a power of two, so no bf16 output can meet a
literal 2e-3 bound against the unrounded value. The bound is therefore applied
to the arithmetic before the output's one mandated rounding:

    gpu_i must be the bf16 rounding of some value within 2e-3 * max|ref| of ref_i,

i.e. ref_i lies within the rounding interval of gpu_i widened by that amount.
A second, much tighter check proves the arithmetic error is below one bf16 ulp
wherever the element is not tiny: gpu_i is one of the two bf16 neighbours of
ref_i whenever |ref_i| >= 2^-6 * max|ref|.
"""
import numpy as np

from oracle.formats import bf16_from_f64, bf16_to_f32

REL_TOL = 2e-3
MIN_SUB = 2.0 ** -133


def bf16_neighbors(bits):
    """Values of the next bf16 below and above each pattern (finite inputs)."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = bits & 0x7FFF
    neg = (bits >> 15) == 1

    def val(m, negative):
        v = bf16_to_f32(m.astype(np.uint16)).astype(np.float64)
        return np.where(negative, -v, v)

    bigger = val(mag + 1, neg)                       # away from zero
    smaller = np.where(mag > 0, val(np.maximum(mag - 1, 0), neg),
                       np.where(neg, MIN_SUB, -MIN_SUB))   # toward / across zero
    up = np.where(neg, smaller, bigger)
    down = np.where(neg, bigger, smaller)
    return down, up


def check_bf16_output(gpu_bits, ref, name="out", tol=REL_TOL, faithful_floor=2.0 ** -6,
                      min_exact=0.99, faithful_rows=None, bound_rows=None, amax=None):
    """Assert the 2e-3 bound (as read above) on `bound_rows` of the first
    axis (all rows by default), faithful rounding for non-tiny elements of
    `faithful_rows`, and a high exact-match rate; return a stats dict. `amax`
    overrides max|ref| as the normalizer (when a subset of rows is checked)."""
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu_bits.shape == ref.shape, (gpu_bits.shape, ref.shape)
    g = bf16_to_f32(gpu_bits).astype(np.float64)
    assert np.isfinite(g).all(), f"{name}: non-finite output"
    if amax is None:
        amax = float(np.abs(ref).max()) if ref.size else 0.0
    down, up = bf16_neighbors(gpu_bits)
    lo = (g + down) / 2
    hi = (g + up) / 2
    slack = tol * amax
    bad = (ref < lo - slack) | (ref > hi + slack)
    if bound_rows is not None:
        bad &= np.asarray(bound_rows, bool).reshape((-1,) + (1,) * (ref.ndim - 1))
    stats = {
        "max_rel_literal": float(np.abs(g - ref).max() / amax) if amax > 0 else 0.0,
        "exact": float((gpu_bits == bf16_from_f64(ref)).mean()) if ref.size else 1.0,
        "cos": cosine(g, ref),
    }
    if amax > 0:
        beyond = np.maximum(lo - ref, ref - hi).clip(min=0)
        stats["max_rel_beyond_rounding"] = float(beyond.max() / amax)
        stats["beyond_rounding_rows"] = (beyond / amax).reshape(ref.shape[0], -1).max(axis=1)
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements beyond the bound; worst at "
                           f"{np.unravel_index(np.argmax(np.maximum(lo - ref, ref - hi)), ref.shape)}; {stats}")
    big = np.abs(ref) >= faithful_floor * amax
    if faithful_rows is not None:
        big &= np.asarray(faithful_rows, bool).reshape((-1,) + (1,) * (ref.ndim - 1))
    unfaithful = big & ((ref < down) | (ref > up))
    assert not unfaithful.any(), f"{name}: {int(unfaithful.sum())} non-tiny elements off by more than one ulp; {stats}"
    assert stats["exact"] >= min_exact, f"{name}: exact-match rate {stats['exact']:.4f}; {stats}"
    return stats


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    if na == 0 or nb == 0:
        return 0.0
    return float(a @ b / (na * nb))


def bf16_ulp_distance(a_bits, b_bits):
    """Number of bf16 steps between two patterns (monotone integer mapping)."""
    def key(b):
        b = np.asarray(b, np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(key(a_bits) - key(b_bits))


def make_layer(cfg, experts=None, w13_parts=1, up_scale=1.0):
    """Oracle-side inputs of a layer config: x, routing, weights quantized with
    the oracle's rule (O-Q along K). `experts` limits which experts get real
    weights (the others are zero and must be unused by the routing).
    w13_parts = 2 quantizes gate and up with their own global scales (w13a
    becomes (E, 2)); up_scale multiplies the up half of the bf16 weights first
    (a power of two keeps them exact)."""
    import workloads as W
    from oracle.quantize import quantize_weight_bf16, quantize_weight_bf16_parts
    x = W.activations(cfg)
    ids, wts = W.routing(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    w13q = np.zeros((E, H // 2, 2 * I), np.uint8)
    w13sf = np.zeros((E, H // 16, 2 * I), np.uint8)
    w2q = np.zeros((E, I // 2, H), np.uint8)
    w2sf = np.zeros((E, I // 16, H), np.uint8)
    w13a = np.zeros(E, np.float32) if w13_parts == 1 else np.zeros((E, w13_parts), np.float32)
    w2a = np.zeros(E, np.float32)
    for e in (range(E) if experts is None else experts):
        w13, w2 = W.expert_weights_bf16(cfg, e)
        if up_scale != 1.0:
            from oracle.formats import bf16_from_f64, bf16_to_f32
            f = bf16_to_f32(w13).astype(np.float64)
            f[:, I:] *= up_scale
            w13 = bf16_from_f64(f)
        if w13_parts == 1:
            w13q[e], w13sf[e], w13a[e] = quantize_weight_bf16(w13)
        else:
            w13q[e], w13sf[e], w13a[e] = quantize_weight_bf16_parts(w13, w13_parts)
        w2q[e], w2sf[e], w2a[e] = quantize_weight_bf16(w2)
    if cfg.alpha_loguniform:
        w13a, w2a = W.alphas_loguniform(cfg)
    return dict(x=x, ids=ids, wts=wts, w13q=w13q, w13sf=w13sf, w13a=w13a,
                w2q=w2q, w2sf=w2sf, w2a=w2a)


def run_oracle_layer(L, keep=True, pool=None):
    from oracle.moe import moe_forward
    return moe_forward(L["x"], L["ids"], L["wts"], L["w13q"], L["w13sf"], L["w13a"],
                       L["w2q"], L["w2sf"], L["w2a"], keep=keep, pool=pool,
                       x_gs=L.get("x_gs"))


def gpu_packed_weights(nv, L):
    """Upload the canonical weights of L and prepack them on the device."""
    from conftest import to_dev
    w13, w13_sf = nv.prepack_weights(to_dev(L["w13q"]), to_dev(L["w13sf"]))
    w2, w2_sf = nv.prepack_weights(to_dev(L["w2q"]), to_dev(L["w2sf"]))
    return dict(w13=w13, w13_sf=w13_sf, w13a=to_dev(L["w13a"]),
                w2=w2, w2_sf=w2_sf, w2a=to_dev(L["w2a"]))


def run_gpu_layer(nv, L, repeat=1, packed=None):
    """Run nvfp4_moe_forward `repeat` times, the last call with the gate/up
    tap; return y bits of every call, the tapped gate/up values ("gu", sorted
    rows) and the workspace intermediates (quantized operands cut to their
    unpadded widths)."""
    import torch
    from conftest import to_dev, to_host
    d = {k: to_dev(L[k]) for k in ("x", "ids", "wts")}
    pw = gpu_packed_weights(nv, L) if packed is None else packed
    T, H = L["x"].shape
    k = L["ids"].shape[1]
    E = L["w13q"].shape[0]
    I = L["w2q"].shape[1] * 2
    nws = nv.moe_workspace_size(T, H, I, E, k)
    ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
    x_gs = to_dev(np.array([L["x_gs"]], np.float32)) if L.get("x_gs") is not None else None
    I2 = 2 * I
    tap = torch.zeros((T * k, I2), dtype=torch.bfloat16, device="cuda")
    ys = []
    for i in range(repeat):
        y = nv.moe_forward(d["x"], d["ids"], d["wts"], pw["w13"], pw["w13_sf"], pw["w13a"],
                           pw["w2"], pw["w2_sf"], pw["w2a"], workspace=ws, x_gs=x_gs,
                           gate_up_tap=tap if i == repeat - 1 else None)
        ys.append(to_host(y))
    torch.cuda.synchronize()
    lay = nv.moe_workspace_layout(T, H, I, E, k)
    wsh = ws.cpu().numpy()
    S = T * k
    ldq_h, ldsf_h, _ = nv.operand_pitches(H)
    ldq_i, ldsf_i, _ = nv.operand_pitches(I)

    def view(name, dtype, count):
        o = lay[name]
        return wsh[o:o + count * np.dtype(dtype).itemsize].view(dtype)

    out = {"y": ys[-1], "ys": ys, "gu": to_host(tap),
           "xq": view("xq", np.uint8, T * ldq_h).reshape(T, ldq_h)[:, :H // 2],
           "xsf": view("xsf", np.uint8, T * ldsf_h).reshape(T, ldsf_h)[:, :H // 16],
           "gs1": view("gs1", np.float32, 1)[0], "gs2": view("gs2", np.float32, 1)[0],
           "counts": view("counts", np.int32, E), "offsets": view("offsets", np.int32, E + 1),
           "sorted_slot": view("sorted_slot", np.int32, S), "slot_row": view("slot_row", np.int32, S),
           "act": view("act", np.uint16, S * I).reshape(S, I),
           "aq": view("aq", np.uint8, S * ldq_i).reshape(S, ldq_i)[:, :I // 2],
           "asf": view("asf", np.uint8, S * ldsf_i).reshape(S, ldsf_i)[:, :I // 16]}
    return out
