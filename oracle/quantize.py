"""NVFP4 two-level quantization and dequantization (test infrastructure).

Follows the rule the pages give for the weight loader and for
``stage_activation`` (NVFP4 MegaMoE Debug Log, Hypothesis 6 steps 1-5 and "NVFP4 MoE
Pipeline"; NVFP4 MegaMoE Debug Log, later revision, "input_scale red herring"; src commit log,
quantizer fix and E4M3 `.view` fix):

1. global scale  gs = amax / (6 * 448), amax over the whole tensor;
2. block scale   s  = block_amax / (6 * gs), one per 16 consecutive elements
                      along the reduction axis, stored as an E4M3 byte;
3. element       nearest E2M1 value of x / (s_stored * gs);
4. packing       element 2j in the low nibble, element 2j+1 in the high one.

The pages leave the arithmetic open. This oracle takes the plainest reading and
every GPU path must follow the same one:

* all of it is IEEE float32 with round-to-nearest-even, no fused multiply-add,
  in exactly this order: gs = fl(amax / 2688); six_gs = fl(6 * gs);
  s = fl(bmax / six_gs), clamped to 448; den = fl(s_stored * gs);
  v = fl(|x| / den);
* the element divides by the *stored* (decoded) block scale, the byte that
  dequantization will multiply by (the nvfp4-megamoe-kernel src commit log,
  quantizer fix, item 2, which calls the stored block_max/6 the dequant factor);
* gs == 0 gives scale 0; den == 0 gives magnitude 0;
* the nibble's sign bit is the sign bit of x, also for -0.0 and for negative
  values that round to magnitude 0.

Parity pins (tests/test_oracle_quantize.py): the block holding the tensor amax
always gets scale byte 0x7E and its amax element magnitude 6.0 (closed form);
the pages' own (amax, global scale) pairs 3.86 -> 1.4e-3 and 2.86e-4 -> 0.77
(tests/golden/global_scale_pairs.txt); nibble order; sign symmetry Q(-x);
power-of-two invariance Q(2^j x); the round-trip error bound; bit-for-bit
agreement with the exact-rational twin in ``oracle.loops``. The static-scale
variant is pinned to the dynamic rule through its saturation property
(Q_static(x, gs(c)) == Q(clamp(x, +-c)), tests/test_oracle_ext.py); the
per-part weight rule is the per-matrix rule on each part, pinned through the
layer invariants there (equal part scales reproduce the per-matrix layer).
"""
import numpy as np

from .formats import (bf16_to_f32, e2m1_decode, e2m1_encode_magnitude,
                      e4m3_decode, e4m3_encode_nonneg)

F32 = np.float32
SIX_TIMES_E4M3_MAX = F32(2688.0)   # 6 * 448, exact
BLOCK = 16


def global_scale(amax):
    """gs = fl32(amax / 2688)."""
    return F32(F32(amax) / SIX_TIMES_E4M3_MAX)


def quantize_f32(x):
    """Quantize a float32 matrix (rows, cols), blocks of 16 along cols.

    Returns (q uint8 (rows, cols/2), sf uint8 (rows, cols/16), gs float32).
    The global scale needs the whole tensor's amax first; after that every
    row is independent, so rows are processed in chunks to bound memory.
    """
    x = np.asarray(x, dtype=F32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize expects a 2-D array with cols % 16 == 0")
    amax = F32(np.abs(x).max()) if x.size else F32(0.0)
    return quantize_f32_static(x, global_scale(amax))


def quantize_f32_static(x, gs):
    """Steps 2-4 of the rule with a global scale given by the caller.

    The static variant of stage_activation: gs is a fixed (e.g. calibrated)
    activation scale instead of amax / 2688 of this tensor (the later NVFP4 MegaMoE Debug Log
    revision discusses the checkpoint's calibrated ``input_scale`` in that
    role). Nothing else changes: a block whose amax exceeds 6 * 448 * gs gets
    the largest scale (s is clamped to 448, byte 0x7E) and its elements
    saturate at magnitude 6. Returns (q, sf, gs) like quantize_f32.
    """
    x = np.asarray(x, dtype=F32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize expects a 2-D array with cols % 16 == 0")
    gs = F32(gs)
    rows, cols = x.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    sf = np.empty((rows, cols // BLOCK), dtype=np.uint8)
    step = max(1, (1 << 18) // max(cols, 1))
    for r0 in range(0, rows, step):
        q[r0:r0 + step], sf[r0:r0 + step] = _quantize_rows(x[r0:r0 + step], gs)
    return q, sf, gs


def _quantize_rows(x, gs):
    """Steps 2-4 of the rule for some rows, given the tensor's global scale."""
    rows, cols = x.shape
    ax = np.abs(x)
    six_gs = F32(F32(6.0) * gs)
    bmax = ax.reshape(rows, cols // BLOCK, BLOCK).max(axis=2)
    if gs > 0:
        s = (bmax / six_gs).astype(F32)
        s = np.minimum(s, F32(448.0))
    else:
        s = np.zeros_like(bmax)
    sf = e4m3_encode_nonneg(s)
    s_dec = e4m3_decode(sf).astype(F32)                 # exact in float32
    den = (s_dec * gs).astype(F32)

    den_e = np.repeat(den, BLOCK, axis=1)
    ok = den_e > 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        v = np.where(ok, ax / np.where(ok, den_e, F32(1.0)), F32(0.0)).astype(F32)
    mag = e2m1_encode_magnitude(v)
    nib = (np.signbit(x).astype(np.uint8) << 3) | mag
    q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return q, sf.astype(np.uint8)


def quantize_bf16(x_bits):
    """O-Q on bf16 input bits (uint16, rows x cols)."""
    return quantize_f32(bf16_to_f32(x_bits))


def quantize_weight_bf16(w_bits):
    """Weight rule: W (K, N) bf16 bits, blocks of 16 along K, amax over all of W.

    Returns (q (K/2, N), sf (K/16, N), alpha) with byte [kh, n] holding
    W[2kh, n] in its low nibble and W[2kh+1, n] in its high nibble, i.e. the
    activation rule applied to W transposed and stored transposed back.
    """
    q_t, sf_t, gs = quantize_bf16(np.ascontiguousarray(np.asarray(w_bits).T))
    return np.ascontiguousarray(q_t.T), np.ascontiguousarray(sf_t.T), gs


def quantize_bf16_static(x_bits, gs):
    """quantize_f32_static on bf16 input bits."""
    return quantize_f32_static(bf16_to_f32(x_bits), gs)


def quantize_weight_bf16_parts(w_bits, parts):
    """Weight rule with one global scale per column part.

    W (K, N) is split along N into `parts` equal column ranges; each range is
    quantized with the weight rule on its own (its own amax), and the results
    are concatenated back along N. For w13 = [gate | up] with parts = 2 this is
    the per-half weight global scale of the NVFP4 MegaMoE Debug Log ("Bugs Fixed", BF16
    reference item 4: a global scale of shape (2,), applied per half) and of
    the later revision's code-review item 5 (scaling the up half by the ratio
    of the halves' scales is a per-column alpha).

    Returns (q (K/2, N), sf (K/16, N), alphas float32 (parts,)).
    """
    w_bits = np.asarray(w_bits)
    K, N = w_bits.shape
    if parts < 1 or N % parts:
        raise ValueError("N must be a multiple of parts")
    w = N // parts
    out = [quantize_weight_bf16(w_bits[:, p * w:(p + 1) * w]) for p in range(parts)]
    q = np.concatenate([o[0] for o in out], axis=1)
    sf = np.concatenate([o[1] for o in out], axis=1)
    return q, sf, np.array([o[2] for o in out], dtype=F32)


def unpack_nibbles(q, axis):
    """Split packed bytes into nibbles along `axis`: low nibble first."""
    q = np.asarray(q, dtype=np.uint8)
    lo = q & 0xF
    hi = q >> 4
    st = np.stack([lo, hi], axis=axis + 1)
    shape = list(q.shape)
    shape[axis] *= 2
    return st.reshape(shape)


def dequantize_rows(q, sf):
    """Row-blocked operand (rows, cols/2) + (rows, cols/16) -> float64 values.

    The value excludes the global scale, which the GEMM applies through alpha.
    """
    nib = unpack_nibbles(q, axis=1)
    scale = np.repeat(e4m3_decode(sf), BLOCK, axis=1)
    return e2m1_decode(nib) * scale


def dequantize_cols(q, sf):
    """K-packed operand (K/2, N) + (K/16, N) -> float64 (K, N), gs excluded."""
    nib = unpack_nibbles(q, axis=0)
    scale = np.repeat(e4m3_decode(sf), BLOCK, axis=0)
    return e2m1_decode(nib) * scale
