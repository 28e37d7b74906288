"""Python binding of libnvfp4moe (NVFP4 expert layer on MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch provides device memory and the current stream. The functions
mirror the C ABI in include/nvfp4moe.h:

    quantize(x)                      -> (q, sf, gs)
    quantize_static(x, gs)           -> (q, sf)           caller-given global scale
    quantize_weights(w)              -> (q, sf, alpha)    canonical weight layout
    quantize_weights_parts(w, parts) -> (q, sf, alpha (E, parts))
    operand_pitches(K)               -> (ldq, ldsf, ldwsf)
    packed_shapes(E, K, N)           -> shapes of the packed weight tensors
    prepack_weights(q, sf)           -> (q_t, sf_t)       packed layout the GEMMs read
    gemm(aq, asf, a_gs, bq_t, bsf_t, b_alpha) -> out (bf16), K % 16 == 0
    moe_forward(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha,
                w2, w2_sf, w2_alpha, workspace=None, stage_events=None,
                x_gs=None, gate_up_tap=None) -> y   (w13_alpha (E,) or per half (E, 2))
    moe_forward_noalloc(...)         -> y     the same without a workspace
    route_topk(logits, topk)         -> (topk_ids, topk_weights)

The library must be built in-tree first (``python -m
nvfp4_block_scaled_quant_amd.build``); importing this package without it
raises ImportError, so no caller can silently fall back to anything else.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python nvfp4_block_scaled_quant_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int

_SIGS = {
    "nvfp4_strerror": ([_int], ctypes.c_char_p),
    "nvfp4_version": ([], _int),
    "nvfp4_quantize_workspace": ([_i64, _i64], _sz),
    "nvfp4_quantize": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nvfp4_quantize_weights_workspace": ([_i64, _i64, _i64], _sz),
    "nvfp4_quantize_weights": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nvfp4_operand_pitches": ([_i64] + [ctypes.POINTER(_i64)] * 3, _int),
    "nvfp4_prepack_weights": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "nvfp4_gemm_workspace": ([_i64, _i64, _i64], _sz),
    "nvfp4_gemm": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp], _int),
    "nvfp4_moe_workspace": ([_i64, _i64, _i64, _i64, _i64], _sz),
    "nvfp4_moe_workspace_layout": ([_i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_sz)], _int),
    "nvfp4_moe_forward": ([_vp] * 9 + [_i64] * 5 + [_vp, _vp, _sz, _vp, _vp], _int),
    "nvfp4_quantize_static": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "nvfp4_quantize_weights_parts_workspace": ([_i64, _i64, _i64, _i64], _sz),
    "nvfp4_quantize_weights_parts": ([_vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp],
                                     _int),
    "nvfp4_moe_forward_ex": ([_vp] * 9 + [_i64] * 5 + [_vp, _vp, _sz, _vp, _vp, _vp], _int),
    "nvfp4_route_topk": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "nvfp4_moe_forward_noalloc": ([_vp] * 9 + [_i64] * 5 + [_vp, _vp, _vp, _vp], _int),
}

# NVFP4_MOE_SCRATCH_BYTES (include/nvfp4moe.h): the static workspace of
# nvfp4_moe_forward_noalloc
MOE_SCRATCH_BYTES = 32 << 20


class MoeOptions(ctypes.Structure):
    """struct nvfp4_moe_options."""
    _fields_ = [("w13_alpha_per_half", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x_global_scale", ctypes.c_void_p), ("gate_up_tap", ctypes.c_void_p)]


for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)

# stage / workspace indices (include/nvfp4moe.h)
STAGES = ("route", "quant_x", "l1", "requant", "l2", "combine")
NUM_EVENTS = len(STAGES) + 1
WS_NAMES = ("xq", "xsf", "gs1", "gs2", "counts", "offsets", "sorted_slot", "slot_row",
            "act", "aq", "asf", "o2", "xh", "ah")


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        msg = _lib.nvfp4_strerror(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def _check(status, where):
    if status != 0:
        raise Nvfp4Error(status, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, dim=None, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _out(t, shape, dtype, device, name):
    """A caller-given output tensor (checked: the kernels write exactly
    `shape`), or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, dtype, name, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(t, nbytes, device):
    """A caller-given workspace (any dtype, its size in bytes is passed on and
    checked by the library), or a new uint8 one of nbytes."""
    if t is None:
        return torch.empty((nbytes,), dtype=torch.uint8, device=device)
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA (HIP) tensor")
    if t.device != device:
        raise ValueError(f"workspace is on {t.device}, the other operands on {device}")
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


def version():
    v = _lib.nvfp4_version()
    return (v >> 16, v & 0xFFFF)


def strerror(status):
    return _lib.nvfp4_strerror(status).decode()


def quantize(x, q=None, sf=None, gs=None, workspace=None):
    """NVFP4-quantize a bf16 (M, K) activation. Returns (q uint8 (M, K/2),
    sf uint8 (M, K/16) E4M3 bits, gs float32 (1,))."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    dev = x.device
    q = _out(q, (M, K // 2), torch.uint8, dev, "q")
    sf = _out(sf, (M, K // 16), torch.uint8, dev, "sf")
    gs = _out(gs, (1,), torch.float32, dev, "gs")
    ws = _workspace(workspace, _lib.nvfp4_quantize_workspace(M, K), dev)
    _check(_lib.nvfp4_quantize(_ptr(x), M, K, _ptr(q), _ptr(sf), _ptr(gs), _ptr(ws),
                               _nbytes(ws), _stream()), "nvfp4_quantize")
    return q, sf, gs


def quantize_static(x, gs, q=None, sf=None):
    """NVFP4-quantize a bf16 (M, K) activation with the given global scale gs
    (float32 (1,) on the device). Returns (q uint8 (M, K/2), sf uint8 (M, K/16))."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    dev = x.device
    _need(gs, torch.float32, "gs", 1, dev)
    if gs.numel() < 1:
        raise ValueError("gs must hold one float32")
    q = _out(q, (M, K // 2), torch.uint8, dev, "q")
    sf = _out(sf, (M, K // 16), torch.uint8, dev, "sf")
    _check(_lib.nvfp4_quantize_static(_ptr(x), M, K, _ptr(gs), _ptr(q), _ptr(sf), _stream()),
           "nvfp4_quantize_static")
    return q, sf


def quantize_weights_parts(w, parts):
    """quantize_weights with one global scale per column part: W[e] (K, N)
    split along N into `parts` equal ranges. Returns (q (E, K/2, N), sf
    (E, K/16, N), alpha float32 (E, parts))."""
    _need(w, torch.bfloat16, "w", 3)
    E, K, N = w.shape
    dev = w.device
    q = torch.empty((E, K // 2, N), dtype=torch.uint8, device=dev)
    sf = torch.empty((E, K // 16, N), dtype=torch.uint8, device=dev)
    alpha = torch.empty((E, parts), dtype=torch.float32, device=dev)
    nws = _lib.nvfp4_quantize_weights_parts_workspace(E, K, N, parts)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    _check(_lib.nvfp4_quantize_weights_parts(_ptr(w), E, K, N, parts, _ptr(q), _ptr(sf),
                                             _ptr(alpha), _ptr(ws), _nbytes(ws), _stream()),
           "nvfp4_quantize_weights_parts")
    return q, sf, alpha


def route_topk(logits, topk, ids=None, weights=None):
    """Top-k router: logits float32 (T, E) -> (topk_ids int32 (T, topk),
    topk_weights float32 (T, topk)), softmax renormalized over the selected."""
    _need(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    dev = logits.device
    if topk < 1:
        raise ValueError("route_topk: topk must be at least 1")
    ids = _out(ids, (T, topk), torch.int32, dev, "ids")
    weights = _out(weights, (T, topk), torch.float32, dev, "weights")
    _check(_lib.nvfp4_route_topk(_ptr(logits), T, E, topk, _ptr(ids), _ptr(weights), _stream()),
           "nvfp4_route_topk")
    return ids, weights


def quantize_weights(w):
    """Quantize E bf16 weight matrices W[e] (K, N) with blocks along K.
    Returns (q uint8 (E, K/2, N), sf uint8 (E, K/16, N), alpha float32 (E,))."""
    _need(w, torch.bfloat16, "w", 3)
    E, K, N = w.shape
    dev = w.device
    q = torch.empty((E, K // 2, N), dtype=torch.uint8, device=dev)
    sf = torch.empty((E, K // 16, N), dtype=torch.uint8, device=dev)
    alpha = torch.empty((E,), dtype=torch.float32, device=dev)
    nws = _lib.nvfp4_quantize_weights_workspace(E, K, N)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    _check(_lib.nvfp4_quantize_weights(_ptr(w), E, K, N, _ptr(q), _ptr(sf), _ptr(alpha), _ptr(ws),
                                       _nbytes(ws), _stream()), "nvfp4_quantize_weights")
    return q, sf, alpha


def operand_pitches(K):
    """Row pitches (bytes) for reduction length K: ldq (packed data, K/2
    rounded up to 64), ldsf (activation scales, K/16 rounded up to 8), ldwsf
    (packed weight scales, whole groups of four 128-element steps)."""
    ldq, ldsf, ldwsf = _i64(), _i64(), _i64()
    _check(_lib.nvfp4_operand_pitches(K, ctypes.byref(ldq), ctypes.byref(ldsf), ctypes.byref(ldwsf)),
           "nvfp4_operand_pitches")
    return ldq.value, ldsf.value, ldwsf.value


def packed_shapes(E, K, N):
    """Shapes of the packed weight tensors of E matrices (K, N), in 16-row
    blocks: data (E, N/16, halves, 16, 32), one 64-element half step of the
    block's 16 rows after another, halves = ldq / 32; scales (E, N/16, quads,
    16, 32), quads = ldwsf / 32: per group of four 128-element K steps, row,
    pair of scale groups (4), step of the four (4), then the pair's two
    bytes."""
    ldq, _, ldwsf = operand_pitches(K)
    if N % 16:
        raise ValueError("packed weights need N % 16 == 0")
    return (E, N // 16, ldq // 32, 16, 32), (E, N // 16, ldwsf // 32, 16, 32)


def prepack_weights(q, sf):
    """Canonical quantized weights q (E, K/2, N), sf (E, K/16, N) -> the packed
    layout that gemm and moe_forward read (see packed_shapes)."""
    _need(q, torch.uint8, "q", 3)
    _need(sf, torch.uint8, "sf", 3, q.device)
    E, Kh, N = q.shape
    K = 2 * Kh
    if sf.shape != (E, K // 16, N):
        raise ValueError("prepack_weights: q and sf shapes do not match")
    shq, shs = packed_shapes(E, K, N)
    q_t = torch.empty(shq, dtype=torch.uint8, device=q.device)
    sf_t = torch.empty(shs, dtype=torch.uint8, device=q.device)
    _check(_lib.nvfp4_prepack_weights(_ptr(q), _ptr(sf), E, K, N, _ptr(q_t), _ptr(sf_t),
                                      _stream()), "nvfp4_prepack_weights")
    return q_t, sf_t


def gemm(aq, asf, a_gs, bq, bsf, b_alpha, out=None, workspace=None):
    """Block-scaled NVFP4 GEMM of one expert: A (M, K/2) + (M, K/16) times one
    packed weight matrix bq (N/16, halves, 16, 32) + bsf (N/16, quads, 16, 32)
    (packed_shapes with E dropped) -> bf16 (M, N). K % 16 == 0. The workspace
    (nvfp4_gemm_workspace bytes) receives A's exact f16 values."""
    _need(aq, torch.uint8, "aq")
    for t, n, d in ((asf, "asf", torch.uint8), (bq, "bq", torch.uint8),
                    (bsf, "bsf", torch.uint8), (a_gs, "a_gs", torch.float32),
                    (b_alpha, "b_alpha", torch.float32)):
        _need(t, d, n, None, aq.device)
    if a_gs.numel() < 1 or b_alpha.numel() < 1:
        raise ValueError("gemm: a_gs and b_alpha must hold one float32 each")
    if aq.dim() != 2 or bq.dim() != 4:
        raise ValueError("gemm: aq must be (M, K/2) and bq (N/16, halves, 16, 32)")
    M = aq.shape[0]
    K = aq.shape[1] * 2
    N = bq.shape[0] * 16
    if K % 16:
        raise ValueError("gemm: K must be a multiple of 16")
    shq, shs = packed_shapes(1, K, N)
    if tuple(bq.shape) != shq[1:] or asf.shape != (M, K // 16) or tuple(bsf.shape) != shs[1:]:
        raise ValueError("operand shapes do not match")
    out = _out(out, (M, N), torch.bfloat16, aq.device, "out")
    ws = _workspace(workspace, max(1, _lib.nvfp4_gemm_workspace(M, N, K)), aq.device)
    _check(_lib.nvfp4_gemm(_ptr(aq), _ptr(asf), _ptr(a_gs), _ptr(bq), _ptr(bsf), _ptr(b_alpha),
                           M, N, K, _ptr(out), _ptr(ws), _nbytes(ws), _stream()), "nvfp4_gemm")
    return out


def moe_workspace_size(T, H, I, E, topk):
    n = _lib.nvfp4_moe_workspace(T, H, I, E, topk)
    if n == 0:
        raise Nvfp4Error(2, "nvfp4_moe_workspace")
    return n


def moe_workspace_layout(T, H, I, E, topk):
    arr = (_sz * len(WS_NAMES))()
    _check(_lib.nvfp4_moe_workspace_layout(T, H, I, E, topk, arr), "nvfp4_moe_workspace_layout")
    return dict(zip(WS_NAMES, list(arr)))


def _moe_args(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2, w2_sf, w2_alpha, y, x_gs,
              gate_up_tap):
    """Checks shared by moe_forward and moe_forward_noalloc; returns the sizes,
    y and the options struct (None when every option is at its default)."""
    _need(x, torch.bfloat16, "x", 2)
    dev = x.device
    _need(topk_ids, torch.int32, "topk_ids", 2, dev)
    _need(topk_weights, torch.float32, "topk_weights", 2, dev)
    for t, n in ((w13, "w13"), (w13_sf, "w13_sf"), (w2, "w2"), (w2_sf, "w2_sf")):
        _need(t, torch.uint8, n, 5, dev)
    _need(w13_alpha, torch.float32, "w13_alpha", None, dev)
    _need(w2_alpha, torch.float32, "w2_alpha", 1, dev)
    if x_gs is not None:
        _need(x_gs, torch.float32, "x_gs", 1, dev)
        if x_gs.numel() < 1:
            raise ValueError("x_gs must hold one float32")
    T, H = x.shape
    topk = topk_ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] * 8
    if H % 16 or H == 0 or I == 0:
        raise ValueError("moe_forward: H and I must be positive multiples of 16")
    s13, s13f = packed_shapes(E, H, 2 * I)
    s2, s2f = packed_shapes(E, I, H)
    if (tuple(w13.shape) != s13 or tuple(w13_sf.shape) != s13f
            or tuple(w2.shape) != s2 or tuple(w2_sf.shape) != s2f
            or w13_alpha.shape not in ((E,), (E, 2)) or w2_alpha.shape != (E,)
            or topk_ids.shape != (T, topk) or topk_weights.shape != (T, topk)):
        raise ValueError("moe_forward: inconsistent shapes")
    y = _out(y, (T, H), torch.bfloat16, dev, "y")
    if gate_up_tap is not None:
        _out(gate_up_tap, (T * topk, 2 * I), torch.bfloat16, dev, "gate_up_tap")
    per_half = w13_alpha.dim() == 2
    opts = None
    if per_half or x_gs is not None or gate_up_tap is not None:
        opts = MoeOptions(1 if per_half else 0, 0, x_gs.data_ptr() if x_gs is not None else None,
                          gate_up_tap.data_ptr() if gate_up_tap is not None else None)
    return T, H, I, E, topk, y, opts


def moe_forward(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2, w2_sf, w2_alpha,
                y=None, workspace=None, stage_events=None, x_gs=None, gate_up_tap=None):
    """The five-stage NVFP4 expert layer. Weights in the packed layout
    (prepack_weights of the canonical (E, H/2, 2I) and (E, I/2, H) tensors).

    w13_alpha: (E,) one weight global scale per expert, or (E, 2) per half
    (gate, up). x_gs: None (dynamic gs1) or a float32 (1,) static gs1.
    gate_up_tap: None, or a bf16 (T * topk, 2I) tensor that receives the
    rounded L1 output (sorted rows, gate | up), for stage-by-stage checks.
    stage_events: None or a StageEvents; returns y (T, H) bf16.
    """
    T, H, I, E, topk, y, opts = _moe_args(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2,
                                          w2_sf, w2_alpha, y, x_gs, gate_up_tap)
    workspace = _workspace(workspace, moe_workspace_size(T, H, I, E, topk), x.device)
    ev = stage_events.handles if stage_events is not None else None
    args = (_ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w13), _ptr(w13_sf), _ptr(w13_alpha),
            _ptr(w2), _ptr(w2_sf), _ptr(w2_alpha), T, H, I, E, topk, _ptr(y), _ptr(workspace),
            _nbytes(workspace), _stream(), ev)
    if opts is None:
        _check(_lib.nvfp4_moe_forward(*args), "nvfp4_moe_forward")
    else:
        _check(_lib.nvfp4_moe_forward_ex(*args, ctypes.byref(opts)), "nvfp4_moe_forward_ex")
    return y


def moe_forward_noalloc(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2, w2_sf, w2_alpha,
                        y=None, stage_events=None, x_gs=None, gate_up_tap=None):
    """moe_forward without a workspace: the library's static per-GPU scratch
    (MOE_SCRATCH_BYTES) holds the intermediates and the call allocates
    nothing on the device (pass y to allocate nothing at all). Calls that
    overlap on one GPU share that scratch and must not run concurrently."""
    T, H, I, E, topk, y, opts = _moe_args(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2,
                                          w2_sf, w2_alpha, y, x_gs, gate_up_tap)
    ev = stage_events.handles if stage_events is not None else None
    _check(_lib.nvfp4_moe_forward_noalloc(
        _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w13), _ptr(w13_sf), _ptr(w13_alpha),
        _ptr(w2), _ptr(w2_sf), _ptr(w2_alpha), T, H, I, E, topk, _ptr(y), _stream(), ev,
        ctypes.byref(opts) if opts is not None else None), "nvfp4_moe_forward_noalloc")
    return y


class _Hip:
    """The few HIP runtime calls the stage timer needs (events)."""
    _rt = None

    @classmethod
    def rt(cls):
        if cls._rt is None:
            rt = ctypes.CDLL("libamdhip64.so")
            rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            cls._rt = rt
        return cls._rt


class StageEvents:
    """HIP events recorded by nvfp4_moe_forward around each stage (on the
    stream the stage's kernels run on)."""

    def __init__(self, n=NUM_EVENTS):
        rt = _Hip.rt()
        self._arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._arr[i] = h
        self.n = n

    @property
    def handles(self):
        return ctypes.cast(self._arr, ctypes.c_void_p)

    def elapsed_ms(self):
        """Per-stage milliseconds of the last recorded forward."""
        rt = _Hip.rt()
        if rt.hipEventSynchronize(self._arr[self.n - 1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = []
        for i in range(self.n - 1):
            ms = ctypes.c_float()
            if rt.hipEventElapsedTime(ctypes.byref(ms), self._arr[i], self._arr[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return dict(zip(STAGES, out))

    def __del__(self):
        try:
            rt = _Hip.rt()
            for i in range(self.n):
                rt.hipEventDestroy(self._arr[i])
        except Exception:
            pass
