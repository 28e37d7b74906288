"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before touching any device (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quant_amd as nv
    return nv


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("nvfp4_quantize", "nvfp4_moe_forward", "nvfp4_gemm", "nvfp4_strerror",
                 "nvfp4_quantize_weights", "nvfp4_moe_workspace", "nvfp4_prepack_weights",
                 "nvfp4_operand_pitches", "nvfp4_quantize_static", "nvfp4_quantize_weights_parts",
                 "nvfp4_moe_forward_ex", "nvfp4_route_topk"):
        assert must in names


def test_library_exports_every_declared_symbol(nv):
    lib = ctypes.CDLL(nv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in nvfp4moe.h but not exported"
    assert set(declared_functions()) == set(nv.EXPORTED)


def test_strerror_and_version(nv):
    assert nv.version() == (5, 0)
    for code in range(7):
        assert len(nv.strerror(code)) > 0
    assert nv.strerror(99) == "unknown status"


L = None


def lib(nv):
    return nv._lib


def p(v):
    return ctypes.c_void_p(v)


A16 = 1 << 20          # a fake, aligned, never-dereferenced address


def test_quantize_argument_errors(nv):
    f = lib(nv).nvfp4_quantize
    ws = p(A16)
    assert f(p(A16), 4, 15, p(A16), p(A16), p(A16), ws, 256, None) == 2     # K % 16
    assert f(p(A16), -1, 16, p(A16), p(A16), p(A16), ws, 256, None) == 1    # M < 0
    assert f(p(A16), 4, 16, p(A16), p(A16), p(0), ws, 256, None) == 1       # gs null
    assert f(p(0), 4, 16, p(A16), p(A16), p(A16), ws, 256, None) == 1       # x null
    assert f(p(A16 + 2), 4, 16, p(A16), p(A16), p(A16), ws, 256, None) == 1  # x misaligned
    assert f(p(A16), 4, 16, p(A16), p(A16), p(A16), ws, 8, None) == 3       # ws small
    assert f(p(A16), 4, 16, p(A16), p(A16), p(A16), p(A16 + 8), 256, None) == 3  # ws align
    assert lib(nv).nvfp4_quantize_workspace(4, 16) >= 4


def test_quantize_weights_argument_errors(nv):
    f = lib(nv).nvfp4_quantize_weights
    assert f(p(A16), 2, 24, 16, p(A16), p(A16), p(A16), p(A16), 256, None) == 2
    assert f(p(A16), -2, 32, 16, p(A16), p(A16), p(A16), p(A16), 256, None) == 1
    assert f(p(0), 2, 32, 16, p(A16), p(A16), p(A16), p(A16), 256, None) == 1
    assert f(p(A16), 2, 32, 16, p(A16), p(A16), p(A16), p(A16), 4, None) == 3
    assert f(p(0), 0, 32, 16, p(0), p(0), p(0), p(0), 0, None) == 0          # E == 0: nothing


def test_gemm_argument_errors(nv):
    f = lib(nv).nvfp4_gemm
    ws = lib(nv).nvfp4_gemm_workspace
    args = [p(A16)] * 6
    big = 1 << 40

    def call(a, M, N, K, wsp=A16, nbytes=big):
        return f(*a, M, N, K, p(A16), p(wsp), nbytes, None)

    assert call(args, 4, 16, 24) == 2                   # K % 16
    assert call(args, 4, 24, 128) == 2                  # N % 16
    assert call(args, -4, 16, 128) == 1
    assert call(args, 0, 16, 128) == 0                  # M == 0: nothing to do
    bad = [p(A16)] * 5 + [p(0)]
    assert call(bad, 4, 16, 128) == 1
    mis = [p(A16)] * 3 + [p(A16 + 8)] + [p(A16)] * 2   # bq not 16-byte aligned
    assert call(mis, 4, 16, 128) == 1
    assert call(args, 1 << 20, 16, 1 << 13) == 2        # A beyond 32-bit offsets
    # the workspace holds A as f16, rows padded to whole 128-element steps
    assert ws(4, 16, 144) == 4 * 512                    # K = 144 pads to 256 elements: 512 bytes a row
    assert ws(3, 16, 16) == 3 * 256                      # K = 16: one 128-element step, 256 bytes a row
    # 256-row tiles would be only 24: the dense GEMM takes 48 tiles of 128 x 256
    # and cuts K's 112 64-element steps into 5 chunks of up to 23 (240
    # work-groups, at most one per CU), each chunk with an fp32 partial-sum
    # plane of M x N after the f16 A
    assert ws(256, 6144, 7168) == 256 * 7168 * 2 + 5 * 256 * 6144 * 4
    assert ws(4096, 6144, 7168) == 4096 * 7168 * 2      # 384 tiles: no split
    # 512 rows: 96 tiles of 128 x 256, 2 chunks; 1280 rows: 240 tiles of
    # 128 x 256 fill the GPU without a split (256-row tiles would be 120);
    # 3072 rows: 288 tiles of 256 x 256, no split
    assert ws(512, 6144, 7168) == 512 * 7168 * 2 + 2 * 512 * 6144 * 4
    assert ws(1280, 6144, 7168) == 1280 * 7168 * 2
    assert ws(3072, 6144, 7168) == 3072 * 7168 * 2
    assert ws(4, 16, 24) == 0 and ws(-1, 16, 128) == 0
    assert call(args, 4, 16, 144, nbytes=ws(4, 16, 144) - 1) == 3
    assert call(args, 4, 16, 144, wsp=A16 + 64) == 3    # misaligned workspace
    assert call(args, 4, 16, 144, wsp=0) == 3


def test_operand_pitches(nv):
    # (ldq, ldsf, ldwsf): data in whole 128-element steps, activation scales
    # in whole 8-byte steps, packed weight scales in whole groups of four steps
    for K, want in [(16, (64, 8, 32)), (128, (64, 8, 32)), (144, (128, 16, 32)),
                    (272, (192, 24, 32)), (7168, (3584, 448, 448)), (3072, (1536, 192, 192)),
                    (400, (256, 32, 32)), (640, (320, 40, 64))]:
        assert nv.operand_pitches(K) == want
    ldq, ldsf, ldw = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    f = lib(nv).nvfp4_operand_pitches
    assert f(24, ctypes.byref(ldq), ctypes.byref(ldsf), ctypes.byref(ldw)) == 2
    assert f(0, ctypes.byref(ldq), ctypes.byref(ldsf), ctypes.byref(ldw)) == 1
    assert f(32, None, ctypes.byref(ldsf), ctypes.byref(ldw)) == 1
    assert f(32, ctypes.byref(ldq), ctypes.byref(ldsf), None) == 1


def test_prepack_argument_errors(nv):
    f = lib(nv).nvfp4_prepack_weights
    assert f(p(A16), p(A16), 2, 24, 16, p(A16), p(A16), None) == 2        # K % 16
    assert f(p(A16), p(A16), 2, 32, 24, p(A16), p(A16), None) == 2        # N % 16
    assert f(p(A16), p(A16), -1, 32, 16, p(A16), p(A16), None) == 1
    assert f(p(A16), p(A16), 2, 32, 0, p(A16), p(A16), None) == 1
    assert f(p(0), p(A16), 2, 32, 16, p(A16), p(A16), None) == 1
    assert f(p(A16), p(A16), 2, 32, 16, p(A16 + 4), p(A16), None) == 1    # w_t alignment
    assert f(p(0), p(0), 0, 32, 16, p(0), p(0), None) == 0                 # E == 0: nothing


def test_moe_argument_errors(nv):
    f = lib(nv).nvfp4_moe_forward
    ptrs9 = [p(A16)] * 9

    def call(T, H, I, E, k, ws_bytes=1 << 40, ws=A16, ptrs=ptrs9, y=A16):
        return f(*ptrs, T, H, I, E, k, p(y), p(ws), ws_bytes, None, None)

    assert call(8, 7168, 3072, 48, 49) == 2          # topk > E
    assert call(8, 7000, 3072, 48, 8) == 2           # H % 16
    assert call(8, 7168, 3000, 48, 8) == 2           # I % 16
    assert call(8, 7168, 3072, 513, 8) == 2          # E above the supported maximum
    assert call(-1, 7168, 3072, 48, 8) == 1
    assert call(8, 7168, 3072, 48, 0) == 1
    assert call(8, 7168, 3072, 48, 8, ws_bytes=1024) == 3
    assert call(8, 7168, 3072, 48, 8, ws=A16 + 64) == 3
    assert call(8, 7168, 3072, 48, 8, ptrs=[p(A16 + 4)] + ptrs9[1:]) == 1   # x misaligned
    assert call(8, 7168, 3072, 48, 8, ptrs=ptrs9[:3] + [p(0)] + ptrs9[4:]) == 1
    assert call(8, 7168, 3072, 48, 8, y=0) == 1


def test_moe_forward_ex_option_errors(nv):
    f = lib(nv).nvfp4_moe_forward_ex
    ptrs9 = [p(A16)] * 9

    def call(opts, T=8):
        ref = ctypes.byref(opts) if opts is not None else None
        return f(*ptrs9, T, 7168, 3072, 48, 8, p(A16), p(A16), 1024, None, None, ref)

    # a null options pointer is nvfp4_moe_forward: same validation order
    assert call(None) == 3                                   # workspace too small
    assert call(nv.MoeOptions(2, 0, None)) == 1              # per_half must be 0 or 1
    assert call(nv.MoeOptions(-1, 0, None)) == 1
    assert call(nv.MoeOptions(0, 0, A16 + 2)) == 1           # misaligned static scale
    assert call(nv.MoeOptions(0, 7, None)) == 1               # reserved must be 0
    assert call(nv.MoeOptions(0, 0, None, A16 + 2)) == 1     # misaligned gate/up tap
    assert call(nv.MoeOptions(1, 0, A16)) == 3               # valid options, then the workspace
    assert call(nv.MoeOptions(1, 0, A16, A16)) == 3
    assert call(nv.MoeOptions(1, 0, A16), T=0) == 3


def test_moe_forward_noalloc_argument_errors(nv):
    # validated on the host before the scratch array or any device is touched
    f = lib(nv).nvfp4_moe_forward_noalloc
    ptrs9 = [p(A16)] * 9

    def call(T, H=7168, I=3072, E=48, k=8):
        return f(*ptrs9, T, H, I, E, k, p(A16), None, None, None)

    assert call(4096) == 6                     # the prefill batch needs ~1.2 GB: beyond the scratch
    assert call(-1) == 1
    assert call(8, k=49) == 2                  # topk > E
    assert call(8, H=7000) == 2
    assert nv.moe_workspace_size(8, 7168, 3072, 48, 8) <= nv.MOE_SCRATCH_BYTES
    assert nv.moe_workspace_size(4096, 7168, 3072, 48, 8) > nv.MOE_SCRATCH_BYTES
    assert "scratch" in nv.strerror(6)


def test_quantize_static_argument_errors(nv):
    f = lib(nv).nvfp4_quantize_static
    assert f(p(A16), 4, 40, p(A16), p(A16), p(A16), None) == 2      # K % 16
    assert f(p(A16), -1, 32, p(A16), p(A16), p(A16), None) == 1
    assert f(p(A16), 4, 32, p(0), p(A16), p(A16), None) == 1        # gs null
    assert f(p(A16 + 2), 4, 32, p(A16), p(A16), p(A16), None) == 1  # x alignment
    assert f(p(0), 0, 32, p(0), p(0), p(0), None) == 0              # M == 0: nothing


def test_quantize_weights_parts_argument_errors(nv):
    f = lib(nv).nvfp4_quantize_weights_parts
    ws = lib(nv).nvfp4_quantize_weights_parts_workspace
    assert ws(48, 7168, 6144, 2) >= 48 * 2 * 4
    assert f(p(A16), 2, 64, 48, 5, p(A16), p(A16), p(A16), p(A16), 1 << 20, None) == 2   # N % parts
    assert f(p(A16), 2, 64, 60, 5, p(A16), p(A16), p(A16), p(A16), 1 << 20, None) == 2   # N/parts % 8
    assert f(p(A16), 2, 64, 48, 0, p(A16), p(A16), p(A16), p(A16), 1 << 20, None) == 1
    assert f(p(A16), 2, 64, 48, 17, p(A16), p(A16), p(A16), p(A16), 1 << 20, None) == 2
    assert f(p(A16), 2, 64, 48, 2, p(A16), p(A16), p(A16), p(A16), 8, None) == 3         # workspace
    assert f(p(A16), 0, 64, 48, 2, p(0), p(0), p(0), p(0), 0, None) == 0                 # E == 0


def test_route_topk_argument_errors(nv):
    f = lib(nv).nvfp4_route_topk
    assert f(p(A16), 16, 48, 49, p(A16), p(A16), None) == 2         # topk > E
    assert f(p(A16), 16, 513, 8, p(A16), p(A16), None) == 2         # E above the maximum
    assert f(p(A16), 16, 48, 0, p(A16), p(A16), None) == 1
    assert f(p(A16), -1, 48, 8, p(A16), p(A16), None) == 1
    assert f(p(0), 16, 48, 8, p(A16), p(A16), None) == 1
    assert f(p(A16 + 2), 16, 48, 8, p(A16), p(A16), None) == 1      # alignment
    assert f(p(0), 0, 48, 8, p(0), p(0), None) == 0                 # T == 0: nothing


def test_moe_workspace_layout_is_consistent(nv):
    for shape in [(32, 256, 128, 4, 2), (8, 7168, 3072, 48, 8), (4096, 7168, 3072, 48, 8),
                  (1, 16, 16, 1, 1), (0, 16, 16, 1, 1)]:
        T, H, I, E, k = shape
        total = nv.moe_workspace_size(*shape)
        lay = nv.moe_workspace_layout(*shape)
        S = T * k
        qh, sh, _ = nv.operand_pitches(H)
        qi, si, _ = nv.operand_pitches(I)
        ends = {"xq": T * qh, "xsf": T * sh, "gs1": 4, "gs2": 4, "counts": 4 * E,
                "offsets": 4 * (E + 1), "sorted_slot": 4 * S, "slot_row": 4 * S,
                "act": 2 * S * I, "aq": S * qi, "asf": S * si, "o2": 4 * S * H}
        spans = sorted((lay[n], lay[n] + ends[n]) for n in ends)
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(lay[n] % 256 == 0 for n in lay)
        assert spans[-1][1] <= total
    with pytest.raises(Exception):
        nv.moe_workspace_size(8, 7168, 3072, 48, 49)


def test_weight_streaming_path_stops_at_its_lds_limit(nv):
    # a decode-size batch (8 tokens, top-8 of 48) takes the weight-streaming
    # GEMMs while a 16-row activation tile fits their LDS (K up to 17,024);
    # above that it takes the tiled GEMMs, whose workspace also holds the f16
    # copies of x (T rows of pitch_h(H)) and act (S rows of pitch_h(I))
    T, E, k = 8, 48, 8
    for H0, I0, H1, I1 in [(17024, 256, 17040, 256), (256, 17024, 256, 17040)]:
        a = nv.moe_workspace_size(T, H0, I0, E, k)
        b = nv.moe_workspace_size(T, H1, I1, E, k)
        f16 = T * 4 * nv.operand_pitches(H1)[0] + T * k * 4 * nv.operand_pitches(I1)[0]
        assert b - a >= f16, (H1, I1, b - a, f16)     # one K step more alone adds a few KB


def test_binding_requires_device_tensors(nv):
    import torch
    with pytest.raises(TypeError):
        nv.quantize(torch.zeros((4, 16), dtype=torch.bfloat16))
