"""Block-scaled NVFP4 GEMM (test infrastructure).

C = (gs_A * alpha_B) * deq(A) @ deq(B), every product of an E2M1 value and an
E4M3 scale exact, accumulated in float64 and left unrounded.

The per-tensor / per-expert fp32 scales enter only as the GEMM's alpha and are
never folded into the E4M3 block scales (NVFP4 MegaMoE Debug Log, Hypothesis 3; src commit
log, per-expert global scale fix); the activation's global scale times the
weight's global scale is that alpha (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline": L1 and L2
GEMM lines). A is row-major with K packed along its rows; B is (K/2, N) packed
along K (NVFP4 MegaMoE Debug Log, Hypothesis 2 shapes; Hypothesis 5 packing).

Parity pins (tests/test_oracle_gemm.py): exact-rational brute force on tiny
shapes (oracle.loops), single-scale probes that move only their own row or
column by the predicted amount, the one-hot K-group probes, the constant-scale
case, and the unpack inverse on non-square operands.
"""
import numpy as np

from .quantize import dequantize_cols, dequantize_rows


def gemm(aq, asf, a_gs, bq, bsf, b_alpha):
    """Unrounded float64 result of the block-scaled GEMM, shape (M, N)."""
    a = dequantize_rows(aq, asf)
    b = dequantize_cols(bq, bsf)
    alpha = np.float64(np.float32(a_gs)) * np.float64(np.float32(b_alpha))
    return alpha * (a @ b)
