/*
 * nvfp4moe.h - C ABI of the NVFP4 mixture-of-experts expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * Formats (the pages: "nvfp4-megamoe-kernel" DEBUG_LOG, the "NVFP4 MoE
 * Pipeline" and Hypotheses 2, 3, 5, 6; its later revision's "input_scale red
 * herring" and code-review items; the src commit log's quantizer, E4M3 and
 * gate/up fixes):
 *
 *   - packed FP4 (E2M1): one byte holds two elements; the even element is in
 *     the low nibble, the odd one in the high nibble. A nibble is
 *     sign-magnitude: bit 3 the sign, bits 2:0 index {0,0.5,1,1.5,2,3,4,6}.
 *   - block scales: one byte per 16 consecutive elements along the reduction
 *     (K) axis, an OCP E4M3FN bit pattern (bias 7, max 448), reinterpreted,
 *     never value-converted.
 *   - global scale: float32 amax / (6 * 448) over the whole quantized tensor.
 *     It is kept out of the E4M3 bytes and enters the GEMMs as alpha.
 *   - dequantized element = e2m1(nibble) * e4m3(scale byte) * global scale.
 *
 * Layouts (all row-major):
 *   activation   x        (M, K) bf16 (uint16 bit patterns)
 *   quantized A  q        (M, K/2) bytes, packed along K
 *                sf       (M, K/16) E4M3 bytes, sf[m][g] covers k in [16g, 16g+16)
 *   canonical    w        (E, K/2, N) bytes, packed along K: byte [e][kh][n]
 *   weights               holds W[2kh][n] (low) and W[2kh+1][n] (high)
 *                w_sf     (E, K/16, N) E4M3 bytes
 *                w_alpha  (E) float32 weight global scales (dequant direction)
 *   packed       w_t      E * N * pitch_q(K) bytes: row n of matrix e holds
 *   weights               column n of W[e], packed along K like an A row
 *                         (byte kh = W[2kh][n] | W[2kh+1][n] << 4), zero-padded
 *                         to pitch_q(K) bytes; rows are stored in blocks of 16
 *                         and inside a block by 128-element K step: byte kh of
 *                         row n is at
 *                           e * N * pitch_q(K) + (n / 16) * 16 * pitch_q(K)
 *                           + (kh / 64) * 1024 + (n % 16) * 64 + kh % 64
 *                w_sf_t   E * N * pitch_wsf(K) E4M3 bytes, zero-padded, in the
 *                         same 16-row blocks, by groups of four K steps (st =
 *                         g / 8 is the step of scale group g): scale g of row
 *                         n is at
 *                           e * N * pitch_wsf(K) + (n / 16) * 16 * pitch_wsf(K)
 *                           + (st / 4) * 512 + (n % 16) * 32
 *                           + ((g % 8) / 2) * 8 + (st % 4) * 2 + g % 2
 *                         so the two groups of one 32-element quarter of a
 *                         step sit together for four consecutive steps.
 *   pitch_q(K)   = K/2 rounded up to a multiple of 64 bytes (a 128-element step)
 *   pitch_sf(K)  = K/16 rounded up to a multiple of 8 bytes (activation scales)
 *   pitch_wsf(K) = 32 bytes per group of four steps: pitch_q(K) / 64 rounded up
 *                  to a multiple of 4, times 8
 *   The packed weights are the canonical ones with every matrix byte-transposed
 *   (the pages' GEMM took its weight operand column-major) and blocked so that
 *   one K step of 16 rows, the unit a matrix-core operand load covers, is one
 *   contiguous kilobyte. They are made once, at load time, by
 *   nvfp4_prepack_weights and are what the GEMMs read. N % 16 == 0.
 *   w13 is the plain concatenation [gate; up] along N: columns [0, I) are the
 *   gate projection, [I, 2I) the up projection (rows [0, I) / [I, 2I) packed).
 *
 * Ownership and execution. Every pointer argument is a DEVICE pointer unless
 * its comment says host. The caller owns all memory, including workspaces; the
 * library allocates nothing, keeps no state besides cached device properties,
 * never synchronizes the host with the device, and enqueues all work on the
 * caller's stream in order. Entry points are safe to call concurrently on
 * different streams with different workspaces. No hipMemset is issued, so the
 * calls may be captured into a HIP graph.
 *
 * Errors. Arguments are validated on the host before anything is enqueued;
 * a failed validation returns a non-zero status and enqueues nothing. Launch
 * errors are reported as NVFP4_EHIP. Inputs that are NaN or infinite give
 * unspecified outputs.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_EINVAL = 1,       /* null pointer or negative size */
    NVFP4_ESHAPE = 2,       /* a K dimension not a multiple of 16, topk > E, ... */
    NVFP4_EWORKSPACE = 3,   /* workspace missing, too small or misaligned */
    NVFP4_EHIP = 4,         /* a HIP call or kernel launch failed */
    NVFP4_EDEVICE = 5       /* the current device is not gfx950 */
} nvfp4_status;

/* Human-readable text of a status code (host string, static storage). */
const char* nvfp4_strerror(int status);

/* Library ABI version: (major << 16) | minor. */
int nvfp4_version(void);

/* ------------------------------------------------------------------------ *
 * nvfp4_quantize - dynamic NVFP4 quantization of an activation
 * (the pages' stage_activation: hidden -> x_fp4, x_sf, input_global_scale).
 *
 *   x   (M, K) bf16, K % 16 == 0
 *   q   (M, K/2) bytes out;  sf (M, K/16) bytes out
 *   gs  one float32 out: amax(|x|) / 2688, computed in IEEE float32
 *
 * Every step is IEEE float32 round-to-nearest-even, in this order:
 *   gs = amax / 2688;  s = min(bmax / (6 * gs), 448) (0 when gs == 0);
 *   scale byte = E4M3 nearest-even of s;  den = e4m3(byte) * gs;
 *   nibble = sign(x) << 3 | nearest-even E2M1 magnitude of |x| / den
 *   (magnitude 0 when den == 0; |x| / den above 6 saturates to 6).
 * Results are bit-identical to that definition.
 *
 * Workspace: nvfp4_quantize_workspace(M, K) bytes, 256-byte aligned.
 * M == 0 is valid and enqueues one tiny kernel that writes gs = 0.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace(int64_t M, int64_t K);
int nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K,
                   uint8_t* q, uint8_t* sf, float* gs,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_quantize_weights - the loader's rule for a batch of E weight
 * matrices (DEBUG_LOG, Hypothesis 6 steps 1-5): per matrix one global scale,
 * blocks of 16 along K, output in the K-packed weight layout.
 *
 *   w        (E, K, N) bf16, W[e] is the math layout (y = x @ W[e]), K % 16 == 0
 *   q        (E, K/2, N) bytes out;  sf (E, K/16, N) bytes out
 *   alpha    (E) float32 out: amax(|W[e]|) / 2688
 *
 * The arithmetic is the one of nvfp4_quantize applied to W[e] transposed.
 * Workspace: nvfp4_quantize_weights_workspace(E, K, N) bytes.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_weights_workspace(int64_t E, int64_t K, int64_t N);
int nvfp4_quantize_weights(const uint16_t* w, int64_t E, int64_t K, int64_t N,
                           uint8_t* q, uint8_t* sf, float* alpha,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_operand_pitches - the padded row pitches of the packed weight layout
 * (and of the quantized operands inside the expert layer's workspace).
 *   K > 0, K % 16 == 0; ldq, ldsf, ldwsf: host int64 out (pitch_q(K),
 *   pitch_sf(K), pitch_wsf(K)). Returns NVFP4_ESHAPE for K % 16 != 0 and
 *   NVFP4_EINVAL for K <= 0 or a null pointer.
 * ------------------------------------------------------------------------ */
int nvfp4_operand_pitches(int64_t K, int64_t* ldq, int64_t* ldsf, int64_t* ldwsf);

/* ------------------------------------------------------------------------ *
 * nvfp4_prepack_weights - canonical (K-packed, N fastest) quantized weights to
 * the packed layout the GEMMs read (a blocked byte transpose per matrix,
 * padding bytes written as zero). A pure data movement, no arithmetic.
 *
 *   w (E, K/2, N), w_sf (E, K/16, N): canonical bytes (nvfp4_quantize_weights)
 *   w_t (E * N * pitch_q(K) bytes), w_sf_t (E * N * pitch_wsf(K) bytes): packed
 *   out, separate buffers (no in-place), w_t 16-byte and w_sf_t 8-byte aligned.
 *   K % 16 == 0, N % 16 == 0, E <= 65535. E == 0 is valid and enqueues nothing.
 * ------------------------------------------------------------------------ */
int nvfp4_prepack_weights(const uint8_t* w, const uint8_t* w_sf, int64_t E, int64_t K, int64_t N,
                          uint8_t* w_t, uint8_t* w_sf_t, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_gemm - block-scaled NVFP4 GEMM, one expert
 * (DEBUG_LOG, "NVFP4 MoE Pipeline": GEMM with alpha = igs * weight global).
 *
 *   out[m][n] = bf16( (a_gs[0] * b_alpha[0]) * sum_k deqA[m][k] * deqB[k][n] )
 *
 *   aq (M, K/2), asf (M, K/16): the quantized activation (nvfp4_quantize),
 *           aq 16-byte and asf 8-byte aligned
 *   a_gs    one float32, the activation's global scale
 *   bq (N * K/2 bytes), bsf (N * pitch_wsf(K) bytes): one packed weight
 *           matrix (nvfp4_prepack_weights with E = 1; for K % 128 == 0,
 *           pitch_q(K) is exactly K/2), bq 16-byte and bsf 8-byte aligned
 *   b_alpha one float32
 *   out (M, N) bf16
 * Products of dequantized elements are exact; the sum is float32; the alpha
 * product and its multiply are float32; the one bf16 rounding is the last step.
 * K % 128 == 0, N % 16 == 0, M * K/2 and N * K/2 below 2^31. No workspace.
 * ------------------------------------------------------------------------ */
int nvfp4_gemm(const uint8_t* aq, const uint8_t* asf, const float* a_gs,
               const uint8_t* bq, const uint8_t* bsf, const float* b_alpha,
               int64_t M, int64_t N, int64_t K, uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_moe_forward - the five-stage NVFP4 expert layer on one GPU's experts
 * (DEBUG_LOG, "NVFP4 MoE Pipeline"):
 *   1. quantize x (T, H) -> xq, xsf, gs1 (nvfp4_quantize's rule, one gs1 over x)
 *   2. route: one slot per (t, j) whose id topk_ids[t][j] is in [0, E);
 *      slots with other ids are skipped and contribute nothing
 *   3. L1: gate_up = bf16((gs1 * w13_alpha[e]) * xq[t] @ w13[e])   (S, 2I)
 *   4. act = bf16(silu(gate) * up) in float32, silu(z) = z / (1 + exp(-z));
 *      quantize all valid slots' act rows -> aq, asf, gs2 (one gs2)
 *   5. L2: o[s] = (gs2 * w2_alpha[e]) * aq[s] @ w2[e] in float32, then
 *      y[t] = bf16( sum_j topk_weights[t][j] * o[slot(t, j)] ), float32, j order
 *
 *   x             (T, H) bf16
 *   topk_ids      (T, topk) int32
 *   topk_weights  (T, topk) float32, used as given (no renormalization)
 *   w13 (E * 2I * pitch_q(H) bytes), w13_sf (E * 2I * pitch_wsf(H)), w13_alpha (E)
 *   w2  (E * H * pitch_q(I) bytes),  w2_sf  (E * H * pitch_wsf(I)),  w2_alpha  (E)
 *                 packed weights (nvfp4_prepack_weights of the canonical
 *                 (E, H/2, 2I) and (E, I/2, H) tensors); w13, w2 16-byte and
 *                 the scale tensors 8-byte aligned
 *   y             (T, H) bf16 out
 *   H % 16 == 0, I % 16 == 0, 1 <= topk <= E, T >= 0; each of
 *   2I * pitch_q(H), H * pitch_q(I), T * pitch_q(H), T * topk * pitch_q(I)
 *   below 2^31 (32-bit buffer offsets), else NVFP4_ESHAPE.
 *
 * Workspace: nvfp4_moe_workspace(T, H, I, E, topk) bytes, 256-byte aligned.
 * The intermediates stay in the workspace after the call; their byte offsets
 * are given by nvfp4_moe_workspace_layout (for tests and debugging).
 *
 * stage_events: NULL, or a host array of NVFP4_MOE_NUM_EVENTS hipEvent_t
 * created by the caller; event i is recorded on `stream` before stage i's
 * first launch and the last one after the last launch, so that
 * hipEventElapsedTime(ev[i], ev[i+1]) is stage i's device time.
 * ------------------------------------------------------------------------ */
enum {
    NVFP4_MOE_STAGE_ROUTE = 0,      /* routing tables, tile list */
    NVFP4_MOE_STAGE_QUANT_X = 1,    /* amax + quantization of x */
    NVFP4_MOE_STAGE_L1 = 2,         /* L1 grouped GEMM + fused SiLU*up */
    NVFP4_MOE_STAGE_REQUANT = 3,    /* quantization of act */
    NVFP4_MOE_STAGE_L2 = 4,         /* L2 grouped GEMM */
    NVFP4_MOE_STAGE_COMBINE = 5,    /* weighted combine */
    NVFP4_MOE_NUM_STAGES = 6,
    NVFP4_MOE_NUM_EVENTS = 7
};

/* Offsets (bytes from the workspace base) of the intermediates, indexed by: */
enum {
    NVFP4_MOE_WS_XQ = 0,            /* (T, pitch_q(H)) bytes, row t's first H/2 are x's */
    NVFP4_MOE_WS_XSF = 1,           /* (T, pitch_sf(H)) bytes, first H/16 used */
    NVFP4_MOE_WS_GS1 = 2,           /* float32 */
    NVFP4_MOE_WS_GS2 = 3,           /* float32 */
    NVFP4_MOE_WS_COUNTS = 4,        /* int32 (E): valid slots per expert */
    NVFP4_MOE_WS_OFFSETS = 5,       /* int32 (E+1): first sorted row of each expert */
    NVFP4_MOE_WS_SORTED_SLOT = 6,   /* int32 (S): slot t*topk+j of each sorted row */
    NVFP4_MOE_WS_SLOT_ROW = 7,      /* int32 (S): sorted row of each slot, -1 if skipped */
    NVFP4_MOE_WS_ACT = 8,           /* bf16 (S, I), sorted rows */
    NVFP4_MOE_WS_AQ = 9,            /* (S, pitch_q(I)) bytes, sorted rows, first I/2 used */
    NVFP4_MOE_WS_ASF = 10,          /* (S, pitch_sf(I)) bytes, sorted rows, first I/16 used */
    NVFP4_MOE_WS_O2 = 11,           /* float32 (S, H), sorted rows, weight not applied */
    NVFP4_MOE_WS_NUM = 12
};

size_t nvfp4_moe_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);
/* offsets: host array of NVFP4_MOE_WS_NUM entries, filled. */
int nvfp4_moe_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                               size_t* offsets);

int nvfp4_moe_forward(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                      const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha,
                      int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                      uint16_t* y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, hipEvent_t* stage_events);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
