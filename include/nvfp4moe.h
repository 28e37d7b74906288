/*
 * nvfp4moe.h - C ABI of the NVFP4 mixture-of-experts expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * Formats (the pages: the NVFP4 MegaMoE Debug Log of nvfp4-megamoe-kernel, the "NVFP4 MoE
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
 *                         and inside a block by 64-element half step (32 bytes
 *                         of each of the 16 rows): byte kh of row n is at
 *                           e * N * pitch_q(K) + (n / 16) * 16 * pitch_q(K)
 *                           + (kh / 32) * 512 + (n % 16) * 32 + kh % 32
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
 *   pitch_h(K)   = 4 * pitch_q(K): bytes of a row of f16 values, K rounded up
 *                  to whole 128-element steps
 *   The packed weights are the canonical ones with every matrix byte-transposed
 *   (the pages' GEMM took its weight operand column-major) and blocked so that
 *   one 64-element half step of 16 rows (what a tiled-GEMM stage holds) is 512
 *   contiguous bytes and one 128-element K step (what a streaming load covers)
 *   one contiguous kilobyte. They are made once, at load time, by
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
    NVFP4_EDEVICE = 5,      /* the current device is not gfx950 */
    NVFP4_ESCRATCH = 6      /* nvfp4_moe_forward_noalloc: the problem needs more
                               than NVFP4_MOE_SCRATCH_BYTES of workspace */
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
 * nvfp4_quantize_static - stage_activation with a global scale given by the
 * caller instead of amax / 2688 of x (the later revision of the NVFP4 MegaMoE Debug Log, "input_scale
 * red herring": a calibrated activation scale in that role; the pages found
 * the checkpoint's calibrated value unsuitable for their runtime data, so the
 * scale is entirely the caller's choice). Saves the amax pass.
 *
 *   x   (M, K) bf16, K % 16 == 0, 16-byte aligned
 *   gs  one float32 (device), the global scale to use
 *   q   (M, K/2) bytes out (8-byte aligned);  sf (M, K/16) bytes out
 *
 * The arithmetic is nvfp4_quantize's with gs taken as given: a block whose
 * amax exceeds 6 * 448 * gs gets scale 448 (byte 0x7E) and its elements
 * saturate at magnitude 6; gs <= 0 (or NaN) gives all-zero scale bytes and
 * magnitudes (sign bits kept). M == 0 enqueues nothing. No workspace.
 * ------------------------------------------------------------------------ */
int nvfp4_quantize_static(const uint16_t* x, int64_t M, int64_t K, const float* gs,
                          uint8_t* q, uint8_t* sf, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_quantize_weights - the loader's rule for a batch of E weight
 * matrices (NVFP4 MegaMoE Debug Log, Hypothesis 6 steps 1-5): per matrix one global scale,
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
 * nvfp4_quantize_weights_parts - the weight rule with one global scale per
 * column part: W[e] (K, N) is split along N into `parts` equal ranges and
 * each range is quantized as its own matrix (own amax, own alpha). For w13 =
 * [gate | up] with parts = 2 these are the per-half weight global scales of
 * the NVFP4 MegaMoE Debug Log ("Bugs Fixed": a global scale of shape (2,) applied per half;
 * later revision, code-review item 5: a per-column alpha), which the layer
 * takes through nvfp4_moe_options.w13_alpha_per_half.
 *
 *   w, q, sf  as nvfp4_quantize_weights
 *   alpha     (E, parts) float32 out: alpha[e][p] = amax(|W[e][:, part p]|) / 2688
 *   1 <= parts <= 16, E * parts <= 65535, N % parts == 0, (N / parts) % 8 == 0,
 *   else NVFP4_ESHAPE.
 * Workspace: nvfp4_quantize_weights_parts_workspace(E, K, N, parts) bytes,
 * 256-byte aligned. parts = 1 gives exactly nvfp4_quantize_weights' output.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_weights_parts_workspace(int64_t E, int64_t K, int64_t N, int64_t parts);
int nvfp4_quantize_weights_parts(const uint16_t* w, int64_t E, int64_t K, int64_t N,
                                 int64_t parts, uint8_t* q, uint8_t* sf, float* alpha,
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
 * (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline": GEMM with alpha = igs * weight global).
 *
 *   out[m][n] = bf16( (a_gs[0] * b_alpha[0]) * sum_k deqA[m][k] * deqB[k][n] )
 *
 *   aq (M, K/2), asf (M, K/16): the quantized activation (nvfp4_quantize),
 *           aq 8-byte aligned
 *   a_gs    one float32, the activation's global scale
 *   bq (N * pitch_q(K) bytes), bsf (N * pitch_wsf(K) bytes): one packed weight
 *           matrix (nvfp4_prepack_weights with E = 1), bq 16-byte and bsf
 *           8-byte aligned
 *   b_alpha one float32
 *   out (M, N) bf16
 * Products of dequantized elements are exact; the sum is float32; the alpha
 * product and its multiply are float32; the one bf16 rounding is the last step.
 * K % 16 == 0, N % 16 == 0, M * pitch_h(K) and N * pitch_q(K) below 2^31
 * (pitch_h(K) = 4 * pitch_q(K)), else NVFP4_ESHAPE.
 *
 * Workspace: nvfp4_gemm_workspace(M, N, K) bytes, 256-byte aligned. It
 * receives A in its exact f16 form (e2m1 * e4m3 per element, M rows of
 * pitch_h(K) bytes padded with zeros to whole 128-element steps), the operand
 * the matrix cores read, and, when 256 x 256 output tiles would fill less
 * than half the GPU, the float32 partial sums of the chunks K is cut into
 * (the tiles are then 128 x 256; one M x N plane per chunk, added in chunk
 * order before alpha and the bf16 rounding). nvfp4_gemm_workspace returns 0
 * for invalid sizes.
 * ------------------------------------------------------------------------ */
size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K);
int nvfp4_gemm(const uint8_t* aq, const uint8_t* asf, const float* a_gs,
               const uint8_t* bq, const uint8_t* bsf, const float* b_alpha,
               int64_t M, int64_t N, int64_t K, uint16_t* out,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * nvfp4_moe_forward - the five-stage NVFP4 expert layer on one GPU's experts
 * (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline"):
 *   1. quantize x (T, H) -> xq, xsf, gs1 (nvfp4_quantize's rule, one gs1 over x)
 *   2. route: one slot per (t, j) whose id topk_ids[t][j] is in [0, E);
 *      slots with other ids are skipped and contribute nothing
 *   3. L1: gate_up = bf16((gs1 * w13_alpha[e]) * xq[t] @ w13[e])   (S, 2I)
 *   4. act = bf16(silu(gate) * up), silu(z) = z / (1 + exp(-z)), rounded to
 *      nearest-even from the float64 value of that formula (computed in
 *      float32 where float32 decides the same rounding; where 1 + exp(-gate)
 *      is 1 in float64 the product is first moved one float64 step toward
 *      zero, as the exact value lies just inside it);
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
 *   2I * pitch_q(H), H * pitch_q(I), T * pitch_h(H), T * topk * pitch_h(I)
 *   below 2^31 (32-bit buffer offsets), else NVFP4_ESHAPE.
 *
 * Kernels: batches of at most 16 valid slots per expert on average take
 * weight-streaming GEMMs whose LDS holds a 16-row tile of the activation
 * (so H and I up to about 17,000); other batches, and larger H or I, take
 * the tiled GEMMs, whose LDS use does not depend on K. The choice is made on
 * the host from the shapes alone.
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
    NVFP4_MOE_STAGE_ROUTE = 0,      /* amax of x, then routing tables, tile list
                                       and the quantization of x (one launch) */
    NVFP4_MOE_STAGE_QUANT_X = 1,    /* empty: x is quantized with the routing */
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
    NVFP4_MOE_WS_XH = 12,           /* f16 (T, pitch_h(H) / 2): the exact values of xq
                                       (e2m1 * e4m3), read by the tiled L1 GEMM;
                                       empty when the batch takes the weight-
                                       streaming kernels (at most 16 slots per
                                       expert on average) */
    NVFP4_MOE_WS_AH = 13,           /* f16 (S, pitch_h(I) / 2): the exact values of
                                       aq, sorted rows; empty like XH */
    NVFP4_MOE_WS_NUM = 14
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

/* ------------------------------------------------------------------------ *
 * nvfp4_moe_forward_ex - nvfp4_moe_forward with options (a NULL options
 * pointer, or a zero-initialized struct, is exactly nvfp4_moe_forward):
 *
 *   w13_alpha_per_half  0: w13_alpha is (E), one weight global scale per
 *                       expert; 1: w13_alpha is (E, 2) float32, [e][0] for
 *                       the gate columns [0, I) and [e][1] for the up columns
 *                       [I, 2I) (nvfp4_quantize_weights_parts with parts = 2):
 *                       stage 3 becomes gate = bf16((gs1 * w13_alpha[e][0]) *
 *                       ...), up = bf16((gs1 * w13_alpha[e][1]) * ...).
 *                       Other values: NVFP4_EINVAL.
 *   x_global_scale      NULL: gs1 = amax(x) / 2688 (dynamic); else a device
 *                       float32 (4-byte aligned) used as gs1 for stage 1, as
 *                       in nvfp4_quantize_static (no amax pass; blocks beyond
 *                       6 * 448 * gs1 saturate). gs2 stays dynamic.
 *   gate_up_tap         NULL (production), or a device buffer of
 *                       T * topk * 2I bf16 values (4-byte aligned) that
 *                       receives stage 3's rounded output: row r (sorted
 *                       order, as the act rows in the workspace; rows beyond
 *                       the valid slots are not written) holds the gate
 *                       values in columns [0, I) and the up values in
 *                       [I, 2I), exactly the bf16 values the SiLU consumes.
 *                       A debugging and test tap (the pages' lesson: compare
 *                       each stage on identical inputs); it adds stores and
 *                       changes no other output.
 * ------------------------------------------------------------------------ */
typedef struct nvfp4_moe_options {
    int32_t w13_alpha_per_half;
    int32_t reserved;               /* must be 0 (else NVFP4_EINVAL) */
    const float* x_global_scale;
    uint16_t* gate_up_tap;
} nvfp4_moe_options;

int nvfp4_moe_forward_ex(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                         const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha,
                         int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                         uint16_t* y, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipEvent_t* stage_events,
                         const nvfp4_moe_options* options);

/* ------------------------------------------------------------------------ *
 * nvfp4_moe_forward_noalloc - nvfp4_moe_forward_ex for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * semantics and results as nvfp4_moe_forward_ex, minus the workspace: the
 * library keeps it in a static device array of NVFP4_MOE_SCRATCH_BYTES
 * (32 MiB) per GPU, held from the library's load until the process ends, and
 * this call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine). 32 MiB covers decode-sized batches, e.g. up to about 110 tokens
 * at top-8 with hidden 7168 and intermediate 3072; compare
 * nvfp4_moe_workspace(T, H, I, E, topk) with NVFP4_MOE_SCRATCH_BYTES.
 *
 * Errors: those of nvfp4_moe_forward_ex, and NVFP4_ESCRATCH (before anything
 * is enqueued) when nvfp4_moe_workspace(T, H, I, E, topk) exceeds
 * NVFP4_MOE_SCRATCH_BYTES. The first call on a device looks up that device's
 * copy of the array (a host-side runtime query, no allocation).
 *
 * Sharing: every call on one GPU uses that GPU's single array, which keeps
 * the previous call's intermediates (no call relies on its contents: each
 * writes what it reads). Calls that may overlap on one GPU (different
 * streams, or graph replays in flight together) race on it and must be
 * serialized by the caller. The intermediates are not exposed: use
 * nvfp4_moe_forward with a workspace to inspect them.
 * ------------------------------------------------------------------------ */
#define NVFP4_MOE_SCRATCH_BYTES (32u << 20)
int nvfp4_moe_forward_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                              const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                              const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha,
                              int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                              uint16_t* y, hipStream_t stream, hipEvent_t* stage_events,
                              const nvfp4_moe_options* options);

/* ------------------------------------------------------------------------ *
 * nvfp4_route_topk - the router that produces the layer's topk_ids and
 * topk_weights (the weights of the routing-weighted scatter that ends the
 * NVFP4 MegaMoE Debug Log's "NVFP4 MoE Pipeline"; the pages do not define the
 * router, this is the usual top-k with renormalized softmax):
 *
 *   logits        (T, E) float32, finite
 *   topk_ids      (T, topk) int32 out: the topk largest logits of each row in
 *                 descending order; among equal values the smaller expert
 *                 index comes first
 *   topk_weights  (T, topk) float32 out: exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *                 over the selected logits l_0 >= l_1 >= ..., float32, the sum
 *                 in selection order (a renormalized softmax; rows sum to 1
 *                 up to rounding)
 *   1 <= topk <= E <= 512, T * E < 2^31, else NVFP4_ESHAPE; pointers 4-byte
 *   aligned. T == 0 enqueues nothing. The ids are exact (comparisons of the
 *   given float32 values); the weights carry float32 rounding and expf.
 * ------------------------------------------------------------------------ */
int nvfp4_route_topk(const float* logits, int64_t T, int64_t E, int64_t topk,
                     int32_t* topk_ids, float* topk_weights, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
