// Host-side launchers of the NVFP4 kernels. Each returns hipSuccess or the
// launch error; none synchronizes and none allocates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// Raise a kernel's dynamic-LDS limit to at least `bytes` on the current
// device. The attribute belongs to the (kernel, device) pair, so the largest
// value set so far is remembered per device (one cache per kernel, indexed by
// device); concurrent callers may both set it, which is harmless, and the
// remembered maximum only grows.
constexpr int kMaxDevices = 64;
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<int> (&done)[kMaxDevices]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return e;
    int cur = done[dev].load(std::memory_order_relaxed);
    while (cur < bytes && !done[dev].compare_exchange_weak(cur, bytes, std::memory_order_release)) {
    }
    return hipSuccess;
}

// Tile descriptor of the grouped GEMMs: rows [row_start, row_start + row_count)
// of the sorted slot order, all routed to `expert`.
struct Tile {
    int32_t expert;
    int32_t row_start;
    int32_t row_count;
    int32_t pad;
};

constexpr int kGemmBM = 256;      // rows per GEMM tile
constexpr int kGemmBN = 256;      // B columns per GEMM tile (L1: 128 gate + 128 up)
constexpr int kRouteThreads = 1024;
constexpr int kMaxExperts = 512;

// zero `n` 32-bit words
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);

// amax over `n` bf16 values (n % 8 == 0, 16-byte aligned) into *slot as float
// bits (atomic max; *slot must hold 0 or a smaller value).
hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* slot, hipStream_t s);

// Per-matrix amax of E matrices of `per` bf16 values each into slots[e].
hipError_t launch_amax_bf16_batched(const uint16_t* x, int64_t E, int64_t per, uint32_t* slots,
                                    hipStream_t s);

// Row pitches of the GEMM operand layout: packed data padded to whole
// 128-element K steps, scales to whole 8-byte steps; the exact f16 form of a
// quantized activation (e2m1 * e4m3 per element, the global scale left out)
// has the same padded length, 2 bytes per element.
__host__ __device__ inline int64_t pitch_q(int64_t K) { return (K / 2 + 63) / 64 * 64; }
__host__ __device__ inline int64_t pitch_sf(int64_t K) { return (K / 16 + 7) / 8 * 8; }
__host__ __device__ inline int64_t pitch_h(int64_t K) { return 4 * pitch_q(K); }

// Row-block quantization of x (M, K) with amax taken from *amax_slot, or with
// the global scale *gs_in when gs_in is not null. Rows at or beyond *m_dev
// (when m_dev is not null) are left untouched. gs_out receives gs.
// Output rows are ldq bytes (q) and ldsf bytes (sf) apart; when h is not null
// the dequantized f16 values (without gs) go to rows of pitch_h(K) bytes too.
hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, const int32_t* m_dev,
                             const uint32_t* amax_slot, uint8_t* q, int64_t ldq, uint8_t* sf,
                             int64_t ldsf, float* gs_out, hipStream_t s,
                             const float* gs_in = nullptr, uint16_t* h = nullptr);

// Quantized rows (M, K/2) + (M, K/16), K % 16 == 0, unpadded -> their exact
// f16 values in rows of pitch_h(K) bytes, zero padded.
hipError_t launch_dequant_rows_f16(const uint8_t* q, const uint8_t* sf, int64_t M, int64_t K,
                                   uint16_t* h, hipStream_t s);

// Packed weight layout. A weight matrix is N rows (one per output column) of
// pitch_q(K) bytes, K-packed; rows are grouped in blocks of 16, and inside a
// block the 32 bytes of one 64-element half of a K step of all 16 rows are
// stored together (512 bytes), half step after half step. So one half step of
// a 16-row block, the unit a GEMM stage holds, is contiguous, and so is one
// whole 128-element K step (1 KB, the unit a streaming load covers).
// Scales: per block, groups of four K steps (512 bytes): row c (0..15), pair q
// (0..3: groups 2q, 2q+1 of a step), step u of the four, then the two bytes.
// The two scale bytes a streaming lane needs for four consecutive steps are
// thus one 8-byte piece, and a wave reads 512 contiguous bytes at once.
constexpr int kWqStep = 16 * 64;      // bytes of one K step of a 16-row block
constexpr int kWqHalf = 16 * 32;      // bytes of one half step of a 16-row block
constexpr int kWsfQuad = 16 * 32;     // scale bytes of four K steps of a block
// offset of byte kh (0..pitch_q - 1) of packed row n
__host__ __device__ inline int64_t wq_off(int64_t n, int64_t ldq, int64_t kh) {
    return (n >> 4) * 16 * ldq + (kh >> 5) * kWqHalf + (n & 15) * 32 + (kh & 31);
}
// scale row pitch of the packed weights: whole groups of four K steps
__host__ __device__ inline int64_t pitch_wsf(int64_t K) { return (pitch_q(K) / 64 + 3) / 4 * 32; }
// offset of scale pair q of K step st of row n (two bytes: groups 8st + 2q, +1)
__host__ __device__ inline int64_t wsf_off(int64_t n, int64_t ldsf, int64_t st, int q) {
    return (n >> 4) * 16 * ldsf + (st >> 2) * kWsfQuad + (n & 15) * 32 + q * 8 + (st & 3) * 2;
}

// Canonical (R, C) byte matrices (E of them, R = K-packed rows, C = N) into
// the packed layout: element (r, c) goes to row c, byte r of a row of pitch
// ldo; scales (scale_layout) in the four-step groups above, data in steps of
// 64 bytes. Padding bytes are 0.
hipError_t launch_pack_weights(const uint8_t* in, int64_t E, int64_t R, int64_t C, uint8_t* out,
                               int64_t ldo, bool scale_layout, hipStream_t s);

// Per-part amax of E weight matrices (E, K, N), each split along N into
// `parts` equal column ranges (N / parts % 8 == 0), into slots[e * parts + p].
hipError_t launch_amax_cols(const uint16_t* w, int64_t E, int64_t K, int64_t N, int parts,
                            uint32_t* slots, hipStream_t s);

// Column-block quantization of E weight matrices (E, K, N), one amax (and one
// alpha out) per column part: amax_slots / alpha [e * parts + p].
hipError_t launch_quant_cols(const uint16_t* w, int64_t E, int64_t K, int64_t N, int parts,
                             const uint32_t* amax_slots, uint8_t* q, uint8_t* sf, float* alpha,
                             hipStream_t s);

// Quantization of the activation done inside the routing launch by extra
// work-groups, concurrently with the routing work-groups: each takes the
// global scale from gs_in (static), else from the maximum of the pre-pass's
// partial maxima, else reduces the whole amax itself (small inputs), then
// quantizes its share of the 16-element blocks.
struct SmallQuant {
    const uint16_t* x;
    const float* gs_in;      // static global scale, or null
    const uint32_t* amax_partials;  // partial maxima (bf16 magnitude bits) of x, or null
    int n_partials;
    int64_t M, K;
    uint8_t* q;
    int64_t ldq;
    uint8_t* sf;
    int64_t ldsf;
    float* gs;
    uint16_t* h;             // exact f16 values, rows of pitch_h(K) bytes, or null
};
constexpr int64_t kSmallQuantMax = 1 << 17;   // elements: larger inputs take the two-kernel path

// Routing in chunks: up to kRouteChunk slots take one routing work-group
// (which counts them itself); more take one work-group per chunk of
// route_chunk(S) slots (at most kRouteMaxChunks chunks), whose counts the
// pre-pass provides.
constexpr int64_t kRouteChunk = 4096;
constexpr int64_t kRouteMaxChunks = 64;
constexpr int kRouteMaxPartials = 1024;
int64_t route_chunk(int64_t S);
// number of partial maxima the pre-pass writes for n activation values
int route_amax_partials(int64_t n);

// Pre-pass of the routing launch: when x is not null, the partial maxima of
// its n bf16 values (route_amax_partials(n) words into `partial`); when S >
// kRouteChunk, the per-expert counts of every chunk of slots into wg_counts
// (chunks x E int32).
hipError_t launch_route_prepass(const uint16_t* x, int64_t n, uint32_t* partial, const int32_t* ids,
                                int64_t S, int E, int32_t* wg_counts, hipStream_t s);

// Routing tables and the tile list, plus the quantization of *xq when xq is
// not null (further work-groups of the same launch). Also zeroes `zero_slots`
// (n_zero words) before anything else in the layer runs. wg_counts: the
// pre-pass's chunk counts (used when S > kRouteChunk).
hipError_t launch_route(const int32_t* ids, int64_t S, int topk, int E, int BM, const int32_t* wg_counts,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row, Tile* tiles,
                        int32_t* num_tiles, uint32_t* zero_slots, int n_zero, const SmallQuant* xq,
                        hipStream_t s);

// Top-k router: ids (T, k) = the k largest logits of each row of (T, E)
// (ties: smaller expert first), weights (T, k) = softmax over the selected
// logits. E <= kMaxExperts, 1 <= k <= E.
hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids,
                             float* weights, hipStream_t s);

// y[t] = bf16(sum_j w[t][j] * o2[slot_row[t*topk+j]]) for rows that exist.
hipError_t launch_combine(const float* o2, const int32_t* slot_row, const float* weights,
                          int64_t T, int topk, int64_t H, uint16_t* y, hipStream_t s);

enum GemmMode { kGemmDense = 0, kGemmL1 = 1, kGemmL2 = 2 };

struct GemmParams {
    int mode;
    // A: rows of quantized activations, pitches pitch_q(K) / pitch_sf(K)
    // (weight-streaming kernel), or their exact f16 values, pitch pitch_h(K)
    // (tiled kernel)
    const uint8_t* aq;
    const uint8_t* asf;
    const uint16_t* ah;
    int64_t M;                 // dense: rows of A
    int64_t a_rows;            // rows in the A tensor (bounds of the buffer loads)
    const int32_t* a_gather;   // L1: sorted row -> slot index; token = slot / topk
    int topk;
    // B: per-expert weights, one K-packed row per output column (N rows of
    // pitch_q(K) bytes, scales N rows of pitch_wsf(K) bytes, packed layout)
    const uint8_t* bq;
    const uint8_t* bsf;
    int64_t N;                 // columns of B
    int64_t K;
    const float* a_gs;         // device scalar
    const float* b_alpha;      // device, alpha_stride per expert
    int alpha_stride;          // L1: 2 = (gate, up) per expert, else 1
    // grouped tiles
    const Tile* tiles;
    const int32_t* num_tiles;
    int64_t max_tiles;
    // outputs
    uint16_t* out_bf16;        // dense: (M, N); L1: act (S, I)
    float* out_f32;            // L2: (S, N)
    int64_t I;                 // L1: act columns (N = 2I)
    uint32_t* amax_slot;       // L1: act amax (atomic max of float bits)
    uint16_t* gu_tap;          // L1: null, or (rows, 2I) bf16 gate | up values out
    // dense with ksplit > 1: the K steps are cut into ksplit chunks, each
    // summed by its own work-groups into partial[chunk] (M, N) float32 (no
    // alpha); launch_splitk_reduce then forms out_bf16
    int ksplit;
    float* partial;
};

hipError_t launch_gemm(const GemmParams& p, hipStream_t s);

// Number of K chunks of the dense GEMM: 1 when its tiles fill half the GPU,
// else as many as keep (tiles x chunks) within one work-group per CU, each
// chunk at least 4 K steps and none empty.
int dense_ksplit(int64_t M, int64_t N, int64_t K);

// Rows per dense GEMM tile: 128 when 256-row tiles would fill less than half
// the GPU (the split-K regime: half-height tiles double the tiles and halve
// the K chunks, and with them the partial sums written and read back), else 256.
__host__ __device__ inline int64_t dense_tile_rows(int64_t M, int64_t N) {
    const int64_t t256 = (M + kGemmBM - 1) / kGemmBM * ((N + kGemmBN - 1) / kGemmBN);
    return t256 < 128 ? kGemmBM / 2 : kGemmBM;
}

// out[m][n] = bf16((a_gs[0] * b_alpha[0]) * sum over chunks c, in order, of
// partial[c][m][n]) for (M, N), N % 4 == 0.
hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const float* a_gs,
                                const float* b_alpha, uint16_t* out, hipStream_t s);

// Weight-streaming variant for tiles of at most kSkinnyBM rows (L1 / L2 only).
// It stages the tile's A rows whole in LDS: skinny_lds_bytes(K) must not
// exceed kSkinnyMaxLds (K up to about 17,000).
constexpr int kSkinnyBM = 16;
constexpr int64_t kSkinnyMaxLds = 150 * 1024;
__host__ __device__ inline int64_t skinny_lds_bytes(int64_t K) {
    return (int64_t)kSkinnyBM * (pitch_q(K) + 16 + pitch_sf(K));
}
hipError_t launch_skinny(const GemmParams& p, hipStream_t s);

}  // namespace nvfp4
