// NVFP4 dynamic quantization kernels (gfx950).
//
// The rule is the pages' stage_activation / weight-loader rule (NVFP4 MegaMoE Debug Log,
// Hypothesis 6 steps 1-5; "NVFP4 MoE Pipeline"): global scale amax/(6*448) over
// the whole tensor, E4M3 block scale block_amax/(6*global) per 16 elements,
// nearest E2M1, even element in the low nibble. The arithmetic order is fixed
// in common.hpp (quantize_block16) and is float32 IEEE throughout.
//
// Two passes: an amax pass (integer max of bf16 magnitude bits, which orders
// like the values; one atomic max per work-group) and a quantize pass in which
// every thread owns one 16-element block. Both are HBM-bound streaming kernels:
// 16-byte loads, consecutive threads on consecutive addresses.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
// 16-element blocks per thread and pass of the row quantizer
constexpr int kRowBlocks = 4;

__global__ void zero_u32_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

__device__ __forceinline__ void block_atomic_max(uint32_t v, uint32_t* slot) {
    __shared__ uint32_t red[kThreads / 64];
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = red[0];
        for (int w = 1; w < kThreads / 64; ++w) m = max(m, red[w]);
        // bf16 magnitude bits -> float bits of the same value
        atomicMax(slot, m << 16);
    }
}

// x: n bf16 values, n % 8 == 0, 16-byte aligned. Segment `blockIdx.y` of
// length `per` (batched variant) or the whole array (gridDim.y == 1).
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t* __restrict__ x, int64_t per,
                                                        uint32_t* __restrict__ slots) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x + (int64_t)blockIdx.y * per);
    const int64_t nvec = per / 8;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t m = 0;
    // four independent 16-byte loads in flight per iteration
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < nvec; i0 += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + u * stride;
            v[u] = i < nvec ? p[i] : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                m = max(m, v[u][c] & 0x7FFFu);
                m = max(m, (v[u][c] >> 16) & 0x7FFFu);
            }
    }
    block_atomic_max(m, slots + blockIdx.y);
}

// One thread per 16-element block of a row-major (M, K) bf16 matrix. The
// global scale is amax / 2688 of *amax_slot, or *gs_in when gs_in is not null
// (static scale); either way it is also written to *gs_out when gs_out is not
// null.
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ m_dev,
    const uint32_t* __restrict__ amax_slot, const float* __restrict__ gs_in, uint8_t* __restrict__ q,
    int64_t ldq, uint8_t* __restrict__ sf, int64_t ldsf, float* __restrict__ gs_out,
    uint8_t* __restrict__ h) {
    const QuantScales qs = gs_in ? scales_from_gs(*gs_in) : make_scales(__uint_as_float(*amax_slot));
    if (gs_out && blockIdx.x == 0 && threadIdx.x == 0) *gs_out = qs.gs;
    const int64_t rows = m_dev ? min((int64_t)(*m_dev), M) : M;
    const int64_t groups = K / 16;
    const int64_t nblocks = rows * groups;
    const int64_t step = (int64_t)gridDim.x * kThreads;
    int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // kRowBlocks blocks per thread and pass, all their loads issued before the
    // first is quantized (one block's two loads alone leave HBM underused)
    for (; b + (kRowBlocks - 1) * step < nblocks; b += kRowBlocks * step) {
        u32x4 v[kRowBlocks][2];
#pragma unroll
        for (int u = 0; u < kRowBlocks; ++u) {
            const u32x4* src = reinterpret_cast<const u32x4*>(x + (b + u * step) * 16);
            v[u][0] = src[0];
            v[u][1] = src[1];
        }
#pragma unroll
        for (int u = 0; u < kRowBlocks; ++u)
            quantize_row_block_loaded(v[u][0], v[u][1], b + u * step, groups, qs, q, ldq, sf, ldsf, h);
    }
    for (; b < nblocks; b += step) quantize_row_block(x, b, groups, qs, q, ldq, sf, ldsf, h);
}

// One thread per 16-element block of quantized rows (M, K/2) + (M, K/16):
// its exact f16 values into rows of pitch_h(K) bytes; the thread of a row's
// last block also zeroes the row's padding.
__global__ __launch_bounds__(kThreads) void dequant_rows_f16_kernel(const uint8_t* __restrict__ q,
                                                                    const uint8_t* __restrict__ sf,
                                                                    int64_t M, int64_t K,
                                                                    uint8_t* __restrict__ h) {
    // 32-bit index arithmetic: callers keep M * pitch_h(K) (> 32 M * K / 16) below 2^31
    const uint32_t groups = (uint32_t)(K / 16), ldh = (uint32_t)pitch_h(K);
    const uint32_t total = (uint32_t)M * groups;
    for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
        const uint32_t r = b / groups, g = b - r * groups;
        const u32x2 w = *reinterpret_cast<const u32x2*>(q + b * 8);
        store_block_f16(h + r * ldh + g * 32, w[0], w[1], sf[b]);
        if (g == groups - 1)
            for (uint32_t j = groups * 32; j < ldh; j += 16)
                *reinterpret_cast<u32x4*>(h + r * ldh + j) = (u32x4){0u, 0u, 0u, 0u};
    }
}

// Canonical (R, C) byte matrices -> the packed weight layout (launch.hpp),
// through a 64 x 64 LDS tile: reads along C are coalesced, writes land in
// 32-byte runs (data) or 2-byte pieces (scales).
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(
    const uint8_t* __restrict__ in, int64_t R, int64_t C, uint8_t* __restrict__ out, int64_t ldo,
    int scale_layout) {
    __shared__ uint8_t tile[64][65];
    const int64_t e = blockIdx.z;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const uint8_t* src = in + e * R * C;
    uint8_t* dst = out + e * C * ldo;
    for (int i = threadIdx.x; i < 64 * 64; i += kThreads) {
        const int rr = i >> 6, cc = i & 63;
        const int64_t r = r0 + rr, c = c0 + cc;
        tile[rr][cc] = (r < R && c < C) ? src[r * C + c] : (uint8_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += kThreads) {
        const int cc = i >> 6, rr = i & 63;
        const int64_t r = r0 + rr, c = c0 + cc;
        if (c < C && r < ldo) {
            const int64_t o = scale_layout ? wsf_off(c, ldo, r >> 3, (int)((r & 7) >> 1)) + (r & 1)
                                           : wq_off(c, ldo, r);
            dst[o] = tile[rr][cc];
        }
    }
}

// Per-part amax of E row-major (K, N) matrices split along N into `parts`
// column ranges of width Np (Np % 8 == 0): slot e * parts + p.
__global__ __launch_bounds__(kThreads) void amax_cols_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                             int64_t N, int64_t Np, int parts,
                                                             uint32_t* __restrict__ slots) {
    const int64_t e = blockIdx.y / parts, part = blockIdx.y - e * parts;
    const uint16_t* base = x + e * K * N + part * Np;
    const int64_t vrow = Np / 8, nvec = K * vrow;
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / vrow, c = i - r * vrow;
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + r * N + 8 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(v[k] & 0x7FFFu, (v[k] >> 16) & 0x7FFFu));
    }
    block_atomic_max(m, slots + blockIdx.y);
}

// One thread per (matrix e, K-group g, column n) of E row-major (K, N) bf16
// matrices; blocks run along K. Output byte [e][8g + j][n] holds the nibbles
// of k = 16g + 2j (low) and 16g + 2j + 1 (high). Column n belongs to part
// n / Np of its matrix, whose amax is amax_slots[e * parts + n / Np] and whose
// global scale goes to alpha[e * parts + n / Np].
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const uint16_t* __restrict__ w, int64_t K, int64_t N, int64_t Np, int parts,
    const uint32_t* __restrict__ amax_slots, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
    float* __restrict__ alpha) {
    const int64_t e = blockIdx.y;
    const int64_t groups = K / 16;
    const int64_t per = groups * N;
    const uint16_t* we = w + e * K * N;
    if (blockIdx.x == 0 && (int)threadIdx.x < parts)
        alpha[e * parts + threadIdx.x] = make_scales(__uint_as_float(amax_slots[e * parts + threadIdx.x])).gs;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < per;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t g = i / N, n = i - g * N;
        const QuantScales qs = make_scales(__uint_as_float(amax_slots[e * parts + n / Np]));
        uint32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t lo = we[(16 * g + 2 * j) * N + n];
            const uint32_t hi = we[(16 * g + 2 * j + 1) * N + n];
            v[j] = lo | (hi << 16);
        }
        uint32_t packed[2];
        const uint32_t code = quantize_block16(v, qs, packed);
        uint8_t* qe = q + e * (K / 2) * N;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t word = packed[j >> 2];
            qe[(8 * g + j) * N + n] = (uint8_t)(word >> (8 * (j & 3)));
        }
        sf[e * per + g * N + n] = (uint8_t)code;
    }
}

int grid_for(int64_t work, int64_t cap) {
    int64_t g = (work + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
    zero_u32_kernel<<<1, 64, 0, s>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* slot, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    // at most 256 work-groups: every work-group ends with one atomic on the
    // same slot, and those serialize (about 10 ns each, measured: 2048
    // work-groups took 29.6 us for 58.7 MB, 256 took 12.3 us)
    const int g = grid_for(n / 8, 256);
    amax_kernel<<<dim3(g, 1), kThreads, 0, s>>>(x, n, slot);
    return hipGetLastError();
}

hipError_t launch_amax_bf16_batched(const uint16_t* x, int64_t E, int64_t per, uint32_t* slots,
                                    hipStream_t s) {
    if (E <= 0 || per <= 0) return hipSuccess;
    const int g = grid_for(per / 8, 512);
    amax_kernel<<<dim3(g, (unsigned)E), kThreads, 0, s>>>(x, per, slots);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int64_t K, const int32_t* m_dev,
                             const uint32_t* amax_slot, uint8_t* q, int64_t ldq, uint8_t* sf,
                             int64_t ldsf, float* gs_out, hipStream_t s, const float* gs_in,
                             uint16_t* h) {
    const int g = grid_for((M * (K / 16) + kRowBlocks - 1) / kRowBlocks, 1 << 20);
    quant_rows_kernel<<<g, kThreads, 0, s>>>(x, M, K, m_dev, amax_slot, gs_in, q, ldq, sf, ldsf, gs_out,
                                             reinterpret_cast<uint8_t*>(h));
    return hipGetLastError();
}

hipError_t launch_dequant_rows_f16(const uint8_t* q, const uint8_t* sf, int64_t M, int64_t K,
                                   uint16_t* h, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const int g = grid_for(M * (K / 16), 1 << 16);
    dequant_rows_f16_kernel<<<g, kThreads, 0, s>>>(q, sf, M, K, reinterpret_cast<uint8_t*>(h));
    return hipGetLastError();
}

hipError_t launch_pack_weights(const uint8_t* in, int64_t E, int64_t R, int64_t C, uint8_t* out,
                               int64_t ldo, bool scale_layout, hipStream_t s) {
    if (E <= 0 || C <= 0) return hipSuccess;
    // rows of the output beyond R (padding) are covered by extra row tiles
    const int64_t rt = (ldo + 63) / 64, ct = (C + 63) / 64;
    pack_weights_kernel<<<dim3((unsigned)ct, (unsigned)rt, (unsigned)E), kThreads, 0, s>>>(
        in, R, C, out, ldo, scale_layout ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_amax_cols(const uint16_t* w, int64_t E, int64_t K, int64_t N, int parts,
                            uint32_t* slots, hipStream_t s) {
    if (E <= 0 || parts <= 0) return hipSuccess;
    const int64_t Np = N / parts;
    const int g = grid_for(K * Np / 8, 512);
    amax_cols_kernel<<<dim3(g, (unsigned)(E * parts)), kThreads, 0, s>>>(w, K, N, Np, parts, slots);
    return hipGetLastError();
}

hipError_t launch_quant_cols(const uint16_t* w, int64_t E, int64_t K, int64_t N, int parts,
                             const uint32_t* amax_slots, uint8_t* q, uint8_t* sf, float* alpha,
                             hipStream_t s) {
    if (E <= 0) return hipSuccess;
    const int g = grid_for((K / 16) * N, 4096);
    quant_cols_kernel<<<dim3(g, (unsigned)E), kThreads, 0, s>>>(w, K, N, N / parts, parts, amax_slots,
                                                                  q, sf, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
