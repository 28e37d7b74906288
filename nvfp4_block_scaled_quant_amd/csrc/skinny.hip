// Weight-streaming grouped GEMMs for small batches (decode): the same two
// expert GEMMs as gemm.hip (DEBUG_LOG, "NVFP4 MoE Pipeline", L1 with fused
// SiLU(gate) * up and L2), for tiles of at most 16 rows.
//
// With a handful of rows per expert the layer is bound by reading the expert
// weights from HBM once, so the kernel is built around the weight stream:
//
// * A work-group owns one 16-row tile and one slab of 128 weight rows (output
//   columns; for L1: 64 gate columns and the 64 matching up columns). Its 16 A
//   rows are staged once in LDS, still packed.
// * Each of the 4 waves streams a quarter of K. Per 128-element K step, lane
//   (c, q) = (lane % 16, lane / 16) loads 16 contiguous bytes (32 K values,
//   [32q, 32q + 32) of the step) from each of 8 weight rows: column c of the
//   8 MFMA column blocks f (block f holds weight rows 16f + c of the slab).
//   In the packed weight layout one such load instruction (16 rows x 64 bytes
//   of one K step of a 16-row block) reads one contiguous kilobyte.
//   Dword s of a load is the B operand of v_mfma_f32_16x16x32_f16 for
//   substep s (K values 32q + 8s .. +8 of the step); A rows are read from LDS
//   with the same K permutation, so every k meets its own partner. Nothing of
//   B goes through LDS.
// * Dequantization is exact (E2M1 x E4M3 in f16, see common.hpp); the partial
//   sums of the 4 K quarters are added in a fixed order through LDS, then the
//   epilogue applies alpha once (and for L1 the bf16 roundings and SiLU).
//
// For L1, blocks f < 4 are gate columns 16f + c of the slab's 64 and blocks
// f + 4 the matching up columns, so gate and up of one output column sit in
// the same lane and accumulator position.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int NT = 256;
constexpr int SM = 16;            // rows per tile
constexpr int NB = 8;             // MFMA column blocks per lane (weight rows 16f + c)
constexpr int SLAB = 16 * NB;     // weight rows per work-group
constexpr int GB = NB / 2;        // L1: gate blocks (and as many up blocks)
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void skinny_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t K = p.K, N = p.N, Kg = K / 16;
    const int64_t ldq = pitch_q(K), ldsf = pitch_sf(K);
    const int nslab = (MODE == kGemmL1) ? (int)((p.I + 16 * GB - 1) / (16 * GB))
                                        : (int)((N + SLAB - 1) / SLAB);
    const int tile_idx = blockIdx.x / nslab;
    const int slab = blockIdx.x - tile_idx * nslab;
    if (tile_idx >= *p.num_tiles) return;
    const Tile tl = p.tiles[tile_idx];
    const int expert = tl.expert, row_start = tl.row_start, row_count = tl.row_count;

    // ---- stage the tile's A rows (packed, pitch ldq) and scales into LDS ------
    uint8_t* sA = smem;                              // [16][ldq + 16]
    const int a_pitch = (int)ldq + 16;               // 16-byte skew between rows
    uint8_t* sAsf = smem + SM * a_pitch;             // [16][ldsf]
    {
        const int chunks = (int)(ldq / 16);
        for (int i = tid; i < SM * chunks; i += NT) {
            const int r = i / chunks, cch = i - r * chunks;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < row_count) {
                int64_t src = row_start + r;
                if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
                v = *reinterpret_cast<const u32x4*>(p.aq + src * ldq + 16 * cch);
            }
            *reinterpret_cast<u32x4*>(sA + r * a_pitch + 16 * cch) = v;
        }
        for (int i = tid; i < SM * (int)ldsf; i += NT) {
            const int r = i / (int)ldsf, g = i - r * (int)ldsf;
            uint8_t v = 0;
            if (r < row_count && g < Kg) {
                int64_t src = row_start + r;
                if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
                v = p.asf[src * ldsf + g];
            }
            sAsf[r * ldsf + g] = v;
        }
    }
    __syncthreads();

    // ---- this lane's NB weight rows -------------------------------------------
    const int c = lane & 15, q = lane >> 4;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bq + (int64_t)expert * N * ldq, N * ldq);
    const __amdgpu_buffer_rsrc_t rbsf = make_rsrc(p.bsf + (int64_t)expert * N * ldsf, N * ldsf);
    uint32_t boff[NB], sfoff[NB];
    bool ok[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
        int64_t row;
        if (MODE == kGemmL1) {
            const int64_t a = (int64_t)slab * 16 * GB + 16 * (f % GB) + c;
            ok[f] = a < p.I;
            row = ok[f] ? ((f < GB) ? a : p.I + a) : 0;
        } else {
            row = (int64_t)slab * SLAB + 16 * f + c;
            ok[f] = row < N;
            row = ok[f] ? row : 0;
        }
        boff[f] = (uint32_t)(wq_row(row, ldq) + 16 * q);
        sfoff[f] = (uint32_t)(wsf_row(row, ldsf) + 2 * q);
    }

    const int nsteps = (int)(ldq / 64);
    const int per_wave = (nsteps + 3) / 4;
    const int s_begin = wave * per_wave;
    const int s_end = min(nsteps, s_begin + per_wave);

    float4_t acc[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};

    struct Raw {
        u32x4 w[NB];
        uint32_t s[NB];
    };
    auto load = [&](int st, Raw& rw) {
        const uint32_t kd = (uint32_t)st * kWqStep, ksf = (uint32_t)st * kWsfStep;
#pragma unroll
        for (int f = 0; f < NB; ++f) {
            rw.w[f] = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[f], kd, 0);
            rw.s[f] = __builtin_amdgcn_raw_buffer_load_b16(rbsf, sfoff[f], ksf, 0);
        }
    };
    auto compute = [&](int st, const Raw& rw) {
        // A row c, bytes [16q, 16q + 16) of the step; scale groups 2q, 2q + 1
        const u32x4 aw = *reinterpret_cast<const u32x4*>(sA + c * a_pitch + st * 64 + 16 * q);
        uint32_t as = (uint32_t)sAsf[c * ldsf + st * 8 + 2 * q] |
                      ((uint32_t)sAsf[c * ldsf + st * 8 + 2 * q + 1] << 8);
        // groups beyond K (padding of the last step) get scale 0
        const int64_t g0 = (int64_t)st * 8 + 2 * q;
        const uint32_t mask = (g0 < Kg ? 0xFFu : 0u) | (g0 + 1 < Kg ? 0xFF00u : 0u);
        as &= mask;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8_t ha = dequant8(aw[s], scale_pair((as >> (8 * (s >> 1))) & 0xFFu));
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                const uint32_t code = ((rw.s[f] & mask) >> (8 * (s >> 1))) & 0xFFu;
                const half8_t hb = dequant8(rw.w[f][s], scale_pair(code));
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, acc[f], 0, 0, 0);
            }
        }
    };

    // two steps in flight per wave
    Raw r0, r1;
    int st = s_begin;
    if (st < s_end) load(st, r0);
    while (st < s_end) {
        if (st + 1 < s_end) load(st + 1, r1);
        compute(st, r0);
        ++st;
        if (st >= s_end) break;
        if (st + 1 < s_end) load(st + 1, r0);
        compute(st, r1);
        ++st;
    }

    // ---- fixed-order reduction of the 4 K quarters through LDS ----------------
    // acc[f][i] = partial D[row 4q + i][weight row of block f, lane c]
    __syncthreads();                                  // A staging no longer needed
    float* red = reinterpret_cast<float*>(smem);      // [wave][i][lane][f]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4_t* dst = reinterpret_cast<float4_t*>(red + ((wave * 4 + i) * 64 + lane) * NB);
#pragma unroll
        for (int f4 = 0; f4 < NB / 4; ++f4)
            dst[f4] = (float4_t){acc[4 * f4][i], acc[4 * f4 + 1][i], acc[4 * f4 + 2][i], acc[4 * f4 + 3][i]};
    }
    __syncthreads();
    // wave w finishes row 4q + w of every block
    const int i = wave;
    float sum[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) sum[f] = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float4_t* src = reinterpret_cast<const float4_t*>(red + ((w * 4 + i) * 64 + lane) * NB);
#pragma unroll
        for (int f4 = 0; f4 < NB / 4; ++f4) {
            const float4_t v = src[f4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[4 * f4 + e] = sum[4 * f4 + e] + v[e];
        }
    }
    const int local = 4 * q + i;
    const bool row_ok = local < row_count;
    const int64_t prow = row_start + local;
    const float alpha = p.a_gs[0] * p.b_alpha[expert];
    if (MODE == kGemmL1) {
        uint32_t amax_bits = 0;
#pragma unroll
        for (int f = 0; f < GB; ++f) {
            if (!(row_ok && ok[f])) continue;
            const float g = bf16_to_f32(f32_to_bf16_rne(alpha * sum[f]));
            const float u = bf16_to_f32(f32_to_bf16_rne(alpha * sum[f + GB]));
            const uint32_t a = silu_mul_bf16(g, u);
            amax_bits = max(amax_bits, a & 0x7FFFu);
            p.out_bf16[prow * p.I + (int64_t)slab * 16 * GB + 16 * f + c] = (uint16_t)a;
        }
        __shared__ uint32_t wred[NT / 64];
        amax_bits = wave_max_u32(amax_bits);
        if (lane == 0) wred[wave] = amax_bits;
        __syncthreads();
        if (tid == 0) atomicMax(p.amax_slot, max(max(wred[0], wred[1]), max(wred[2], wred[3])) << 16);
    } else {
#pragma unroll
        for (int f = 0; f < NB; ++f) {
            if (!(row_ok && ok[f])) continue;
            p.out_f32[prow * N + (int64_t)slab * SLAB + 16 * f + c] = alpha * sum[f];
        }
    }
}

template <int MODE>
hipError_t launch_skinny_mode(const GemmParams& p, hipStream_t s) {
    const int64_t nslab = (MODE == kGemmL1) ? (p.I + 16 * GB - 1) / (16 * GB) : (p.N + SLAB - 1) / SLAB;
    const int64_t grid = p.max_tiles * nslab;
    if (grid <= 0) return hipSuccess;
    const int64_t ldq = pitch_q(p.K), ldsf = pitch_sf(p.K);
    size_t lds = (size_t)SM * (ldq + 16 + ldsf);
    const size_t red = (size_t)4 * 4 * 64 * NB * sizeof(float);
    if (lds < red) lds = red;
    if (lds > 150 * 1024) return hipErrorInvalidValue;
    static size_t configured = 0;      // largest dynamic LDS size enabled so far
    if (lds > configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = lds;
    }
    skinny_kernel<MODE><<<(unsigned)grid, NT, lds, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const GemmParams& p, hipStream_t s) {
    if (p.N * pitch_q(p.K) >= 0x7FFFFFFF) return hipErrorInvalidValue;
    switch (p.mode) {
        case kGemmL1: return launch_skinny_mode<kGemmL1>(p, s);
        case kGemmL2: return launch_skinny_mode<kGemmL2>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
