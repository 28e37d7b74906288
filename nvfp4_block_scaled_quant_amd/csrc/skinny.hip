// Weight-streaming grouped GEMMs for small batches (decode): the same two
// expert GEMMs as gemm.hip (DEBUG_LOG, "NVFP4 MoE Pipeline", L1 with fused
// SiLU(gate) * up and L2), for tiles of at most 16 rows.
//
// With a handful of rows per expert the layer is bound by reading the expert
// weights from HBM once, so the kernel is built around the weight stream:
//
// * A work-group owns one 16-row tile and one slab of 256 weight columns (for
//   L1: 128 gate columns and the 128 matching up columns). Its 16 A rows are
//   staged once in LDS, still packed.
// * Each of the 4 waves streams a quarter of K. Per 32-element K chunk, lane
//   (c, q) = (lane % 16, lane / 16) loads 16 weight bytes from each of 4 K-packed
//   rows 4q..4q+3 (16 columns, 256 contiguous bytes per row across the lanes);
//   a 4x4 byte transpose in registers turns them into 8 consecutive K values
//   for each of its 16 columns, which is exactly the B operand of
//   v_mfma_f32_16x16x32_f16 for 16 column blocks (block f holds columns
//   16c + f of the slab). Nothing of B goes through LDS.
// * Dequantization is exact (E2M1 x E4M3 in f16, see common.hpp); partial sums
//   of the 4 K quarters are added in a fixed order through LDS, then the
//   epilogue applies alpha once (and for L1 the bf16 roundings and SiLU).
//
// For L1 the slab's 16 columns of lane c are 8 gate columns n0 + 8c .. +8 (f < 8)
// and the matching 8 up columns (f >= 8), so gate and up of one output column
// sit in the same lane and accumulator position.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int NT = 256;
constexpr int SM = 16;            // rows per tile

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void skinny_kernel(GemmParams p, int a_pitch, int sf_pitch) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t K = p.K, N = p.N, Kh = K / 2, Kg = K / 16;
    const int nslab = (MODE == kGemmL1) ? (int)((p.I + 127) / 128) : (int)((N + 255) / 256);
    const int tile_idx = blockIdx.x / nslab;
    const int slab = blockIdx.x - tile_idx * nslab;
    if (tile_idx >= *p.num_tiles) return;
    const Tile tl = p.tiles[tile_idx];
    const int expert = tl.expert, row_start = tl.row_start, row_count = tl.row_count;

    // ---- stage the tile's A rows (packed) and their scales into LDS ----------
    uint8_t* sA = smem;                              // [16][a_pitch]
    uint8_t* sAsf = smem + SM * a_pitch;             // [16][sf_pitch]
    {
        const int words = a_pitch / 4;
        for (int i = tid; i < SM * words; i += NT) {
            const int r = i / words, w = i - r * words;
            uint32_t v = 0;
            if (r < row_count && 4 * (int64_t)w < Kh) {
                int64_t src = row_start + r;
                if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
                v = *reinterpret_cast<const uint32_t*>(p.aq + src * Kh + 4 * w);
            }
            *reinterpret_cast<uint32_t*>(sA + r * a_pitch + 4 * w) = v;
        }
        for (int i = tid; i < SM * sf_pitch; i += NT) {
            const int r = i / sf_pitch, g = i - r * sf_pitch;
            uint8_t v = 0;
            if (r < row_count && g < Kg) {
                int64_t src = row_start + r;
                if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
                v = p.asf[src * Kg + g];
            }
            sAsf[r * sf_pitch + g] = v;
        }
    }
    __syncthreads();

    // ---- per-lane weight columns ----------------------------------------------
    const int c = lane & 15, q = lane >> 4;
    const uint8_t* bq_e = p.bq + (int64_t)expert * Kh * N;
    const uint8_t* bsf_e = p.bsf + (int64_t)expert * Kg * N;
    int64_t col0, col1;     // L1: gate and up column bases (8 each); L2: one base of 16
    bool ok;
    if (MODE == kGemmL1) {
        const int64_t a0 = (int64_t)slab * 128 + 8 * c;
        ok = a0 < p.I;
        col0 = ok ? a0 : 0;
        col1 = ok ? p.I + a0 : 0;
    } else {
        const int64_t a0 = (int64_t)slab * 256 + 16 * c;
        ok = a0 < N;
        col0 = ok ? a0 : 0;
        col1 = col0 + 8;
    }

    const int nchunks = (int)((K + 31) / 32);
    const int per_wave = (nchunks + 3) / 4;
    const int c_begin = wave * per_wave;
    const int c_end = min(nchunks, c_begin + per_wave);

    float4_t acc[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};

    struct Raw {
        uint32_t w[4][4];   // [row r][column group]
        uint32_t s[4];      // 16 scale bytes
    };
    auto load = [&](int ch, Raw& rw) {
        const int64_t kh0 = (int64_t)ch * 16 + 4 * q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t kh = kh0 + r;
            const bool v = ok && kh < Kh;
            const uint8_t* row = bq_e + (v ? kh : 0) * N;
            const u32x2 lo = v ? *reinterpret_cast<const u32x2*>(row + col0) : (u32x2){0u, 0u};
            const u32x2 hi = v ? *reinterpret_cast<const u32x2*>(row + col1) : (u32x2){0u, 0u};
            rw.w[r][0] = lo[0];
            rw.w[r][1] = lo[1];
            rw.w[r][2] = hi[0];
            rw.w[r][3] = hi[1];
        }
        const int64_t g = (int64_t)ch * 2 + (q >> 1);
        const bool v = ok && g < Kg;
        const uint8_t* srow = bsf_e + (v ? g : 0) * N;
        const u32x2 lo = v ? *reinterpret_cast<const u32x2*>(srow + col0) : (u32x2){0u, 0u};
        const u32x2 hi = v ? *reinterpret_cast<const u32x2*>(srow + col1) : (u32x2){0u, 0u};
        rw.s[0] = lo[0];
        rw.s[1] = lo[1];
        rw.s[2] = hi[0];
        rw.s[3] = hi[1];
    };
    auto compute = [&](int ch, const Raw& rw) {
        // A fragment: row c, K values [32 ch + 8q, +8)
        const uint32_t aw = *reinterpret_cast<const uint32_t*>(sA + c * a_pitch + ch * 16 + 4 * q);
        const uint32_t as = sAsf[c * sf_pitch + 2 * ch + (q >> 1)];
        const half8_t ha = dequant8(aw, scale_pair(as));
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
            const uint32_t r4[4] = {rw.w[0][cg], rw.w[1][cg], rw.w[2][cg], rw.w[3][cg]};
            uint32_t c4[4];
            transpose4x4(r4, c4);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int f = 4 * cg + cc;
                const uint32_t code = (rw.s[f >> 2] >> (8 * (f & 3))) & 0xFFu;
                const half8_t hb = dequant8(c4[cc], scale_pair(code));
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, acc[f], 0, 0, 0);
            }
        }
    };

    // two chunks in flight per wave
    Raw r0, r1;
    int ch = c_begin;
    if (ch < c_end) load(ch, r0);
    while (ch < c_end) {
        if (ch + 1 < c_end) load(ch + 1, r1);
        compute(ch, r0);
        ++ch;
        if (ch >= c_end) break;
        if (ch + 1 < c_end) load(ch + 1, r0);
        compute(ch, r1);
        ++ch;
    }

    // ---- fixed-order reduction of the 4 K quarters through LDS ----------------
    // acc[f][i] = partial D[row 4q + i][column of block f of lane c]
    __syncthreads();                                  // A staging no longer needed
    float* red = reinterpret_cast<float*>(smem);      // [wave][i][lane][f]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4_t* dst = reinterpret_cast<float4_t*>(red + ((wave * 4 + i) * 64 + lane) * 16);
#pragma unroll
        for (int f4 = 0; f4 < 4; ++f4)
            dst[f4] = (float4_t){acc[4 * f4][i], acc[4 * f4 + 1][i], acc[4 * f4 + 2][i], acc[4 * f4 + 3][i]};
    }
    __syncthreads();
    // wave w finishes row 4q + w of every block
    const int i = wave;
    float sum[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) sum[f] = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float4_t* src = reinterpret_cast<const float4_t*>(red + ((w * 4 + i) * 64 + lane) * 16);
#pragma unroll
        for (int f4 = 0; f4 < 4; ++f4) {
            const float4_t v = src[f4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[4 * f4 + e] = sum[4 * f4 + e] + v[e];
        }
    }
    const int local = 4 * q + i;
    const bool row_ok = local < row_count && ok;
    const int64_t prow = row_start + local;
    const float alpha = p.a_gs[0] * p.b_alpha[expert];
    if (MODE == kGemmL1) {
        uint32_t amax_bits = 0;
        uint32_t packed[4];
#pragma unroll
        for (int f = 0; f < 8; f += 2) {
            uint32_t two = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float g = bf16_to_f32(f32_to_bf16_rne(alpha * sum[f + e]));
                const float u = bf16_to_f32(f32_to_bf16_rne(alpha * sum[f + e + 8]));
                const uint32_t a = silu_mul_bf16(g, u);
                amax_bits = row_ok ? max(amax_bits, a & 0x7FFFu) : amax_bits;
                two |= a << (16 * e);
            }
            packed[f >> 1] = two;
        }
        if (row_ok) {
            u32x4 v = {packed[0], packed[1], packed[2], packed[3]};
            *reinterpret_cast<u32x4*>(p.out_bf16 + prow * p.I + col0) = v;
        }
        __shared__ uint32_t wred[NT / 64];
        amax_bits = wave_max_u32(amax_bits);
        if (lane == 0) wred[wave] = amax_bits;
        __syncthreads();
        if (tid == 0) atomicMax(p.amax_slot, max(max(wred[0], wred[1]), max(wred[2], wred[3])) << 16);
    } else {
        if (row_ok) {
            float4_t* dst = reinterpret_cast<float4_t*>(p.out_f32 + prow * N + col0);
#pragma unroll
            for (int f4 = 0; f4 < 4; ++f4)
                dst[f4] = (float4_t){alpha * sum[4 * f4], alpha * sum[4 * f4 + 1],
                                     alpha * sum[4 * f4 + 2], alpha * sum[4 * f4 + 3]};
        }
    }
}

template <int MODE>
hipError_t launch_skinny_mode(const GemmParams& p, hipStream_t s) {
    const int64_t nslab = (MODE == kGemmL1) ? (p.I + 127) / 128 : (p.N + 255) / 256;
    const int64_t grid = p.max_tiles * nslab;
    if (grid <= 0) return hipSuccess;
    const int64_t Kh = p.K / 2, Kg = p.K / 16;
    // row pitches: whole 32-element chunks plus 4 bytes so rows fall in different banks
    const int a_pitch = (int)(((Kh + 15) / 16) * 16 + 4);
    const int sf_pitch = (int)(((Kg + 1) / 2) * 2 + 4);
    size_t lds = (size_t)SM * (a_pitch + sf_pitch);
    const size_t red = (size_t)4 * 4 * 64 * 16 * sizeof(float);
    if (lds < red) lds = red;
    if (lds > 150 * 1024) return hipErrorInvalidValue;
    static size_t configured = 0;      // largest dynamic LDS size enabled so far
    if (lds > configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = lds;
    }
    skinny_kernel<MODE><<<(unsigned)grid, NT, lds, s>>>(p, a_pitch, sf_pitch);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const GemmParams& p, hipStream_t s) {
    switch (p.mode) {
        case kGemmL1: return launch_skinny_mode<kGemmL1>(p, s);
        case kGemmL2: return launch_skinny_mode<kGemmL2>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
