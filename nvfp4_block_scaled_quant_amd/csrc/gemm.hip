// Block-scaled NVFP4 GEMMs on gfx950 matrix cores: the dense GEMM and the two
// grouped GEMMs of the expert layer (DEBUG_LOG, "NVFP4 MoE Pipeline": L1 with
// alpha = igs * l1_global_sf, SiLU(gate) * up, L2 with alpha = l1_igs *
// l2_global_sf; Hypothesis 3: alphas stay out of the E4M3 scales).
//
// Arithmetic. Every dequantized element e2m1 * e4m3 is exact in f16 (at most 6
// significant bits, range [2^-10, 2688]), so an f16 MFMA with float32
// accumulation sums exact products; the global scales are applied once, as
// float32 alpha, in the epilogue. gfx950's FP4 MFMAs take power-of-two (E8M0)
// scales per 32 elements and cannot carry an E4M3 scale per 16 elements
// exactly, so the operands are dequantized in registers and fed to
// v_mfma_f32_32x32x16_f16.
//
// Tiling. A work-group of 4 waves computes a 256 x 256 tile; each wave owns a
// 128 x 128 quadrant (4 x 4 tiles of v_mfma_f32_32x32x16_f16). The K loop steps 128
// elements (64 packed bytes) at a time through double-buffered LDS holding the
// tiles still packed (4 bits per element), so LDS traffic and capacity are a
// quarter of a bf16 design. Both operands sit in LDS K-contiguous: A rows are
// K-packed already; B arrives (K/2, N) N-contiguous from HBM and is transposed
// 4x4 bytes at a time in registers (v_perm) on its way into LDS.
//
// K permutation. Inside one 128-element K step, lane half h = lane / 32 reads
// the 32 bytes (64 elements) [64h, 64h + 64) of its row or column with two
// 128-bit LDS reads, and MFMA number s (0..7) of the step consumes elements
// [64h + 8s, 64h + 8s + 8) from both halves. A and B use the same
// permutation, and each 8-element run lies inside one 16-element scale group,
// so every k is multiplied with its own partner exactly once. The dequant of
// substep s + 1 is issued before the MFMAs of substep s so that the VALU work
// overlaps the matrix cores.
//
// Grouped scheduling. Tiles come from a device-built list (expert, first
// sorted row, row count); the grid is sized for the worst case and idle
// work-groups leave at once, so the host never waits for routing counts.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int KB = 64;                 // packed bytes of K per step (128 elements)
constexpr int LDT = 80;                // LDS row pitch in bytes (64 data + 16 pad)
constexpr int NT = 256;                // threads per work-group

struct Smem {
    uint8_t a[2][BM * LDT];
    uint8_t b[2][BN * LDT];
    uint8_t asf[2][BM * 8];
    uint8_t bsf[2][8 * BN];
};

struct Stage {
    u32x4 a[4];
    u32x2 asf;
    uint32_t b[16];
    u32x2 bsf;
};

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    const int tid = threadIdx.x;
    const int64_t K = p.K, N = p.N;
    const int64_t Kh = K / 2, Kg = K / 16;
    const int ntn = (MODE == kGemmL1) ? (int)((p.I + 127) / 128) : (int)((N + BN - 1) / BN);
    const int tile_idx = blockIdx.x / ntn;
    const int nt = blockIdx.x - tile_idx * ntn;

    int expert, row_start, row_count;
    if (MODE == kGemmDense) {
        expert = 0;
        row_start = tile_idx * BM;
        row_count = (int)min((int64_t)BM, p.M - row_start);
        if (row_count <= 0) return;
    } else {
        if (tile_idx >= *p.num_tiles) return;
        const Tile t = p.tiles[tile_idx];
        expert = t.expert;
        row_start = t.row_start;
        row_count = t.row_count;
    }

    // ---- per-thread load descriptors -------------------------------------
    // A data: 4 lanes per row, 16 bytes each; rows ar, ar+64, ar+128, ar+192
    const int ar = tid >> 2, ac = tid & 3;
    const uint8_t* a_row[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int local = ar + 64 * i;
        a_ok[i] = local < row_count;
        int64_t src = row_start + (a_ok[i] ? local : 0);
        if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
        a_row[i] = p.aq + src * Kh + 16 * ac;
    }
    // A scales: one row per thread
    const bool asf_ok = tid < row_count;
    int64_t asf_src = row_start + (asf_ok ? tid : 0);
    if (MODE == kGemmL1) asf_src = p.a_gather[asf_src] / p.topk;
    const uint8_t* asf_row = p.asf + asf_src * Kg;

    // B column mapping: virtual column vc of the tile -> weight column
    auto map_col = [&](int vc, bool& ok) -> int64_t {
        if (MODE == kGemmL1) {
            const int w = vc >> 7, r = vc & 127;
            const int64_t base = (int64_t)nt * 128 + 64 * w + (r & 63);
            ok = base < p.I;
            return (r < 64) ? base : p.I + base;
        } else {
            const int64_t c = (int64_t)nt * BN + vc;
            ok = c < N;
            return c;
        }
    };
    const int cq = tid & 63, kb = tid >> 6;
    bool b_ok;
    const int64_t b_col = map_col(4 * cq, b_ok);
    const uint8_t* b_base = p.bq + (int64_t)expert * Kh * N + (int64_t)(16 * kb) * N + (b_ok ? b_col : 0);
    const int g_row = tid >> 5, vc8 = 8 * (tid & 31);
    bool bsf_ok;
    const int64_t bsf_col = map_col(vc8, bsf_ok);
    const uint8_t* bsf_base = p.bsf + (int64_t)expert * Kg * N + (int64_t)g_row * N + (bsf_ok ? bsf_col : 0);

    const bool a_vec16 = (Kh % 16) == 0;
    const bool asf_vec8 = (Kg % 8) == 0;
    const int nk = (int)((K + 127) / 128);

    auto load_stage = [&](int ks, Stage& st) {
        const int64_t kb0 = (int64_t)ks * KB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v = {0u, 0u, 0u, 0u};
            const int64_t off = kb0 + 16 * ac;
            if (a_ok[i] && off < Kh) {
                if (a_vec16) {
                    v = *reinterpret_cast<const u32x4*>(a_row[i] + kb0);
                } else {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(a_row[i] + kb0);
                    v[0] = lo[0];
                    v[1] = lo[1];
                    if (off + 8 < Kh) {
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(a_row[i] + kb0 + 8);
                        v[2] = hi[0];
                        v[3] = hi[1];
                    }
                }
            }
            st.a[i] = v;
        }
        {
            u32x2 v = {0u, 0u};
            const int64_t g0 = (int64_t)ks * 8;
            if (asf_ok) {
                if (asf_vec8 && g0 + 8 <= Kg) {
                    v = *reinterpret_cast<const u32x2*>(asf_row + g0);
                } else {
                    for (int g = 0; g < 8; ++g)
                        if (g0 + g < Kg) v[g >> 2] |= (uint32_t)asf_row[g0 + g] << (8 * (g & 3));
                }
            }
            st.asf = v;
        }
        const uint8_t* bp = b_base + kb0 * N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t kh = kb0 + 16 * kb + r;
            st.b[r] = (b_ok && kh < Kh) ? *reinterpret_cast<const uint32_t*>(bp + (int64_t)r * N) : 0u;
        }
        {
            u32x2 v = {0u, 0u};
            if (bsf_ok && (int64_t)ks * 8 + g_row < Kg)
                v = *reinterpret_cast<const u32x2*>(bsf_base + (int64_t)ks * 8 * N);
            st.bsf = v;
        }
    };

    auto store_stage = [&](int buf, const Stage& st) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(&sm.a[buf][(ar + 64 * i) * LDT + 16 * ac]) = st.a[i];
        *reinterpret_cast<u32x2*>(&sm.asf[buf][tid * 8]) = st.asf;
        uint32_t col[4][4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const uint32_t r4[4] = {st.b[4 * jb], st.b[4 * jb + 1], st.b[4 * jb + 2], st.b[4 * jb + 3]};
            uint32_t c4[4];
            transpose4x4(r4, c4);
#pragma unroll
            for (int c = 0; c < 4; ++c) col[c][jb] = c4[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            u32x4 v = {col[c][0], col[c][1], col[c][2], col[c][3]};
            *reinterpret_cast<u32x4*>(&sm.b[buf][(4 * cq + c) * LDT + 16 * kb]) = v;
        }
        *reinterpret_cast<u32x2*>(&sm.bsf[buf][g_row * BN + vc8]) = st.bsf;
    };

    // ---- main loop ---------------------------------------------------------
    // Wave (wm, wn) owns rows [128 wm, +128) and virtual columns [128 wn, +128)
    // of the tile as 4 x 4 blocks of the 32 x 32 x 16 MFMA. Lane l serves row /
    // column (l & 31) of a block and K half h = l >> 5: inside a 128-element K
    // step it holds elements [64h, 64h + 64) (32 bytes, two 128-bit LDS reads),
    // and substep s (0..7) feeds the MFMA elements [64h + 8s, 64h + 8s + 8),
    // which lie in scale group 4h + s/2.
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Stage st;
    load_stage(0, st);
    store_stage(0, st);
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        const bool more = ks + 1 < nk;
        if (more) load_stage(ks + 1, st);

        u32x4 fa[4][2], fb[4][2];
        uint32_t sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 128 + 32 * i + l32;
            const uint8_t* pa = &sm.a[buf][row * LDT + 32 * h];
            fa[i][0] = *reinterpret_cast<const u32x4*>(pa);
            fa[i][1] = *reinterpret_cast<const u32x4*>(pa + 16);
            sa[i] = *reinterpret_cast<const uint32_t*>(&sm.asf[buf][row * 8 + 4 * h]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int vc = wn * 128 + 32 * j + l32;
            const uint8_t* pb = &sm.b[buf][vc * LDT + 32 * h];
            fb[j][0] = *reinterpret_cast<const u32x4*>(pb);
            fb[j][1] = *reinterpret_cast<const u32x4*>(pb + 16);
            const uint8_t* ps = &sm.bsf[buf][(4 * h) * BN + vc];
            sb[j] = (uint32_t)ps[0] | ((uint32_t)ps[BN] << 8) | ((uint32_t)ps[2 * BN] << 16) |
                    ((uint32_t)ps[3 * BN] << 24);
        }

        half8_t ha[2][4], hb[2][4];
        auto deq = [&](int s, half8_t (&xa)[4], half8_t (&xb)[4]) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xa[i] = dequant8(fa[i][s >> 2][s & 3], scale_pair((sa[i] >> (8 * (s >> 1))) & 0xFFu));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xb[j] = dequant8(fb[j][s >> 2][s & 3], scale_pair((sb[j] >> (8 * (s >> 1))) & 0xFFu));
        };
        deq(0, ha[0], hb[0]);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (s < 7) deq(s + 1, ha[(s + 1) & 1], hb[(s + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[s & 1][i], hb[s & 1][j],
                                                                        acc[i][j], 0, 0, 0);
        }

        if (more) store_stage(buf ^ 1, st);
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
    // acc[i][j][r] = D[row 32i + 8(r/4) + 4h + (r%4)][col 32j + l32] of the quadrant
    const float alpha = p.a_gs[0] * p.b_alpha[expert];
    if (MODE == kGemmL1) {
        // gate = virtual columns [0, 64) of the quadrant (blocks 0, 1), up = [64, 128).
        // The rounded (gate, up) pairs of one half of the tile (128 rows x 128
        // act columns) go through the now idle LDS; then all threads apply
        // SiLU and store act row by row (coalesced), in two halves.
        uint32_t* gu = reinterpret_cast<uint32_t*>(smem_raw);     // [128][128] g | u << 16
        uint32_t amax_bits = 0;
        for (int half = 0; half < 2; ++half) {
            if (wm == half) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                            const int col = wn * 64 + 32 * j + l32;
                            const uint32_t g = f32_to_bf16_rne(alpha * acc[i][j][r]);
                            const uint32_t u = f32_to_bf16_rne(alpha * acc[i][j + 2][r]);
                            gu[row * 128 + col] = g | (u << 16);
                        }
            }
            __syncthreads();
            for (int e = tid; e < 128 * 128; e += NT) {
                const int local = half * 128 + (e >> 7);
                const int64_t col = (int64_t)nt * 128 + (e & 127);
                if (local < row_count && col < p.I) {
                    const uint32_t w = gu[e];
                    const uint32_t a = silu_mul_bf16(bf16_to_f32(w & 0xFFFFu), bf16_to_f32(w >> 16));
                    p.out_bf16[(int64_t)(row_start + local) * p.I + col] = (uint16_t)a;
                    amax_bits = max(amax_bits, a & 0x7FFFu);
                }
            }
            __syncthreads();
        }
        __shared__ uint32_t red[NT / 64];
        amax_bits = wave_max_u32(amax_bits);
        if (lane == 0) red[wave] = amax_bits;
        __syncthreads();
        if (tid == 0) {
            uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
            atomicMax(p.amax_slot, m << 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int local = wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (local >= row_count) continue;
                const int64_t prow = row_start + local;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = (int64_t)nt * BN + wn * 128 + 32 * j + l32;
                    if (col >= N) continue;
                    const float v = alpha * acc[i][j][r];
                    if (MODE == kGemmL2) p.out_f32[prow * N + col] = v;
                    else p.out_bf16[prow * N + col] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
        }
    }
}

template <int MODE>
hipError_t launch_mode(const GemmParams& p, hipStream_t s) {
    const int64_t ntn = (MODE == kGemmL1) ? (p.I + 127) / 128 : (p.N + BN - 1) / BN;
    const int64_t mt = (MODE == kGemmDense) ? (p.M + BM - 1) / BM : p.max_tiles;
    const int64_t grid = mt * ntn;
    if (grid <= 0) return hipSuccess;
    const size_t lds = sizeof(Smem);
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
    }
    gemm_kernel<MODE><<<(unsigned)grid, NT, lds, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
    switch (p.mode) {
        case kGemmDense: return launch_mode<kGemmDense>(p, s);
        case kGemmL1: return launch_mode<kGemmL1>(p, s);
        case kGemmL2: return launch_mode<kGemmL2>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
