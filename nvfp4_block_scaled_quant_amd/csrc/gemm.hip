// Block-scaled NVFP4 GEMMs on gfx950 matrix cores: the dense GEMM and the two
// grouped GEMMs of the expert layer (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline": L1 with
// alpha = igs * l1_global_sf, SiLU(gate) * up, L2 with alpha = l1_igs *
// l2_global_sf; Hypothesis 3: alphas stay out of the E4M3 scales).
//
// Arithmetic. Every dequantized element e2m1 * e4m3 is exact in f16 (at most 6
// significant bits, range [2^-10, 2688]), so an f16 MFMA with float32
// accumulation sums exact products; the global scales are applied once, as
// float32 alpha, in the epilogue. gfx950's FP4 MFMAs take power-of-two (E8M0)
// scales per 32 elements and cannot carry an E4M3 scale per 16 elements
// exactly, so the operands are fed to v_mfma_f32_32x32x16_f16 as f16.
//
// Operands. A is the quantized activation in its exact f16 form (written by
// the quantizer next to the packed bytes: e2m1 * e4m3 per element, the
// global scale left out), rows of pitch_h(K) bytes; every N-tile reads those
// values as they are, with no conversion. B rows (one per weight column: the
// weights in the byte-transposed layout, as the pages' GEMM consumed B
// column-major) are K-packed FP4 with their E4M3 scales, in 16-row blocks
// whose 64-element half steps are contiguous (512 bytes); they are converted
// to f16 in registers (one scaled FP4 -> f16 conversion and one f16 multiply
// per two elements). Tiles move from HBM to LDS by buffer loads that write
// LDS directly (no staging registers; out-of-range offsets read zeros),
// three stages of 64 K elements (42 KB each).
//
// LDS layout of a stage. A: 256 rows of 128 bytes (8 chunks of 16 bytes;
// chunk c of row r stored at chunk c ^ ((r >> 1) & 7), so the 16 rows read by
// a 16-lane group of fragment loads cover all banks). B: 256 rows of 32 bytes
// (2 chunks, chunk c of row r at c ^ ((r >> 3) & 1)). B scales: per row two
// dwords, one per pair of scale groups (the packed weights store a pair of
// groups of four consecutive K steps together, so a half step's pairs are
// 2-byte pieces; each is brought in by a 2-byte load that fills a whole LDS
// dword, zero-extended).
//
// Tiling. A work-group of 8 waves (two per SIMD) computes a 256 x 256 tile;
// wave w owns rows 128 (w / 4) .. +128 and columns 64 (w % 4) .. +64 (4 x 2
// tiles of 32 x 32 x 16, 128 accumulator registers; 32 MI rows per wave row
// in the variants below). With two waves on a SIMD,
// one wave's FP4 conversions, fragment reads and refill loads issue while the
// other's MFMAs run (one wave per SIMD with 128 x 128 each left the matrix
// core idle about a fifth of the loop). Lane l serves row / column
// l % 32 and K half h = l / 32: of a 64-element step it covers elements
// [32h, 32h + 32), and substep s (0..3) feeds the MFMA elements [32h + 8s, +8),
// inside scale group 2h + s / 2; A and B use the same K permutation, so every
// k meets its own partner. A tile whose expert has fewer rows left runs a
// variant with MI (1..3) instead of 4 row blocks of 32 per wave and loads only
// its 64 * MI A rows.
//
// Scheduling. Work-group b runs on XCD b % 8 (the dispatcher deals work-groups
// round-robin over the eight XCDs, each with its own L2), so b = 8 s + x
// takes tile 8 (s / ntn) + x, N-tile s % ntn: all N-tiles of one tile run on
// one XCD, at about the same time, and read its A rows through one L2. Tiles
// come from a device-built list (expert, first sorted row, row count), each
// expert's full tiles followed by its partial one (partial tiles of at most
// half the rows at the end of the list); the grid is sized for the worst
// case and idle work-groups leave at once, so the host never waits for
// routing counts. The dense GEMM has no tile list and few tiles (a 256-row
// M is 24 tiles at N = 6144): its work-groups go in plain order, and when
// 256-row tiles would fill less than half the GPU it takes 128-row tiles
// (twice the tiles) and cuts the K steps into chunks, one work-group per
// (tile, chunk) with at most one work-group per CU, each writing float32
// partial sums that a second kernel adds in chunk order before the one bf16
// rounding (the half-height tiles halve the chunks, and so the partial sums
// written and read back). Invalid rows and columns of a tile read a valid row instead
// (their results are never stored). Rows are read in whole steps: the padding
// of a partial last step is zero in both operands (the quantizers and the
// weight prepack write it as zeros), so it adds nothing.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int NT = 512;                 // threads per work-group: 8 waves, two per SIMD
constexpr int KS = 64;                  // K elements per step
constexpr int NSTAGE = 3;
constexpr int A_ROW = 2 * KS;           // bytes of one f16 A row per step
constexpr int A_BYTES = BM * A_ROW;     // 32 KB
constexpr int B_ROW = KS / 2;           // bytes of one packed B row per step
constexpr int B_BYTES = BN * B_ROW;     // 8 KB
constexpr int BSF_BYTES = BN * 8;       // 2 KB: two dwords per row
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + BSF_BYTES;
constexpr int kGuLd = 130;              // L1 epilogue: words per staged gate/up row
constexpr int EPI_BYTES = BM * kGuLd * 4;
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES > EPI_BYTES ? NSTAGE * STAGE_BYTES : EPI_BYTES;
constexpr uint32_t kRsrcWord3 = 0x00020000u;        // raw buffer, 32-bit data format

// s_waitcnt immediate: vmcnt (6 bits, split 4 + 2), expcnt left at 7, lgkmcnt
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Work-group barrier for the main loop. __syncthreads() (and any workgroup
// fence, since the buffer-to-LDS loads count as LDS writes) first drains every
// outstanding global load, i.e. waits for the stages still in flight. Here the
// DMA of the stage about to be read is waited for explicitly (vmcnt) before
// the barrier, and the empty asm statements keep the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int64_t K = p.K, N = p.N;
    const int64_t ldq = pitch_q(K), lda = pitch_h(K);           // packed B row, f16 A row
    const int64_t ldwsf = pitch_wsf(K);                         // packed weight scales
    const int ntn = (MODE == kGemmL1) ? (int)((p.I + 127) / 128) : (int)((N + BN - 1) / BN);
    // Grouped GEMMs: XCD order (above). Dense: plain order, tile fastest, then
    // N-tile, then K chunk (with ksplit > 1, chunk c sums the c-th range of K
    // steps into its own partial sums): the dense shapes have few tiles, which
    // the XCD order would put on one XCD.
    int tile_idx, nt, chunk = 0;
    if (MODE == kGemmDense) {
        const int mt = (int)((p.M + dense_tile_rows(p.M, N) - 1) / dense_tile_rows(p.M, N));
        tile_idx = blockIdx.x % mt;
        const int rest = blockIdx.x / mt;
        nt = rest % ntn;
        chunk = rest / ntn;
    } else {
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        tile_idx = 8 * (slot / ntn) + xcd;
        nt = slot % ntn;
    }

    int expert, row_start, row_count;
    if (MODE == kGemmDense) {
        expert = 0;
        const int dbm = (int)dense_tile_rows(p.M, N);
        row_start = tile_idx * dbm;
        row_count = (int)min((int64_t)dbm, p.M - row_start);
        if (row_count <= 0) return;
    } else {
        if (tile_idx >= p.max_tiles) return;      // the grid covers whole groups of 8 tiles
        // both loads at once (the entry exists, and is used only when it is
        // one of the num_tiles valid ones)
        const Tile t = p.tiles[tile_idx];
        const int ntiles = *p.num_tiles;
        // keeps the tile load above the branch (the compiler would sink it)
        asm volatile("" ::"s"(t.expert), "s"(t.row_start), "s"(t.row_count));
        if (tile_idx >= ntiles) return;
        expert = t.expert;
        row_start = t.row_start;
        row_count = t.row_count;
    }
    // Each wave covers MI blocks of 32 rows, so a tile computes and loads 64 *
    // MI rows: the last tile of an expert usually holds fewer than 256 (at the
    // prefill shape about 171 of 256 on average).
    const int mi_tile = __builtin_amdgcn_readfirstlane((row_count + 63) / 64);
    __shared__ uint32_t red[NT / 64];
    auto tile = [&](auto mi_c) {
        constexpr int MI = decltype(mi_c)::value;
        constexpr int NA = MI;                  // A loads per wave and stage (8 rows each)
        constexpr int NL = NA + 2;              // all loads per wave and stage (+ B data, B scales)
        constexpr int kWaitStage = waitcnt_imm(NL, 0);   // all but one stage's loads done
        constexpr int kWaitAll = waitcnt_imm(0, 0);
        // VALU per MFMA in the substeps' schedules: the B conversion of one
        // substep is 16 VALU plus the scale pairs, over its 2 * MI MFMAs; the
        // last substep's first kFirst MFMAs cover the fragment reads
        constexpr int kValu = MI == 4 ? 2 : MI == 3 ? 3 : MI == 2 ? 4 : 8;
        constexpr int kFirst = MI == 4 ? 3 : MI == 3 ? 2 : 1;
        constexpr int kValuLast = MI == 4 ? 4 : MI == 3 ? 5 : MI == 2 ? 7 : 20;

        // ---- buffer resources and per-lane DMA offsets ---------------------------
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.ah, p.a_rows * lda);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bq + (int64_t)expert * N * ldq, N * ldq);
        const __amdgpu_buffer_rsrc_t rbsf = make_rsrc(p.bsf + (int64_t)expert * N * ldwsf, N * ldwsf);

        auto a_src = [&](int r) -> int64_t {        // A tensor row of tile row r
            int64_t src = row_start + (r < row_count ? r : 0);
            if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
            return src;
        };
        auto b_src = [&](int vc) -> int64_t {       // weight row (output column) of virtual column vc
            if (MODE == kGemmL1) {
                const int w = vc >> 6, r = vc & 63;
                const int64_t base = (int64_t)nt * 128 + 32 * w + (r & 31);
                if (base >= p.I) return 0;
                return (r < 32) ? base : p.I + base;
            }
            const int64_t c = (int64_t)nt * BN + vc;
            return c < N ? c : 0;
        };
        // A: load u (0 .. 8 MI - 1) fills LDS bytes [1024 u, +1024) of the A
        // region: rows 8u + lane / 8, physical chunk lane % 8. Wave w issues
        // u = NA w + t (NA = MI: the 8 waves cover the 64 MI rows).
        // (fixed size: the host pass of the compiler drops the kernel when a
        // nested lambda captures an array whose size depends on MI)
        uint32_t a_off[8];
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            const int row = 8 * (NA * wave + t) + (lane >> 3);
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            a_off[t] = (uint32_t)(a_src(row) * lda + 16 * chunk);
        }
        // B: wave w's load fills rows 32w + lane / 2, physical chunk lane % 2.
        // B scales: wave w's load fills dword 64w + lane = row (64w + lane) / 2,
        // pair lane % 2 of the half step's two.
        uint32_t b_off, bsf_off;
        {
            const int row = 32 * wave + (lane >> 1);
            const int chunk = (lane & 1) ^ ((row >> 3) & 1);
            b_off = (uint32_t)wq_off(b_src(row), ldq, 16 * chunk);
            const int64_t n = b_src(row);
            bsf_off = (uint32_t)((n >> 4) * 16 * ldwsf + (n & 15) * 32 + (lane & 1) * 8);
        }

        // 64-element steps: all of K, or this work-group's chunk [kb, kb + nk)
        // (dense_ksplit makes every chunk non-empty)
        const int nk_all = (int)(ldq / 32);
        const bool split = MODE == kGemmDense && p.ksplit > 1;
        const int kper = split ? (nk_all + p.ksplit - 1) / p.ksplit : nk_all;
        const int kb = split ? chunk * kper : 0;
        const int nk = split ? min(nk_all, kb + kper) - kb : nk_all;
        // ---- main loop ---------------------------------------------------------
        const int wm = wave >> 2, wn = wave & 3;
        const int l32 = lane & 31, h = lane >> 5;

        float16_t acc[MI][2];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // Fragment rows are wm * 32 MI + 32 i + l32 (A) and wn * 64 + 32 j + l32
        // (B): the 32 i / 32 j parts do not change the swizzles, which then
        // depend on the lane alone. The per-lane offsets within a stage are
        // formed once; the fragments' row offsets are the reads' immediates.
        const uint32_t a_row = (uint32_t)(wm * (32 * MI) + l32), b_row = (uint32_t)(wn * 64 + l32);
        const int sw_a = (l32 >> 1) & 7;
        uint32_t off_a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) off_a[s] = a_row * A_ROW + 16 * ((4 * h + s) ^ sw_a);
        const uint32_t off_b = A_BYTES + b_row * B_ROW + 16 * (h ^ ((l32 >> 3) & 1));
        const uint32_t off_bsf = A_BYTES + B_BYTES + b_row * 8 + 4 * h;

        half8_t fa[2][MI];      // A operands of substep s in fa[s & 1]
        u32x4 fb[2];            // packed B of the step: dword s = substep s
        uint32_t sb[2];         // B scale pair of the step (2 bytes)
        half8_t hb[2][2];       // converted B operands of substep s in hb[s & 1]
        half2_t spb[2];         // scale pairs of the current group of two substeps
        auto read_a = [&](int st, int s, half8_t (&dst)[MI]) {
            const uint8_t* pa = smem_raw + st * STAGE_BYTES + off_a[s];
#pragma unroll
            for (int i = 0; i < MI; ++i) dst[i] = *reinterpret_cast<const half8_t*>(pa + i * 32 * A_ROW);
        };
        auto read_b = [&](int st) {
            const uint8_t* base = smem_raw + st * STAGE_BYTES;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                fb[j] = *reinterpret_cast<const u32x4*>(base + off_b + j * 32 * B_ROW);
                sb[j] = *reinterpret_cast<const uint32_t*>(base + off_bsf + j * 32 * 8);
            }
        };
        auto deq_b = [&](int s, half8_t (&dst)[2]) {
            if ((s & 1) == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) spb[j] = scale_pair((sb[j] >> (8 * (s >> 1))) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) dst[j] = dequant8(fb[j][s], spb[j]);
        };

        // slot q (0..5) of the DMA of stage ks: slots 0 .. MI-1 are this wave's
        // A loads, slot MI its B load, slot MI + 1 its B scale load
        auto issue_one = [&](int ksr, int st, int q) {
            const int ks = kb + ksr;                   // absolute step
            uint8_t* base = smem_raw + st * STAGE_BYTES;
            if (q < MI) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (lds_void*)(base + (NA * wave + q) * 1024), 16, a_off[q], (uint32_t)ks * A_ROW, 0, 0);
            } else if (q == MI) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (lds_void*)(base + A_BYTES + wave * 1024), 16, b_off, (uint32_t)ks * kWqHalf, 0, 0);
            } else if (q == MI + 1) {
                // half step ks of K step kst = ks / 2: pairs 2 (ks % 2) + {0, 1}
                const int kst = ks >> 1;
                const uint32_t ksb = (uint32_t)((kst >> 2) * kWsfQuad + (kst & 3) * 2 + (ks & 1) * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rbsf, (lds_void*)(base + A_BYTES + B_BYTES + wave * 256), 2, bsf_off, ksb, 0, 0);
            }
        };

        auto issue_stage = [&](int ks, int st) {
#pragma unroll
            for (int q = 0; q < 6; ++q) issue_one(ks, st, q);
        };

        // One K step in four substeps. Substeps 0..2 run as two chunks, one
        // per B column block j: its MI MFMAs, the conversion of its operand of
        // the next substep, and one load slot of the refill of stage ks+2 (the
        // loads, issued back to back, stall the wave's instruction stream).
        // Substep 3 starts with the wait for this wave's DMA of stage ks+1 and
        // the barrier (the other waves' DMA of it is then visible, and the
        // buffer the refills of step ks+1 overwrite has been read by
        // everyone), reads the B fragments and the first A fragments of step
        // ks+1, and converts its first B operands between the later MFMAs.
        // Phase 0: steady state (refill, wait until NL loads remain); 1: the
        // last refill has been issued (wait until none remain); 2: the last
        // step. Every condition is a compile-time constant, so a step is one
        // basic block.
        auto step = [&](int ks, auto mode_c, int st) {
            constexpr int PH = decltype(mode_c)::value;
            const int sn = st == NSTAGE - 1 ? 0 : st + 1;          // stage of ks + 1
            const int sr = st == 0 ? NSTAGE - 1 : st - 1;          // stage of ks + 2
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                read_a(st, s + 1, fa[(s + 1) & 1]);
                if (s == 1) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) spb[j] = scale_pair((sb[j] >> 8) & 0xFFu);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s & 1][i], hb[s & 1][j],
                                                                            acc[i][j], 0, 0, 0);
                    hb[(s + 1) & 1][j] = dequant8(fb[j][s + 1], spb[j]);
                    if (PH == 0) issue_one(ks + NSTAGE - 1, sr, 2 * s + j);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);    // its VALU share
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (PH < 2) {
                // this wave's DMA of stage ks+1 is done when at most the loads
                // issued after it are outstanding; lgkmcnt(0): its own fragment
                // reads of this step are complete before it passes the barrier
                if (PH == 0) __builtin_amdgcn_s_waitcnt(kWaitStage);
                if (PH == 1) __builtin_amdgcn_s_waitcnt(kWaitAll);
                lds_barrier();
                read_b(sn);
                read_a(sn, 0, fa[0]);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[1][i], hb[1][j], acc[i][j], 0, 0, 0);
            if (PH < 2) {
                deq_b(0, hb[0]);
                // the fragment reads land under the first MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, MI + 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, kFirst, 0);
#pragma unroll
                for (int k = 0; k < 2 * MI - kFirst; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kValuLast, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // Pipeline: stages ks+1 and ks+2 are in flight while step ks computes;
        // the refill of stage ks+2 goes into the buffer step ks-1 used, which
        // every wave has finished reading at the barrier before step ks.
        issue_stage(0, 0);
        if (nk > 1) issue_stage(1, 1);
        // only stage 0 is needed now: wait until stage 1's loads are all that
        // is outstanding
        if (nk > 1) __builtin_amdgcn_s_waitcnt(kWaitStage);
        else __builtin_amdgcn_s_waitcnt(kWaitAll);
        lds_barrier();
        read_b(0);
        read_a(0, 0, fa[0]);
        deq_b(0, hb[0]);

        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        // steady state, NSTAGE steps per iteration (constant stage buffers);
        // then the remaining steps with the buffer computed at run time
        int ks = 0;
        for (; ks + NSTAGE + 1 < nk; ks += NSTAGE) {
            step(ks, P0{}, 0);
            step(ks + 1, P0{}, 1);
            step(ks + 2, P0{}, 2);
        }
        for (; ks + NSTAGE - 1 < nk; ++ks) step(ks, P0{}, ks % NSTAGE);
        if (ks + 1 < nk) {
            step(ks, P1{}, ks % NSTAGE);
            ++ks;
        }
        step(ks, P2{}, ks % NSTAGE);
        __syncthreads();

        // float32 rows of the tile (L2's output, or a dense K chunk's partial
        // sums): scale * acc to out (rows of N)
        auto store_f32 = [&](float* __restrict__ out, float scale) {
            // A lane holds four consecutive rows of one column per group of
            // four accumulator registers. A 4 x 4 transpose inside each quad of
            // lanes (two butterfly stages of quad-permute DPP moves) gives lane
            // 4c + m row m of that group at columns 4c .. 4c + 3, so every
            // store writes 16 contiguous bytes: 64 stores per lane instead of
            // 256 (the per-wave limit of 63 outstanding memory operations
            // otherwise stalls the epilogue on store latency several times).
            const int m = l32 & 3;
            const bool odd = (m & 1) != 0, upper = (m & 2) != 0;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int local = wm * (32 * MI) + 32 * i + 8 * g + 4 * h + m;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float v0 = scale * acc[i][j][4 * g], v1 = scale * acc[i][j][4 * g + 1];
                        float v2 = scale * acc[i][j][4 * g + 2], v3 = scale * acc[i][j][4 * g + 3];
                        // stage 1 (lanes m, m ^ 1): even lanes take the partner's
                        // v0 / v2 into v1 / v3, odd lanes its v1 / v3 into v0 / v2
                        const float s1a = odd ? v0 : v1, s1b = odd ? v2 : v3;
                        const float r1a = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                            __builtin_bit_cast(int, s1a), 0xB1, 0xF, 0xF, false));   // quad_perm(1,0,3,2)
                        const float r1b = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                            __builtin_bit_cast(int, s1b), 0xB1, 0xF, 0xF, false));
                        if (odd) { v0 = r1a; v2 = r1b; } else { v1 = r1a; v3 = r1b; }
                        // stage 2 (lanes m, m ^ 2): pairs (v0, v1) <-> (v2, v3)
                        const float s2a = upper ? v0 : v2, s2b = upper ? v1 : v3;
                        const float r2a = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                            __builtin_bit_cast(int, s2a), 0x4E, 0xF, 0xF, false));   // quad_perm(2,3,0,1)
                        const float r2b = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                            __builtin_bit_cast(int, s2b), 0x4E, 0xF, 0xF, false));
                        if (upper) { v0 = r2a; v1 = r2b; } else { v2 = r2a; v3 = r2b; }
                        const int64_t col = (int64_t)nt * BN + wn * 64 + 32 * j + 4 * (l32 >> 2);
                        if (local < row_count && col < N)   // N % 16 == 0: four columns are in or out together
                            *reinterpret_cast<float4_t*>(out + (row_start + local) * N + col) =
                                (float4_t){v0, v1, v2, v3};
                    }
                }
            }
        };
        // ---- epilogue ------------------------------------------------------------
        // acc[i][j][r] = D[row 32i + 8(r/4) + 4h + (r%4)][col 32j + l32] of the wave's part
        // L1 with per-half weight scales: gate columns take alpha, up alpha_up
        const int ast = (MODE == kGemmL1 && p.alpha_stride > 1) ? 2 : 1;
        const float alpha = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast];
        if (MODE == kGemmL1) {
            const float alpha_up = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast + ast - 1];
            // gate = the wave's block 0 (32 act columns), up = block 1.
            // All eight waves stage the rounded (gate, up) pairs of the whole
            // tile (64 * MI rows x 128 act columns) in the now idle LDS, rows
            // padded to 130 words (the two lane halves' rows, four apart, then
            // fall in different banks; 8-byte reads stay aligned); then all
            // threads apply SiLU and store act row by row (coalesced).
            constexpr int GU_LD = kGuLd;
            static_assert(64 * MI * GU_LD * 4 <= LDS_BYTES, "gate/up staging fits in LDS");
            uint32_t* gu = reinterpret_cast<uint32_t*>(smem_raw);     // [64 MI][GU_LD] g | u << 16
            uint32_t amax_bits = 0;
            typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
            u16x2_t amax_pair = {0, 0};
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * (32 * MI) + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int col = wn * 32 + l32;
                    gu[row * GU_LD + col] = pack_bf16x2_rne(alpha * acc[i][0][r], alpha_up * acc[i][1][r]);
                }
            __syncthreads();
            // each thread: one pair of adjacent act columns (one 4-byte store)
            // in rows tid / 64, + NT / 64, ...; a wave covers one row (256 contiguous
            // bytes), so the row bound is wave-uniform
            {
                const int cp = tid & 63;
                const int64_t col = (int64_t)nt * 128 + 2 * cp;   // I is even: no pair straddles I
                if (col < p.I) {
                    const int r0 = tid >> 6;
                    uint32_t* dst = reinterpret_cast<uint32_t*>(p.out_bf16 + (int64_t)(row_start + r0) * p.I + col);
                    constexpr int RS = NT / 64;                   // row step of a thread
                    const int64_t dstep = (int64_t)RS * (p.I / 2);    // RS rows of I bf16, in 4-byte units
                    const int rows = min(row_count, 64 * MI);
                    // Four rows per pass: their eight float32 SiLUs form one
                    // branch-free block of independent chains that hide the exp
                    // and rcp latencies, and the elements float32 cannot decide
                    // are redone in float64 after it, behind one branch that is
                    // rarely taken.
                    // optional tap of the rounded gate | up values (same rows,
                    // gate pair at column col, up pair at I + col)
                    // (has_tap is a kernel argument's test: a scalar branch, not a
                    // per-lane pointer test around every tap store)
                    const bool has_tap = p.gu_tap != nullptr;
                    uint32_t* tap = has_tap ? reinterpret_cast<uint32_t*>(
                                                  p.gu_tap + (int64_t)(row_start + r0) * 2 * p.I + col)
                                            : nullptr;
                    const int64_t tstep = (int64_t)RS * p.I;      // RS rows of 2I bf16, in 4-byte units
                    int r = r0;
                    for (; r + 3 * RS < rows; r += 4 * RS, dst += 4 * dstep) {
                        float g[8], u[8], v[8];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const u32x2 w = *reinterpret_cast<const u32x2*>(gu + (r + k * RS) * GU_LD + 2 * cp);
                            g[2 * k] = bf16_to_f32(w[0] & 0xFFFFu);
                            u[2 * k] = bf16_to_f32(w[0] >> 16);
                            g[2 * k + 1] = bf16_to_f32(w[1] & 0xFFFFu);
                            u[2 * k + 1] = bf16_to_f32(w[1] >> 16);
                            if (has_tap) {
                                tap[k * tstep] = (w[0] & 0xFFFFu) | (w[1] << 16);
                                tap[k * tstep + p.I / 2] = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
                            }
                        }
                        if (has_tap) tap += 4 * tstep;
                        // lanes with an element float32 cannot decide, as a
                        // wave mask (scalar ORs of the compare masks)
                        uint64_t redo = 0;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            v[i] = silu_mul_value(g[i], u[i]);
                            redo |= silu_f32_redo_lanes(g[i], v[i]);
                        }
                        uint32_t a[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) a[k] = pack_bf16x2_rne(v[2 * k], v[2 * k + 1]);
                        if (__builtin_expect(redo != 0, 0)) {
                            // the test is repeated here on values the compiler
                            // cannot see through, so the block above keeps only
                            // the combined flag (not eight per-element ones)
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                asm volatile("" : "+v"(g[i]), "+v"(v[i]));
                                if (!silu_f32_decides(g[i], v[i])) {
                                    const uint32_t b = silu_mul_bf16_f64(g[i], u[i]);
                                    a[i >> 1] = (i & 1) ? ((a[i >> 1] & 0xFFFFu) | (b << 16))
                                                        : ((a[i >> 1] & 0xFFFF0000u) | b);
                                }
                            }
                        }
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            dst[k * dstep] = a[k];
                            // |act| bit patterns of both halves, maximum per half
                            amax_pair = __builtin_elementwise_max(amax_pair,
                                                                  __builtin_bit_cast(u16x2_t, a[k] & 0x7FFF7FFFu));
                        }
                    }
                    for (; r < rows; r += RS, dst += dstep) {
                        const u32x2 w = *reinterpret_cast<const u32x2*>(gu + r * GU_LD + 2 * cp);
                        if (has_tap) {
                            tap[0] = (w[0] & 0xFFFFu) | (w[1] << 16);
                            tap[p.I / 2] = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
                            tap += tstep;
                        }
                        const uint32_t a = silu_mul_bf16x2(bf16_to_f32(w[0] & 0xFFFFu), bf16_to_f32(w[0] >> 16),
                                                           bf16_to_f32(w[1] & 0xFFFFu), bf16_to_f32(w[1] >> 16));
                        *dst = a;
                        amax_pair = __builtin_elementwise_max(amax_pair, __builtin_bit_cast(u16x2_t, a & 0x7FFF7FFFu));
                    }
                }
            }
            amax_bits = max((uint32_t)amax_pair[0], (uint32_t)amax_pair[1]);
            amax_bits = wave_max_u32(amax_bits);
            if (lane == 0) red[wave] = amax_bits;
            __syncthreads();
            if (tid == 0) {
                uint32_t m = red[0];
                for (int w = 1; w < NT / 64; ++w) m = max(m, red[w]);
                atomicMax(p.amax_slot, m << 16);
            }
        } else if (MODE == kGemmL2) {
            store_f32(p.out_f32, alpha);
        } else if (p.ksplit > 1) {
            store_f32(p.partial + (int64_t)chunk * p.M * N, 1.0f);
        } else {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int local = wm * (32 * MI) + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (local >= row_count) continue;
                    const int64_t prow = row_start + local;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int64_t col = (int64_t)nt * BN + wn * 64 + 32 * j + l32;
                        if (col >= N) continue;
                        const float v = alpha * acc[i][j][r];
                        p.out_bf16[prow * N + col] = (uint16_t)f32_to_bf16_rne(v);
                    }
                }
            }
        }
    };
    if (mi_tile >= 4) tile(std::integral_constant<int, 4>{});
    else if (mi_tile == 3) tile(std::integral_constant<int, 3>{});
    else if (mi_tile == 2) tile(std::integral_constant<int, 2>{});
    else tile(std::integral_constant<int, 1>{});
}

template <int MODE>
hipError_t launch_mode(const GemmParams& p, hipStream_t s) {
    const int64_t ntn = (MODE == kGemmL1) ? (p.I + 127) / 128 : (p.N + BN - 1) / BN;
    const int64_t mt = (MODE == kGemmDense) ? (p.M + dense_tile_rows(p.M, p.N) - 1) / dense_tile_rows(p.M, p.N)
                                            : p.max_tiles;
    // grouped: whole groups of 8 tiles (one per XCD); dense: every (tile, N-tile, K chunk)
    const int64_t grid = (MODE == kGemmDense) ? mt * ntn * p.ksplit : (mt + 7) / 8 * 8 * ntn;
    if (grid <= 0) return hipSuccess;
    static std::atomic<int> lds_set[kMaxDevices];
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_kernel<MODE>), LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    gemm_kernel<MODE><<<(unsigned)grid, NT, LDS_BYTES, s>>>(p);
    return hipGetLastError();
}

// One thread per 4 columns of one row: the chunks' partial sums in chunk
// order, times alpha, rounded once to bf16.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int ksplit,
                                                            int64_t M, int64_t N, const float* __restrict__ a_gs,
                                                            const float* __restrict__ b_alpha,
                                                            uint16_t* __restrict__ out) {
    const float alpha = a_gs[0] * b_alpha[0];
    const int64_t n4 = M * N / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const float* src = partial + 4 * i;
        float4_t acc = *reinterpret_cast<const float4_t*>(src);
        // loads in batches of 8 chunks, all in flight before the first add
        for (int c0 = 1; c0 < ksplit; c0 += 8) {
            float4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < ksplit) v[j] = *reinterpret_cast<const float4_t*>(src + (int64_t)(c0 + j) * M * N);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < ksplit) {
                    acc[0] = acc[0] + v[j][0];
                    acc[1] = acc[1] + v[j][1];
                    acc[2] = acc[2] + v[j][2];
                    acc[3] = acc[3] + v[j][3];
                }
        }
        u32x2 o;
        o[0] = f32_to_bf16_rne(alpha * acc[0]) | (f32_to_bf16_rne(alpha * acc[1]) << 16);
        o[1] = f32_to_bf16_rne(alpha * acc[2]) | (f32_to_bf16_rne(alpha * acc[3]) << 16);
        *reinterpret_cast<u32x2*>(out + 4 * i) = o;
    }
}

}  // namespace

int dense_ksplit(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = (M + dense_tile_rows(M, N) - 1) / dense_tile_rows(M, N) * ((N + BN - 1) / BN);
    const int64_t nk = pitch_q(K) / 32;
    if (tiles <= 0 || tiles >= 128 || nk < 8) return 1;
    // at most one work-group per CU: a second round would double the time
    int64_t s = 256 / tiles;
    if (s > nk / 4) s = nk / 4;
    if (s < 1) s = 1;
    // chunks of ceil(nk / s) steps; as many as that length needs, so that
    // none is empty
    const int64_t per = (nk + s - 1) / s;
    return (int)((nk + per - 1) / per);
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N, const float* a_gs,
                                const float* b_alpha, uint16_t* out, hipStream_t s) {
    const int64_t n4 = M * N / 4;
    if (n4 <= 0) return hipSuccess;
    const int64_t g = (n4 + 255) / 256;
    splitk_reduce_kernel<<<(unsigned)(g < 4096 ? g : 4096), 256, 0, s>>>(partial, ksplit, M, N, a_gs, b_alpha, out);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
    // 32-bit buffer offsets: every operand must stay below 2 GiB
    if (p.a_rows * pitch_h(p.K) >= 0x7FFFFFFF || p.N * pitch_q(p.K) >= 0x7FFFFFFF) return hipErrorInvalidValue;
    switch (p.mode) {
        case kGemmDense: return launch_mode<kGemmDense>(p, s);
        case kGemmL1: return launch_mode<kGemmL1>(p, s);
        case kGemmL2: return launch_mode<kGemmL2>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
