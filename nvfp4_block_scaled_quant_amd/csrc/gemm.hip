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
// Operands. A rows and B rows (one per weight column: the weights in the
// byte-transposed layout, as the pages' GEMM consumed B column-major) are
// both K-packed, 64 bytes per 128-element K step, with their E4M3 scales
// alongside; B comes in 16-row blocks whose K steps are contiguous (1 KB per
// step), so every load instruction of B reads one contiguous kilobyte. Tiles
// move from HBM to LDS by buffer loads that write LDS directly (no staging
// registers; out-of-range offsets read zeros), four stages deep (38 KB each).
//
// LDS layout. A stage holds 256 A rows and 256 B rows of 64 bytes, unpadded;
// the four 16-byte chunks of a row are XOR-swizzled with bits 2-3 of the row,
// so that the 16 rows read by a 16-lane group of the fragment loads cover all
// banks. Scales: 8 bytes per A row; per B row four dwords, one per pair of
// scale groups (the packed weights store a pair of groups of four consecutive
// K steps together, so a step's pairs are 2-byte pieces, and each is brought
// in by a 2-byte load that fills a whole LDS dword, zero-extended).
//
// Tiling. A work-group of 4 waves computes a 256 x 256 tile; each wave owns a
// 128 x 128 quadrant (4 x 4 tiles of 32 x 32 x 16). Lane l serves row / column
// l % 32 and K half h = l / 32: in a 128-element step it holds elements
// [64h, 64h + 64) (two 16-byte chunks), and substep s (0..7) feeds the MFMA
// elements [64h + 8s, +8), inside scale group 4h + s / 2; A and B use the same
// K permutation, so every k meets its own partner. The dequant of substep s + 1
// is issued between the MFMAs of substep s.
//
// Grouped scheduling. Tiles come from a device-built list (expert, first
// sorted row, row count); the grid is sized for the worst case and idle
// work-groups leave at once, so the host never waits for routing counts.
// Invalid rows and columns of a tile read a valid row instead (their results
// are never stored). Rows are read in whole 128-element steps: the padding of
// a partial last step is zero in both operands (the quantizers and the weight
// prepack write it as zeros), so it adds nothing.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int KB = 64;                 // packed bytes of K per step (128 elements)
constexpr int NT = 256;                // threads per work-group
constexpr int NSTAGE = 4;
constexpr int A_BYTES = BM * KB;       // 16 KB
constexpr int B_BYTES = BN * KB;
constexpr int ASF_BYTES = BM * 8;      // 2 KB
constexpr int BSF_BYTES = BN * 16;     // 4 KB: one dword per scale pair
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + ASF_BYTES + BSF_BYTES;
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;   // 152 KB
constexpr uint32_t kRsrcWord3 = 0x00020000u;        // raw buffer, 32-bit data format

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

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int64_t K = p.K, N = p.N;
    const int64_t ldq = pitch_q(K), ldsf = pitch_sf(K);      // padded row pitches (A)
    const int64_t ldwsf = pitch_wsf(K);                       // packed weight scales
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
        // both loads at once (tile_idx < max_tiles: the entry exists, and is
        // used only when it is one of the num_tiles valid ones)
        const Tile t = p.tiles[tile_idx];
        const int ntiles = *p.num_tiles;
        // keeps the tile load above the branch (the compiler would sink it)
        asm volatile("" ::"s"(t.expert), "s"(t.row_start), "s"(t.row_count));
        if (tile_idx >= ntiles) return;
        expert = t.expert;
        row_start = t.row_start;
        row_count = t.row_count;
    }
    // Each wave covers MI blocks of 32 rows, so a tile computes 64 * MI rows:
    // the last tile of an expert usually holds fewer than 256 (at the prefill
    // shape about 171 of 256 on average), and its MFMAs shrink with it. The
    // loads still bring in all 256 rows (the extra ones repeat a valid row).
    const int mi_tile = __builtin_amdgcn_readfirstlane((row_count + 63) / 64);
    __shared__ uint32_t red[NT / 64];
    auto tile = [&](auto mi_c) {
        constexpr int MI = decltype(mi_c)::value;
        // VALU per MFMA in the substeps' schedules: the dequant of one
        // substep is about 11 VALU per operand (MI + 4 operands) spread over
        // its 4 * MI MFMAs; the last substep's first kFirst MFMAs cover the
        // fragment reads
        constexpr int kValu = MI == 4 ? 5 : MI == 3 ? 6 : MI == 2 ? 8 : 14;
        constexpr int kFirst = MI == 1 ? 2 : 6;
        constexpr int kValuLast = MI == 4 ? 8 : MI == 3 ? 13 : MI == 2 ? 33 : 28;

        // ---- buffer resources and per-lane DMA offsets ---------------------------
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aq, p.a_rows * ldq);
        const __amdgpu_buffer_rsrc_t rasf = make_rsrc(p.asf, p.a_rows * ldsf);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bq + (int64_t)expert * N * ldq, N * ldq);
        const __amdgpu_buffer_rsrc_t rbsf = make_rsrc(p.bsf + (int64_t)expert * N * ldwsf, N * ldwsf);

        auto a_src = [&](int r) -> int64_t {        // A tensor row of tile row r
            int64_t src = row_start + (r < row_count ? r : 0);
            if (MODE == kGemmL1) src = p.a_gather[src] / p.topk;
            return src;
        };
        auto b_src = [&](int vc) -> int64_t {       // weight row (output column) of virtual column vc
            if (MODE == kGemmL1) {
                const int w = vc >> 7, r = vc & 127;
                const int64_t base = (int64_t)nt * 128 + 64 * w + (r & 63);
                if (base >= p.I) return 0;
                return (r < 64) ? base : p.I + base;
            }
            const int64_t c = (int64_t)nt * BN + vc;
            return c < N ? c : 0;
        };
        // data: wave w, instruction t (0..3) fills LDS slots (4w + t) * 64 + lane of
        // 16 bytes: row (4w + t) * 16 + lane / 4, physical chunk lane & 3
        uint32_t a_off[4], b_off[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int row = (4 * wave + t) * 16 + (lane >> 2);
            const int chunk = swz(row, lane & 3);
            a_off[t] = (uint32_t)(a_src(row) * ldq + 16 * chunk);
            b_off[t] = (uint32_t)(wq_row(b_src(row), ldq) + 16 * chunk);
        }
        // A scales: wave w, instruction t (0..1) fills 4-byte slots (2w + t) * 64 +
        // lane: row (2w + t) * 32 + lane / 2, bytes 4 * (lane & 1) .. +4 of the
        // step's 8. B scales: instruction t (0..3) fills dword (4w + t) * 64 + lane
        // with pair lane & 3 of row (4w + t) * 16 + lane / 4.
        uint32_t asf_off[2], bsf_off[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = (2 * wave + t) * 32 + (lane >> 1);
            asf_off[t] = (uint32_t)(a_src(row) * ldsf + 4 * (lane & 1));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bsf_off[t] = (uint32_t)wsf_off(b_src((4 * wave + t) * 16 + (lane >> 2)), ldwsf, 0, lane & 3);

        const int nk = (int)(ldq / KB);
        // part t (0..5) of the DMA of stage ks: t < 4 one A and one B data load,
        // t = 4, 5 one A and two B scale loads
        auto issue_part = [&](int ks, int t) {
            uint8_t* base = smem_raw + (ks % NSTAGE) * STAGE_BYTES;
            // A rows advance by 64 bytes per step, packed weight blocks by 1 KB
            const uint32_t kda = (uint32_t)ks * KB, kdb = (uint32_t)ks * kWqStep;
            const uint32_t ksa = (uint32_t)ks * 8, ksb = (uint32_t)((ks >> 2) * kWsfQuad + (ks & 3) * 2);
            if (t < 4) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(base + (4 * wave + t) * 1024),
                                                         16, a_off[t], kda, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(base + A_BYTES + (4 * wave + t) * 1024),
                                                         16, b_off[t], kdb, 0, 0);
            } else {
                const int u = t - 4;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rasf, (lds_void*)(base + A_BYTES + B_BYTES + (2 * wave + u) * 256), 4, asf_off[u], ksa, 0, 0);
#pragma unroll
                for (int v = 2 * u; v < 2 * u + 2; ++v)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rbsf, (lds_void*)(base + A_BYTES + B_BYTES + ASF_BYTES + (4 * wave + v) * 256), 2,
                        bsf_off[v], ksb, 0, 0);
            }
        };
        auto issue_stage = [&](int ks) {
#pragma unroll
            for (int t = 0; t < 6; ++t) issue_part(ks, t);
        };

        // ---- main loop ---------------------------------------------------------
        const int wm = wave >> 1, wn = wave & 1;
        const int l32 = lane & 31, h = lane >> 5;

        float16_t acc[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        u32x4 fa[MI][2], fb[4][2];
        uint32_t sa[MI];
        u32x2 sb[4];      // B scale pairs 2h, 2h + 1: bytes 0-1 of each dword
        // Fragment rows are wm * 32 MI + 32 i + l32 (A) and wn * 128 + 32 j + l32
        // (B): the 32 i / 32 j parts are multiples of 16, so the swizzle (bits
        // 2-3 of the row) depends on the lane alone. Six per-lane offsets
        // within a stage are formed once; per step each gets the stage base
        // added once, and the fragments' row offsets are constants (the LDS
        // reads' immediate offsets), instead of a full address per read.
        const int sw = (l32 >> 2) & 3;
        const uint32_t a_row = (uint32_t)(wm * (32 * MI) + l32), b_row = (uint32_t)(wn * 128 + l32);
        const uint32_t off_a0 = a_row * KB + 16 * ((2 * h) ^ sw);
        const uint32_t off_a1 = a_row * KB + 16 * ((2 * h + 1) ^ sw);
        const uint32_t off_b0 = A_BYTES + b_row * KB + 16 * ((2 * h) ^ sw);
        const uint32_t off_b1 = A_BYTES + b_row * KB + 16 * ((2 * h + 1) ^ sw);
        const uint32_t off_asf = A_BYTES + B_BYTES + a_row * 8 + 4 * h;
        const uint32_t off_bsf = A_BYTES + B_BYTES + ASF_BYTES + b_row * 16 + 8 * h;
        auto read_frags = [&](int ks) {
            const uint8_t* base = smem_raw + (ks % NSTAGE) * STAGE_BYTES;
            const uint8_t* pa0 = base + off_a0;
            const uint8_t* pa1 = base + off_a1;
            const uint8_t* pb0 = base + off_b0;
            const uint8_t* pb1 = base + off_b1;
            const uint8_t* pas = base + off_asf;
            const uint8_t* pbs = base + off_bsf;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                fa[i][0] = *reinterpret_cast<const u32x4*>(pa0 + i * 32 * KB);
                fa[i][1] = *reinterpret_cast<const u32x4*>(pa1 + i * 32 * KB);
                sa[i] = *reinterpret_cast<const uint32_t*>(pas + i * 32 * 8);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fb[j][0] = *reinterpret_cast<const u32x4*>(pb0 + j * 32 * KB);
                fb[j][1] = *reinterpret_cast<const u32x4*>(pb1 + j * 32 * KB);
                // pairs 2h and 2h + 1, each in the low half of its dword (the
                // dequant picks the byte from either, no joining needed)
                sb[j] = *reinterpret_cast<const u32x2*>(pbs + j * 32 * 16);
            }
        };
        // operands of substep s in registers s & 1
        half8_t ha[2][MI], hb[2][4];
        // scale pairs of the current group of two substeps (one scale group):
        // formed on even substeps, reused on the odd ones (also across the
        // step boundary: substep 0 is dequantized at the end of the previous
        // step)
        half2_t spa[MI], spb[4];
        auto deq = [&](int s, half8_t (&xa)[MI], half8_t (&xb)[4]) {
            if ((s & 1) == 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i) spa[i] = scale_pair((sa[i] >> (8 * (s >> 1))) & 0xFFu);
#pragma unroll
                for (int j = 0; j < 4; ++j) spb[j] = scale_pair((sb[j][s >> 2] >> (8 * ((s >> 1) & 1))) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) xa[i] = dequant8(fa[i][s >> 2][s & 3], spa[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) xb[j] = dequant8(fb[j][s >> 2][s & 3], spb[j]);
        };

        // Pipeline: stages ks+1..ks+3 are in flight while step ks computes. Every
        // substep s issues its 16 MFMAs with the dequant of substep s + 1 between
        // them. Substep 7 starts with the wait for this wave's DMA of stage ks+1
        // and the barrier (the other waves' DMA of it is then visible, and buffer
        // (ks-1) % 4, which the next step refills, has been read by everyone),
        // reads the fragments of step ks+1, and dequantizes substep 0 of step ks+1
        // between its later MFMAs, so that no dequant runs outside an MFMA shadow.
        // Scheduling barriers keep each substep's instructions together.
        for (int s0 = 0; s0 < NSTAGE - 1 && s0 < nk; ++s0) issue_stage(s0);
        // only stage 0 is needed now: wait until the later stages' loads are
        // all that is outstanding (14 per stage), not for all of them
        if (nk >= 3) __builtin_amdgcn_s_waitcnt(0x407C);        // vmcnt(28) lgkmcnt(0)
        else if (nk == 2) __builtin_amdgcn_s_waitcnt(0x007E);   // vmcnt(14) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x0070);                // vmcnt(0) lgkmcnt(0)
        lds_barrier();
        read_frags(0);
        deq(0, ha[0], hb[0]);

        // One K step. Phase 0: steady state (refill a stage, wait until 28 loads
        // remain, fetch the next step); 1 and 2: the last two refills have been
        // issued (wait until 14 / 0 remain); 3: the last step. Every condition is a
        // compile-time constant, so a step is one basic block the scheduler can
        // interleave freely.
        auto step = [&](int ks, auto mode_c) {
            constexpr int PH = decltype(mode_c)::value;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                // the refill of stage ks+3 is spread over substeps 0..5: a burst of
                // fourteen LDS-DMA issues at once stalls the MFMA stream
                if (PH == 0 && s < 6) issue_part(ks + NSTAGE - 1, s);
                if (s < 7) {
                    deq(s + 1, ha[(s + 1) & 1], hb[(s + 1) & 1]);
                } else if (PH < 3) {
                    // this wave's DMA of stage ks+1 is done when at most the stages
                    // issued after it are outstanding; lgkmcnt(0): its own fragment
                    // reads of this step are complete before it passes the barrier
                    if (PH == 0) __builtin_amdgcn_s_waitcnt(0x407C);        // vmcnt(28) lgkmcnt(0)
                    if (PH == 1) __builtin_amdgcn_s_waitcnt(0x007E);        // vmcnt(14) lgkmcnt(0)
                    if (PH == 2) __builtin_amdgcn_s_waitcnt(0x0070);        // vmcnt(0) lgkmcnt(0)
                    lds_barrier();
                    read_frags(ks + 1);
                }
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[s & 1][i], hb[s & 1][j],
                                                                            acc[i][j], 0, 0, 0);
                if (s < 7) {
#pragma unroll
                    for (int k = 0; k < 4 * MI; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);   // its VALU share
                    }
                } else if (PH < 3) {
                    deq(0, ha[0], hb[0]);
                    // the fragment reads land under the first MFMAs
                    __builtin_amdgcn_sched_group_barrier(0x100, 3 * MI + 12, 0);  // the LDS reads
                    __builtin_amdgcn_sched_group_barrier(0x008, kFirst, 0);
#pragma unroll
                    for (int k = 0; k < 4 * MI - kFirst; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, kValuLast, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        int ks = 0;
        for (; ks + NSTAGE - 1 < nk; ++ks) step(ks, std::integral_constant<int, 0>{});
        if (nk - ks == 3) step(ks++, std::integral_constant<int, 1>{});
        if (nk - ks == 2) step(ks++, std::integral_constant<int, 2>{});
        step(ks, std::integral_constant<int, 3>{});
        __syncthreads();

        // ---- epilogue ------------------------------------------------------------
        // acc[i][j][r] = D[row 32i + 8(r/4) + 4h + (r%4)][col 32j + l32] of the quadrant
        // L1 with per-half weight scales: gate columns take alpha, up alpha_up
        const int ast = (MODE == kGemmL1 && p.alpha_stride > 1) ? 2 : 1;
        const float alpha = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast];
        if (MODE == kGemmL1) {
            const float alpha_up = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast + ast - 1];
            // gate = virtual columns [0, 64) of the quadrant (blocks 0, 1), up = [64, 128).
            // All four waves stage the rounded (gate, up) pairs of the whole
            // tile (64 * MI rows x 128 act columns) in the now idle LDS, rows
            // padded to 130 words (the two lane halves' rows, four apart, then
            // fall in different banks; 8-byte reads stay aligned); then all
            // threads apply SiLU and store act row by row (coalesced).
            constexpr int GU_LD = 130;
            static_assert(64 * MI * GU_LD * 4 <= LDS_BYTES, "gate/up staging fits in LDS");
            uint32_t* gu = reinterpret_cast<uint32_t*>(smem_raw);     // [64 MI][GU_LD] g | u << 16
            uint32_t amax_bits = 0;
            typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
            u16x2_t amax_pair = {0, 0};
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int row = wm * (32 * MI) + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                        const int col = wn * 64 + 32 * j + l32;
                        gu[row * GU_LD + col] = pack_bf16x2_rne(alpha * acc[i][j][r], alpha_up * acc[i][j + 2][r]);
                    }
            __syncthreads();
            // each thread: one pair of adjacent act columns (one 4-byte store)
            // in rows tid / 64, + 4, ...; a wave covers one row (256 contiguous
            // bytes), so the row bound is wave-uniform
            {
                const int cp = tid & 63;
                const int64_t col = (int64_t)nt * 128 + 2 * cp;   // I is even: no pair straddles I
                if (col < p.I) {
                    const int r0 = tid >> 6;
                    uint32_t* dst = reinterpret_cast<uint32_t*>(p.out_bf16 + (int64_t)(row_start + r0) * p.I + col);
                    const int64_t dstep = 2 * p.I;                // 4 rows, in 4-byte units
                    const int rows = min(row_count, 64 * MI);
                    // Four rows per pass: their eight float32 SiLUs form one
                    // branch-free block of independent chains (one wave per SIMD
                    // has nothing else to hide the exp / rcp latencies), and the
                    // elements float32 cannot decide are redone in float64 after
                    // it, behind one branch that is rarely taken.
                    constexpr int RS = NT / 64;                   // row step of a thread
                    // optional tap of the rounded gate | up values (same rows,
                    // gate pair at column col, up pair at I + col)
                    uint32_t* tap = p.gu_tap ? reinterpret_cast<uint32_t*>(
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
                            if (tap) {
                                tap[k * tstep] = (w[0] & 0xFFFFu) | (w[1] << 16);
                                tap[k * tstep + p.I / 2] = (w[0] >> 16) | (w[1] & 0xFFFF0000u);
                            }
                        }
                        if (tap) tap += 4 * tstep;
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
                        if (tap) {
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
                uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
                atomicMax(p.amax_slot, m << 16);
            }
        } else if (MODE == kGemmL2) {
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
                    for (int j = 0; j < 4; ++j) {
                        float v0 = alpha * acc[i][j][4 * g], v1 = alpha * acc[i][j][4 * g + 1];
                        float v2 = alpha * acc[i][j][4 * g + 2], v3 = alpha * acc[i][j][4 * g + 3];
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
                        const int64_t col = (int64_t)nt * BN + wn * 128 + 32 * j + 4 * (l32 >> 2);
                        if (local < row_count && col < N)   // N % 16 == 0: four columns are in or out together
                            *reinterpret_cast<float4_t*>(p.out_f32 + (row_start + local) * N + col) =
                                (float4_t){v0, v1, v2, v3};
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int local = wm * (32 * MI) + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
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
    };
    if (mi_tile >= 4) tile(std::integral_constant<int, 4>{});
    else if (mi_tile == 3) tile(std::integral_constant<int, 3>{});
    else if (mi_tile == 2) tile(std::integral_constant<int, 2>{});
    else tile(std::integral_constant<int, 1>{});
}

template <int MODE>
hipError_t launch_mode(const GemmParams& p, hipStream_t s) {
    const int64_t ntn = (MODE == kGemmL1) ? (p.I + 127) / 128 : (p.N + BN - 1) / BN;
    const int64_t mt = (MODE == kGemmDense) ? (p.M + BM - 1) / BM : p.max_tiles;
    const int64_t grid = mt * ntn;
    if (grid <= 0) return hipSuccess;
    static std::atomic<int> lds_set[kMaxDevices];
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_kernel<MODE>), LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    gemm_kernel<MODE><<<(unsigned)grid, NT, LDS_BYTES, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
    // 32-bit buffer offsets: every operand must stay below 2 GiB
    if (p.a_rows * pitch_q(p.K) >= 0x7FFFFFFF || p.N * pitch_q(p.K) >= 0x7FFFFFFF) return hipErrorInvalidValue;
    switch (p.mode) {
        case kGemmDense: return launch_mode<kGemmDense>(p, s);
        case kGemmL1: return launch_mode<kGemmL1>(p, s);
        case kGemmL2: return launch_mode<kGemmL2>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
