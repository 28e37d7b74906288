// Weight-streaming grouped GEMMs for small batches (decode): the same two
// expert GEMMs as gemm.hip (NVFP4 MegaMoE Debug Log, "NVFP4 MoE Pipeline", L1 with fused
// SiLU(gate) * up and L2), for tiles of at most 16 rows.
//
// With a handful of rows per expert the layer is bound by reading the expert
// weights from HBM once, so the kernel is built around the weight stream:
//
// * A work-group of 8 waves (two per SIMD, one work-group per CU) owns one
//   16-row tile and a slab of 8 x 16 NB weight rows (output columns; NB = 10
//   for L2; for L1, NB = 8: 8 x 64 gate columns and the matching up columns).
//   Its 16 A rows are staged once in LDS, still packed, while the first weight
//   loads are already in flight (weight step 0, then the A rows, then weight
//   step 1: loads return in order). (With 4 waves, two work-groups shared a CU and
//   the one dispatched second finished about a third later, alone on the CU
//   for the tail; one 8-wave work-group per CU streams evenly to the end.)
// * Each wave streams its own 16 NB weight rows over the whole of K, two K
//   steps in flight, with non-temporal loads (the weights are read once),
//   and finishes its outputs by itself (no cross-wave reduction). Per
//   128-element K step, lane (c, q) = (lane % 16, lane / 16) loads 16
//   contiguous bytes (32 K values, [32q, 32q + 32) of the step) from each of
//   NB weight rows: column c of the NB MFMA column blocks f (block f
//   holds weight rows 16f + c of the wave's 16 NB). In the packed weight layout
//   one such load instruction (16 rows x 64 bytes of one K step of a 16-row
//   block, stored as two half steps of 16 x 32 bytes) reads one contiguous
//   kilobyte.
//   Dword s of a load is the B operand of v_mfma_f32_16x16x32_f16 for
//   substep s (K values 32q + 8s .. +8 of the step); A rows are read from LDS
//   with the same K permutation, so every k meets its own partner. Nothing of
//   B goes through LDS.
// * The packed weight scales keep the two scale bytes a lane needs per step
//   together for four consecutive steps (8 bytes; a wave's 64 lanes read 512
//   contiguous bytes), so scales are loaded only with the first step of each
//   group of four (and with the first step a wave streams, which may fall
//   inside a group) and are kept in registers for the group's other steps.
// * Dequantization is exact (E2M1 x E4M3 in f16, see common.hpp); the
//   epilogue applies alpha once (and for L1 the bf16 roundings and SiLU).
//
// For L1, blocks f < 4 are gate columns 16f + c of the wave's 64 and blocks
// f + 4 the matching up columns, so gate and up of one output column sit in
// the same lane and accumulator position.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int NT = 512;
constexpr int NW = NT / 64;       // waves per work-group (two per SIMD)
constexpr int SM = 16;            // rows per tile
// MFMA column blocks per lane (weight rows 16f + c of the wave's 16 * NB):
// L1 4 gate + 4 up blocks; L2 10 blocks, so that a tile needs 6 work-groups
// for 7168 output columns instead of 7 at 8 blocks: the decode batch touches
// up to about 42 experts, and 42 x 6 work-groups still fit the 256 that the
// GPU holds at once (one per CU), where 37 x 7 already need a second round
// whose few work-groups each take a whole stream's latency-bound time
template <int MODE> constexpr int kNB = MODE == kGemmL1 ? 8 : 10;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kStreamNT = 2;      // buffer-load cache policy: non-temporal (read once)
constexpr int kStagger = 13;      // start offset (in groups of four K steps) between waves

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// work-group slabs per tile: L1 in act columns (16 * NB / 2 per wave), L2 in rows (16 * NB)
__host__ __device__ inline int64_t skinny_slabs(int mode, int64_t I, int64_t N) {
    constexpr int c1 = NW * 16 * (kNB<kGemmL1> / 2), c2 = NW * 16 * kNB<kGemmL2>;
    return mode == kGemmL1 ? (I + c1 - 1) / c1 : (N + c2 - 1) / c2;
}

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void skinny_kernel(GemmParams p) {
    constexpr int NB = kNB<MODE>;
    constexpr int WROWS = 16 * NB;    // weight rows per wave
    constexpr int GB = NB / 2;        // L1: gate blocks (and as many up blocks) per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t K = p.K, N = p.N, Kg = K / 16;
    const int64_t ldq = pitch_q(K), ldsf = pitch_sf(K), ldwsf = pitch_wsf(K);
    const int nslab = (int)skinny_slabs(MODE, p.I, N);
    const int tile_idx = blockIdx.x / nslab;
    const int slab = blockIdx.x - tile_idx * nslab;
    // both loads at once (tile_idx < max_tiles: the entry exists, and is used
    // only when it is one of the num_tiles valid ones)
    const Tile tl = p.tiles[tile_idx];
    const int ntiles = *p.num_tiles;
    // keeps the tile load above the branch (the compiler would sink it)
    asm volatile("" ::"s"(tl.expert), "s"(tl.row_start), "s"(tl.row_count));
    if (tile_idx >= ntiles) return;
    // the tile is the same for the whole work-group: keep its fields scalar, so
    // that the weight buffer descriptors are uniform
    const int expert = __builtin_amdgcn_readfirstlane(tl.expert);
    const int row_start = __builtin_amdgcn_readfirstlane(tl.row_start);
    const int row_count = __builtin_amdgcn_readfirstlane(tl.row_count);

    // ---- this lane's NB weight rows -------------------------------------------
    const int c = lane & 15, q = lane >> 4;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bq + (int64_t)expert * N * ldq, N * ldq);
    const __amdgpu_buffer_rsrc_t rbsf = make_rsrc(p.bsf + (int64_t)expert * N * ldwsf, N * ldwsf);
    // first output column of this wave: L1 act column, L2 weight row
    const int64_t col0 = (MODE == kGemmL1) ? ((int64_t)slab * NW + wave) * 16 * GB
                                           : ((int64_t)slab * NW + wave) * WROWS;
    uint32_t boff[NB], sfoff[NB];
    bool ok[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
        int64_t row;
        if (MODE == kGemmL1) {
            const int64_t a = col0 + 16 * (f % GB) + c;
            ok[f] = a < p.I;
            row = ok[f] ? ((f < GB) ? a : p.I + a) : 0;
        } else {
            row = col0 + 16 * f + c;
            ok[f] = row < N;
            row = ok[f] ? row : 0;
        }
        boff[f] = (uint32_t)wq_off(row, ldq, 16 * q);       // bytes [16q, 16q + 16) of step 0
        sfoff[f] = (uint32_t)wsf_off(row, ldwsf, 0, q);
    }
    // a wave whose columns all lie beyond the matrix streams nothing
    const bool active = (MODE == kGemmL1) ? (col0 < p.I) : (col0 < N);
    const int nsteps = active ? (int)(ldq / 64) : 0;
    // Waves start at different K steps and wrap around, so that at any moment
    // the concurrent streams spread over the memory channels instead of all
    // starting at the same offset of their blocks. Starts are whole groups of
    // four steps (when K has whole groups; else every wave starts at 0), so
    // that loop step i begins a scale group exactly when i % 4 == 0. The
    // order of the fp32 partial sums is fixed per output column.
    const int ngroups = nsteps / 4;
    const int s0 = (nsteps % 4 == 0 && ngroups)
                       ? 4 * (int)(((int64_t)blockIdx.x * NW + wave) * kStagger % ngroups) : 0;
    auto kstep = [&](int i) { return i + s0 < nsteps ? i + s0 : i + s0 - nsteps; };

    struct Raw {
        u32x4 w[NB];
        u32x2 s[NB];      // scales of four steps, loaded with the group's first step
    };
    // Loop step i with i % 4 == 0 brings (and uses) a new group of scales. `ng`
    // is that condition, a compile-time constant in the steady-state loop:
    // there every iteration issues the same loads, so the compiler's waits
    // for a step's registers let the next step's loads stay in flight.
    auto load = [&](int i, Raw& rw, auto ng) {
        // the step offsets go to the scalar offset operand: keep them uniform
        const int st = kstep(i);
        const uint32_t kd = __builtin_amdgcn_readfirstlane((uint32_t)st * kWqStep);
        if (ng) {
            const uint32_t ksf = __builtin_amdgcn_readfirstlane((uint32_t)(st >> 2) * kWsfQuad);
#pragma unroll
            for (int f = 0; f < NB; ++f)
                rw.s[f] = __builtin_amdgcn_raw_buffer_load_b64(rbsf, sfoff[f], ksf, kStreamNT);
        }
#pragma unroll
        for (int f = 0; f < NB; ++f)
            rw.w[f] = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[f], kd, kStreamNT);
    };
    const std::true_type kNew;
    const std::false_type kOld;

    // Loads return in order, so the prologue issues them in the order they
    // are needed: the A tensor row of each tile row (-1: none), weight step
    // 0, the A rows of the tile (staged into LDS below), then weight step 1.
    // Both weight loads are issued on every path into the main loop, in this
    // order (a wave with fewer steps loads step 0 again), so that the
    // compiler's waits at the loop head are the ones of the steady state.
    int64_t my_src = -1;
    if (tid < SM && tid < row_count) {
        my_src = row_start + tid;
        if (MODE == kGemmL1) my_src = p.a_gather[my_src] / p.topk;
    }
    Raw r0, r1;
    load(0, r0, kNew);
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage the tile's A rows (packed, pitch ldq) and scales into LDS ------
    uint8_t* sA = smem;                              // [16][ldq + 16]
    const int a_pitch = (int)ldq + 16;               // 16-byte skew between rows
    uint8_t* sAsf = smem + SM * a_pitch;             // [16][ldsf]
    __shared__ int64_t src_row[SM];
    if (tid < SM) src_row[tid] = my_src;
    __syncthreads();
    // scales in 8-byte pieces (groups beyond K are masked in compute()), data
    // in 16-byte pieces; the first pass's loads are issued before weight step
    // 1, so that writing them to LDS waits for step 0 only
    const int cs = (int)(ldsf / 8), ns = SM * cs;
    const int cq = (int)(ldq / 16), nq = SM * cq;
    auto load_sf = [&](int i) -> u32x2 {
        const int r = i / cs, j = i - r * cs;
        return (i < ns && src_row[r] >= 0) ? *reinterpret_cast<const u32x2*>(p.asf + src_row[r] * ldsf + 8 * j)
                                           : (u32x2){0u, 0u};
    };
    auto load_q = [&](int i) -> u32x4 {
        const int r = i / cq, j = i - r * cq;
        return (i < nq && src_row[r] >= 0) ? *reinterpret_cast<const u32x4*>(p.aq + src_row[r] * ldq + 16 * j)
                                           : (u32x4){0u, 0u, 0u, 0u};
    };
    auto store_sf = [&](int i, u32x2 v) {
        const int r = i / cs, j = i - r * cs;
        if (i < ns) *reinterpret_cast<u32x2*>(sAsf + r * ldsf + 8 * j) = v;
    };
    auto store_q = [&](int i, u32x4 v) {
        const int r = i / cq, j = i - r * cq;
        if (i < nq) *reinterpret_cast<u32x4*>(sA + r * a_pitch + 16 * j) = v;
    };
    u32x2 vs[4];
    u32x4 vq[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) vs[u] = load_sf(tid + u * NT);
#pragma unroll
    for (int u = 0; u < 8; ++u) vq[u] = load_q(tid + u * NT);
    __builtin_amdgcn_sched_barrier(0);

    load(nsteps > 1 ? 1 : 0, r1, kOld);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < 4; ++u) store_sf(tid + u * NT, vs[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) store_q(tid + u * NT, vq[u]);
    // further passes (long rows), eight loads in flight per thread
    for (int i0 = tid + 4 * NT; i0 < ns; i0 += 4 * NT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) vs[u] = load_sf(i0 + u * NT);
#pragma unroll
        for (int u = 0; u < 4; ++u) store_sf(i0 + u * NT, vs[u]);
    }
    for (int i0 = tid + 8 * NT; i0 < nq; i0 += 8 * NT) {
#pragma unroll
        for (int u = 0; u < 8; ++u) vq[u] = load_q(i0 + u * NT);
#pragma unroll
        for (int u = 0; u < 8; ++u) store_q(i0 + u * NT, vq[u]);
    }
    __syncthreads();

    float4_t acc[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[f] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // scales of the current group; the low 16 bits belong to the step at hand
    uint64_t cur[NB];

    auto compute = [&](int i, const Raw& rw, auto ng) {
        const int st = kstep(i);
        // A row c, bytes [16q, 16q + 16) of the step; scale groups 2q, 2q + 1
        const u32x4 aw = *reinterpret_cast<const u32x4*>(sA + c * a_pitch + st * 64 + 16 * q);
        uint32_t as = (uint32_t)sAsf[c * ldsf + st * 8 + 2 * q] |
                      ((uint32_t)sAsf[c * ldsf + st * 8 + 2 * q + 1] << 8);
        // groups beyond K (padding of the last step) get scale 0
        const int64_t g0 = (int64_t)st * 8 + 2 * q;
        const uint32_t mask = (g0 < Kg ? 0xFFu : 0u) | (g0 + 1 < Kg ? 0xFF00u : 0u);
        as &= mask;
        if (ng) {
#pragma unroll
            for (int f = 0; f < NB; ++f) cur[f] = ((uint64_t)rw.s[f][1] << 32) | rw.s[f][0];
        }
        // B scales of groups beyond K are zero in the packed layout
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8_t ha = dequant8(aw[s], scale_pair((as >> (8 * (s >> 1))) & 0xFFu));
#pragma unroll
            for (int f = 0; f < NB; ++f) {
                const uint32_t code = ((uint32_t)cur[f] >> (8 * (s >> 1))) & 0xFFu;
                const half8_t hb = dequant8(rw.w[f][s], scale_pair(code));
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, acc[f], 0, 0, 0);
            }
        }
#pragma unroll
        for (int f = 0; f < NB; ++f) cur[f] >>= 16;
    };

    // Two steps in flight: r0 holds the even loop steps, r1 the odd ones. The
    // steady-state loop covers four steps per iteration (one scale group);
    // the last at most five steps run through the general loop below.
    // Scheduling barriers keep each step's MFMAs (and so the waits for its
    // registers) from being hoisted into the step before.
    int i = 0;
    for (; i + 5 < nsteps; i += 4) {
        compute(i, r0, kNew);
        load(i + 2, r0, kOld);
        __builtin_amdgcn_sched_barrier(0);
        compute(i + 1, r1, kOld);
        load(i + 3, r1, kOld);
        __builtin_amdgcn_sched_barrier(0);
        compute(i + 2, r0, kOld);
        load(i + 4, r0, kNew);
        __builtin_amdgcn_sched_barrier(0);
        compute(i + 3, r1, kOld);
        load(i + 5, r1, kOld);
        __builtin_amdgcn_sched_barrier(0);
    }
    while (i < nsteps) {
        compute(i, r0, (i & 3) == 0);
        ++i;
        if (i >= nsteps) break;
        if (i + 1 < nsteps) load(i + 1, r0, (i & 3) == 3);
        compute(i, r1, (i & 3) == 0);
        ++i;
        if (i + 1 < nsteps) load(i + 1, r1, (i & 3) == 3);
    }

    // ---- epilogue: acc[f][i] = D[tile row 4q + i][column c of block f] --------
    // L1 with per-half weight scales: gate columns take alpha, up alpha_up
    const int ast = (MODE == kGemmL1 && p.alpha_stride > 1) ? 2 : 1;
    const float alpha = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast];
    if (MODE == kGemmL1) {
        const float alpha_up = p.a_gs[0] * p.b_alpha[(int64_t)expert * ast + ast - 1];
        uint32_t amax_bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int local = 4 * q + i;
            if (local >= row_count) continue;
            const int64_t prow = row_start + local;
#pragma unroll
            for (int f = 0; f < GB; ++f) {
                if (!ok[f]) continue;
                const uint32_t gb = f32_to_bf16_rne(alpha * acc[f][i]);
                const uint32_t ub = f32_to_bf16_rne(alpha_up * acc[f + GB][i]);
                if (p.gu_tap) {
                    uint16_t* t = p.gu_tap + prow * 2 * p.I + col0 + 16 * f + c;
                    t[0] = (uint16_t)gb;
                    t[p.I] = (uint16_t)ub;
                }
                const uint32_t a = silu_mul_bf16(bf16_to_f32(gb), bf16_to_f32(ub));
                amax_bits = max(amax_bits, a & 0x7FFFu);
                p.out_bf16[prow * p.I + col0 + 16 * f + c] = (uint16_t)a;
            }
        }
        __shared__ uint32_t wred[NW];
        amax_bits = wave_max_u32(amax_bits);
        if (lane == 0) wred[wave] = amax_bits;
        __syncthreads();
        if (tid == 0) {
            uint32_t m = wred[0];
            for (int w = 1; w < NW; ++w) m = max(m, wred[w]);
            atomicMax(p.amax_slot, m << 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int local = 4 * q + i;
            if (local >= row_count) continue;
            const int64_t prow = row_start + local;
#pragma unroll
            for (int f = 0; f < NB; ++f)
                if (ok[f]) p.out_f32[prow * N + col0 + 16 * f + c] = alpha * acc[f][i];
        }
    }
}

template <int MODE>
hipError_t launch_skinny_mode(const GemmParams& p, hipStream_t s) {
    const int64_t grid = p.max_tiles * skinny_slabs(MODE, p.I, p.N);
    if (grid <= 0) return hipSuccess;
    const int64_t lds = skinny_lds_bytes(p.K);
    if (lds > kSkinnyMaxLds) return hipErrorInvalidValue;
    static std::atomic<int> lds_set[kMaxDevices];
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&skinny_kernel<MODE>), (int)lds, lds_set);
    if (e != hipSuccess) return e;
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
