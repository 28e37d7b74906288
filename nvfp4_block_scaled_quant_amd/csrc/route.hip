// Token-to-expert permutation and the routing-weighted combine (gfx950).
//
// The pages name the permutation ("slots", "slot_token") and the final
// "scatter with routing weights" (DEBUG_LOG, "Pipeline Trace" and "NVFP4 MoE
// Pipeline") without defining them. The reading implemented here: one slot per
// (token t, choice j), s = t * topk + j, whose expert id is in [0, E); slots
// are sorted by expert, stably by slot index, so every expert's rows form one
// contiguous range of the "sorted row" order the grouped GEMMs walk; slots with
// other ids are skipped. The combine is y[t] = sum over j, in j order, of
// topk_weights[t][j] times the L2 row of slot (t, j), float32, then one bf16
// rounding.
//
// Routing runs in a single 1024-thread work-group: it is a few microseconds of
// integer work on at most a few tens of thousands of slots and it produces the
// whole tile list on the device, so the host never waits for counts. For a
// small batch further work-groups of the same launch quantize the layer input
// (each takes the amax of the whole input, then does its share of the block
// pass), saving two launches.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kWaves = kRouteThreads / 64;
constexpr int kIdBatches = 16;     // batches of 64 ids a lane holds at once

// Dynamic LDS: cnt[E], off[E+1], run[E], wcnt[kWaves][E]
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int BM, int nbits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_row, Tile* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    uint32_t* __restrict__ zero_slots, int n_zero, SmallQuant xq) {
    if (blockIdx.x > 0) {
        // quantization work-groups: the global scale is static, or comes from
        // an amax computed before this launch, or (a small activation: a few
        // hundred KB at most, from L2) every work-group reduces the amax of all
        // of x itself; then each quantizes its share of the 16-element blocks
        __shared__ uint32_t wmax[kWaves];
        const int tid = threadIdx.x;
        QuantScales qs;
        if (xq.gs_in) {
            qs = scales_from_gs(*xq.gs_in);
        } else if (xq.amax_in) {
            qs = make_scales(__uint_as_float(*xq.amax_in));
        } else {
            const int64_t n = xq.M * xq.K;
            const u32x4* v = reinterpret_cast<const u32x4*>(xq.x);
            uint32_t m = 0;
            for (int64_t i = tid; i < n / 8; i += kRouteThreads) {
                const u32x4 w = v[i];
#pragma unroll
                for (int c = 0; c < 4; ++c) m = max(m, max(w[c] & 0x7FFFu, (w[c] >> 16) & 0x7FFFu));
            }
            m = wave_max_u32(m);
            if ((tid & 63) == 0) wmax[tid >> 6] = m;
            __syncthreads();
            m = wmax[0];
            for (int w = 1; w < kWaves; ++w) m = max(m, wmax[w]);
            qs = make_scales(__uint_as_float(m << 16));
        }
        if (blockIdx.x == 1 && tid == 0) *xq.gs = qs.gs;
        const int64_t groups = xq.K / 16;
        for (int64_t b = (int64_t)(blockIdx.x - 1) * kRouteThreads + tid; b < xq.M * groups;
             b += (int64_t)(gridDim.x - 1) * kRouteThreads)
            quantize_row_block(xq.x, b, groups, qs, xq.q, xq.ldq, xq.sf, xq.ldsf,
                               reinterpret_cast<uint8_t*>(xq.h));
        return;
    }
    extern __shared__ int32_t lds[];
    int32_t* cnt = lds;
    int32_t* off = cnt + E;
    int32_t* wcnt = off + E + 1;                     // [kWaves][E]: counts, then running positions
    __shared__ int32_t tile_base[kMaxExperts + 1];   // first full tile of each expert
    __shared__ int32_t part_base[kMaxExperts + 1];   // its partial tile (after all full ones)

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // wave w owns the contiguous slot range [s_lo, s_hi): the sorted order is
    // stable because the waves' ranges are in slot order and each wave scatters
    // its own range in order
    const int64_t per = (S + kWaves - 1) / kWaves;
    const int64_t s_lo = min(S, (int64_t)wave * per), s_hi = min(S, s_lo + per);
    for (int i = tid; i < n_zero; i += kRouteThreads) zero_slots[i] = 0u;
    for (int i = tid; i < kWaves * E; i += kRouteThreads) wcnt[i] = 0;
    __syncthreads();

    // ids in super-chunks of kIdBatches batches of 64 slots, all loads of a
    // super-chunk in flight together (a loop of dependent loads would pay the
    // memory latency once per batch)
    int ids_r[kIdBatches];
    auto load_ids = [&](int64_t c0) {
#pragma unroll
        for (int u = 0; u < kIdBatches; ++u) {
            const int64_t s = c0 + 64 * u + lane;
            ids_r[u] = (s < s_hi) ? ids[s] : -1;
        }
    };
    // per-wave histograms
    for (int64_t c0 = s_lo; c0 < s_hi; c0 += 64 * kIdBatches) {
        load_ids(c0);
#pragma unroll
        for (int u = 0; u < kIdBatches; ++u) {
            const int e = ids_r[u];
            if (e >= 0 && e < E) atomicAdd(&wcnt[wave * E + e], 1);
        }
    }
    __syncthreads();
    // totals, and each wave's exclusive base within an expert
    for (int e = tid; e < E; e += kRouteThreads) {
        int acc = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = acc;
            acc += c;
        }
        cnt[e] = acc;
    }
    __syncthreads();

    // exclusive scans of counts, of full tiles and of partial tiles per expert:
    // wave 0, 64 experts at a time, shuffle-based inclusive scans within the
    // wave. The tile list holds every expert's full BM-row tiles first and the
    // partial tiles (fewer rows, less work) after them: the grouped GEMM's
    // last round of work-groups then consists of the short ones.
    if (wave == 0) {
        int acc = 0, facc = 0, pacc = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = (e < E) ? cnt[e] : 0;
            const int f = c / BM, q = (c % BM) ? 1 : 0;
            int ic = c, jf = f, jq = q;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int uc = __shfl_up(ic, d), uf = __shfl_up(jf, d), uq = __shfl_up(jq, d);
                if (lane >= d) { ic += uc; jf += uf; jq += uq; }
            }
            if (e < E) {
                off[e] = acc + ic - c;
                tile_base[e] = facc + jf - f;
                part_base[e] = pacc + jq - q;
            }
            acc += __shfl(ic, 63);
            facc += __shfl(jf, 63);
            pacc += __shfl(jq, 63);
        }
        if (lane == 0) {
            off[E] = acc;
            tile_base[E] = facc;         // number of full tiles
            part_base[E] = pacc;
            *num_tiles = facc + pacc;
        }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = off[e];
    for (int e = tid; e < E; e += kRouteThreads) {
        counts[e] = cnt[e];
        const int nf = cnt[e] / BM;
        for (int i = 0; i <= nf; ++i) {
            Tile t;
            t.expert = e;
            t.row_start = off[e] + i * BM;
            t.row_count = min(BM, cnt[e] - i * BM);
            t.pad = 0;
            if (i < nf) tiles[tile_base[e] + i] = t;
            else if (t.row_count > 0) tiles[tile_base[E] + part_base[e]] = t;
        }
    }

    // stable scatter, wave by wave with no further barrier: 64 slots at a time,
    // a slot's position is its expert's start + this wave's base + the slots of
    // the same expert before it (earlier batches: the running count in LDS;
    // this batch: lanes below it with the same id, matched bit by bit)
    int32_t* run = wcnt + wave * E;
    for (int64_t c00 = s_lo; c00 < s_hi; c00 += 64 * kIdBatches) {
      load_ids(c00);
#pragma unroll
      for (int u = 0; u < kIdBatches; ++u) {
        const int64_t c0 = c00 + 64 * u;
        if (c0 >= s_hi) break;
        const int64_t s = c0 + lane;
        const int e = ids_r[u];
        const bool valid = (e >= 0 && e < E);
        uint64_t match = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const uint64_t bl = __ballot(bit);
            match &= bit ? bl : ~bl;
        }
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(match & below);
        const int total = __popcll(match);
        if (valid) {
            const int pos = off[e] + run[e] + rank;
            sorted_slot[pos] = (int32_t)s;
            slot_row[s] = pos;
        } else if (s < s_hi) {
            slot_row[s] = -1;
        }
        // every lane has read run[e] above (in-order wave); the last lane of
        // each id advances it for the next batch
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == total - 1) run[e] += total;
        __builtin_amdgcn_wave_barrier();
      }
    }
}

// One thread per 4 consecutive columns of one token; `chunks` blocks of 256
// threads (1,024 columns) per token.
__device__ __forceinline__ void combine_block(const float* __restrict__ o2,
                                              const int32_t* __restrict__ slot_row,
                                              const float* __restrict__ weights, int topk, int64_t H,
                                              int chunks, uint16_t* __restrict__ y, int64_t blk) {
    // one thread: 4 columns of one token (one 16-byte load per slot; with 8
    // columns per thread the same gather measured 211 instead of 171 us at
    // the prefill shape)
    const int64_t t = blk / chunks;
    const int64_t c0 = ((blk % chunks) * 256 + threadIdx.x) * 4;
    if (c0 >= H) return;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // slots in batches of 8: all their loads are issued before the sums, which
    // still run in slot order
    for (int j0 = 0; j0 < topk; j0 += 8) {
        int32_t row[8];
        float w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool in = j0 + u < topk;
            row[u] = in ? slot_row[t * topk + j0 + u] : -1;
            w[u] = in ? weights[t * topk + j0 + u] : 0.0f;
        }
        float4_t a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a[u] = (float4_t){0.f, 0.f, 0.f, 0.f};
            // each L2 row is read once: non-temporal loads
            if (row[u] >= 0)
                a[u] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(o2 + (int64_t)row[u] * H + c0));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (row[u] < 0) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = acc[i] + w[u] * a[u][i];
        }
    }
    u32x2 out;
    out[0] = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    out[1] = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(y + t * H + c0) = out;
}

// (token, 1024-column chunk) blocks, grid-strided
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o2,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ weights, int topk,
                                                      int64_t H, int chunks, int64_t nblk,
                                                      uint16_t* __restrict__ y) {
    for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x)
        combine_block(o2, slot_row, weights, topk, H, chunks, y, b);
}

// Top-k router with renormalized softmax weights, one wave per token: each
// lane holds the logits of experts lane, lane + 64, ... (up to 512 experts);
// k rounds of a wave-wide arg-max over the experts not yet taken, the larger
// value winning and the smaller expert index among equal values; then
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected logits, l_0
// the largest, the sum taken in selection order. float32 throughout.
constexpr int kTopkWaves = 4;
constexpr int kTopkPerLane = kMaxExperts / 64;

__global__ __launch_bounds__(64 * kTopkWaves) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
    if (t >= T) return;                       // uniform per wave
    const float* row = logits + t * E;
    float v[kTopkPerLane];
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) {
        const int e = 64 * i + lane;
        v[i] = e < E ? row[e] : 0.0f;
    }
    uint32_t avail = 0;                       // bit i: expert 64 i + lane is a candidate
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i)
        if (64 * i + lane < E) avail |= 1u << i;
    int32_t sel_id[kTopkPerLane];
    float sel_e[kTopkPerLane];
    float top = 0.0f, sum = 0.0f;
    for (int j = 0; j < k; ++j) {
        // this lane's best candidate (entries are in ascending expert order,
        // so a strict comparison keeps the smallest index among equal values)
        float bv = 0.0f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < kTopkPerLane; ++i)
            if (((avail >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) {
                bv = v[i];
                bi = 64 * i + lane;
            }
        // wave arg-max: larger value, then smaller index; lanes without a
        // candidate carry index INT_MAX and lose to every real one
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            const bool other = (oi != 0x7FFFFFFF) &&
                               (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
            if (other) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
        if (j == 0) top = bv;
        const float ej = expf(bv - top);
        sum += ej;
#pragma unroll
        for (int i = 0; i < kTopkPerLane; ++i)
            if (j == 64 * i + lane) {
                sel_id[i] = bi;
                sel_e[i] = ej;
            }
    }
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) {
        const int j = 64 * i + lane;
        if (j < k) {
            ids[t * k + j] = sel_id[i];
            weights[t * k + j] = sel_e[i] / sum;
        }
    }
}

}  // namespace

hipError_t launch_route(const int32_t* ids, int64_t S, int topk, int E, int BM, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row, Tile* tiles,
                        int32_t* num_tiles, uint32_t* zero_slots, int n_zero, const SmallQuant* xq,
                        hipStream_t s) {
    (void)topk;
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const size_t lds = sizeof(int32_t) * ((size_t)E * (2 + kWaves) + 1);
    const SmallQuant none = {};
    // work-groups 1.. quantize the activation, one 16-element block per thread
    const int64_t qgroups = xq ? (xq->M * (xq->K / 16) + kRouteThreads - 1) / kRouteThreads : 0;
    route_kernel<<<(unsigned)(1 + qgroups), kRouteThreads, lds, s>>>(ids, S, E, BM, nbits, counts, offsets, sorted_slot,
                                                        slot_row, tiles, num_tiles, zero_slots, n_zero,
                                                        xq ? *xq : none);
    return hipGetLastError();
}

hipError_t launch_combine(const float* o2, const int32_t* slot_row, const float* weights,
                          int64_t T, int topk, int64_t H, uint16_t* y, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int chunks = (int)((H / 4 + 255) / 256);
    const int64_t nblk = T * chunks;
    const int64_t grid = nblk < (1 << 22) ? nblk : (1 << 22);
    combine_kernel<<<(unsigned)grid, 256, 0, s>>>(o2, slot_row, weights, topk, H, chunks, nblk, y);
    return hipGetLastError();
}

}  // namespace nvfp4

namespace nvfp4 {

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* ids,
                             float* weights, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t grid = (T + kTopkWaves - 1) / kTopkWaves;
    route_topk_kernel<<<(unsigned)grid, 64 * kTopkWaves, 0, s>>>(logits, T, E, k, ids, weights);
    return hipGetLastError();
}

}  // namespace nvfp4
