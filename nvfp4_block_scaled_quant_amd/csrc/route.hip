// Token-to-expert permutation and the routing-weighted combine (gfx950).
//
// The pages name the permutation (slots, slot_token) and the final
// routing-weighted scatter (NVFP4 MegaMoE Debug Log, "Pipeline Trace" and
// "NVFP4 MoE Pipeline") without defining them. The reading implemented here: one slot per
// (token t, choice j), s = t * topk + j, whose expert id is in [0, E); slots
// are sorted by expert, stably by slot index, so every expert's rows form one
// contiguous range of the "sorted row" order the grouped GEMMs walk; slots with
// other ids are skipped. The combine is y[t] = sum over j, in j order, of
// topk_weights[t][j] times the L2 row of slot (t, j), float32, then one bf16
// rounding.
//
// Routing is a few microseconds of integer work and produces the whole tile
// list on the device, so the host never waits for counts. A small batch is
// routed by one 1024-thread work-group; a large one in chunks of 4,096 slots,
// one work-group each, after a pre-pass that counts every chunk's expert ids
// (each routing work-group then knows the global counts and where its chunk's
// rows of every expert start, and scatters its chunk stably). Further
// work-groups of the same launch quantize the layer input, saving launches:
// for a small batch each takes the amax of the whole input itself, for a
// large one the pre-pass's partial maxima.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kWaves = kRouteThreads / 64;
constexpr int kIdBatches = 16;     // batches of 64 ids a lane holds at once
constexpr int kPreThreads = 256;   // threads of the pre-pass work-groups

// The pre-pass of a large layer input: work-groups [0, n_amax) reduce the
// amax of x (n bf16 values, n % 8 == 0) to one partial maximum each (bf16
// magnitude bits, partial[b]); work-groups from n_amax on count the expert ids
// of one chunk of C slots each (wg_counts[g][e], ids outside [0, E) not
// counted). Partials instead of one atomic slot: the readers take the maximum
// of at most kRouteMaxPartials (1,024) words, and nothing needs zeroing
// first. (At the prefill shape 1,024 work-groups instead of 256 took the
// routing stage from 44.5 to 42.8 us: more loads in flight.)
__global__ __launch_bounds__(kPreThreads) void route_prepass_kernel(
    const uint16_t* __restrict__ x, int64_t n, int n_amax, uint32_t* __restrict__ partial,
    const int32_t* __restrict__ ids, int64_t S, int E, int64_t C, int32_t* __restrict__ wg_counts) {
    __shared__ uint32_t red[kPreThreads / 64];
    extern __shared__ int32_t hist[];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < n_amax) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x);
        const int64_t nvec = n / 8, stride = (int64_t)n_amax * kPreThreads;
        uint32_t m = 0;
        for (int64_t i0 = (int64_t)blockIdx.x * kPreThreads + tid; i0 < nvec; i0 += 4 * stride) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + u * stride;
                v[u] = i < nvec ? p[i] : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) m = max(m, max(v[u][c] & 0x7FFFu, (v[u][c] >> 16) & 0x7FFFu));
        }
        m = wave_max_u32(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
        return;
    }
    const int64_t g = blockIdx.x - n_amax;
    for (int e = tid; e < E; e += kPreThreads) hist[e] = 0;
    __syncthreads();
    const int64_t lo = g * C, hi = min(S, lo + C);
    // all of a thread's ids are loaded before any is counted
    constexpr int kPer = 16;
    int idr[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t sl = lo + (int64_t)u * kPreThreads + tid;
        idr[u] = sl < hi ? ids[sl] : -1;
    }
    for (int64_t b = lo + kPer * kPreThreads; ; b += kPer * kPreThreads) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (idr[u] >= 0 && idr[u] < E) atomicAdd(&hist[idr[u]], 1);
        if (b >= hi) break;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t sl = b + (int64_t)u * kPreThreads + tid;
            idr[u] = sl < hi ? ids[sl] : -1;
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPreThreads) wg_counts[g * E + e] = hist[e];
}

// Dynamic LDS: cnt[E], off[E+1], base[E], wcnt[kWaves][E]
//
// Routing work-groups 0 .. G-1, each over the slots [g C, (g+1) C): with
// wg_counts (the pre-pass's chunk counts) every one of them derives the
// global per-expert counts and its own chunk's base per expert; without
// (G = 1, C = S) the single work-group counts everything itself. Work-group 0
// writes counts, offsets and the tile list. Work-groups G.. quantize x.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int BM, int nbits, int64_t C, int G,
    const int32_t* __restrict__ wg_counts, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row, Tile* __restrict__ tiles,
    int32_t* __restrict__ num_tiles, uint32_t* __restrict__ zero_slots, int n_zero, SmallQuant xq) {
    if ((int)blockIdx.x >= G) {
        // quantization work-groups: the global scale is static, or comes from
        // the pre-pass's partial maxima, or (a small activation: a few
        // hundred KB at most, from L2) every work-group reduces the amax of all
        // of x itself; then each quantizes its share of the 16-element blocks
        __shared__ uint32_t wmax[kWaves];
        const int tid = threadIdx.x;
        const int qb = blockIdx.x - G;
        QuantScales qs;
        if (xq.gs_in) {
            qs = scales_from_gs(*xq.gs_in);
        } else {
            uint32_t m = 0;
            if (xq.amax_partials) {
                for (int i = tid; i < xq.n_partials; i += kRouteThreads) m = max(m, xq.amax_partials[i]);
            } else {
                const int64_t n = xq.M * xq.K;
                const u32x4* v = reinterpret_cast<const u32x4*>(xq.x);
                for (int64_t i = tid; i < n / 8; i += kRouteThreads) {
                    const u32x4 w = v[i];
#pragma unroll
                    for (int c = 0; c < 4; ++c) m = max(m, max(w[c] & 0x7FFFu, (w[c] >> 16) & 0x7FFFu));
                }
            }
            m = wave_max_u32(m);
            if ((tid & 63) == 0) wmax[tid >> 6] = m;
            __syncthreads();
            m = wmax[0];
            for (int w = 1; w < kWaves; ++w) m = max(m, wmax[w]);
            qs = make_scales(__uint_as_float(m << 16));
        }
        if (qb == 0 && tid == 0) *xq.gs = qs.gs;
        const int64_t groups = xq.K / 16;
        for (int64_t b = (int64_t)qb * kRouteThreads + tid; b < xq.M * groups;
             b += (int64_t)(gridDim.x - G) * kRouteThreads)
            quantize_row_block(xq.x, b, groups, qs, xq.q, xq.ldq, xq.sf, xq.ldsf,
                               reinterpret_cast<uint8_t*>(xq.h));
        return;
    }
    extern __shared__ int32_t lds[];
    int32_t* cnt = lds;                              // global count per expert
    int32_t* off = cnt + E;                          // global first sorted row per expert
    int32_t* gbase = off + E + 1;                    // this chunk's first row per expert, past off
    int32_t* wcnt = gbase + E;                       // [kWaves][E]: counts, then running positions
    __shared__ int32_t tile_base[kMaxExperts + 1];   // first tile of each expert
    __shared__ int32_t part_pos[kMaxExperts];        // list position of a short partial tile, or -1

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x;
    const int64_t c_lo = (int64_t)g * C, c_hi = min(S, c_lo + C);
    // wave w owns the contiguous slot range [s_lo, s_hi) of this chunk: the
    // sorted order is stable because the chunks and the waves' ranges are in
    // slot order and each wave scatters its own range in order
    const int64_t per = (c_hi - c_lo + kWaves - 1) / kWaves;
    const int64_t s_lo = min(c_hi, c_lo + (int64_t)wave * per), s_hi = min(c_hi, s_lo + per);
    if (g == 0)
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
    // chunk counts and each wave's exclusive base within an expert; global
    // counts and this chunk's base among the chunks
    for (int e = tid; e < E; e += kRouteThreads) {
        int acc = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = acc;
            acc += c;
        }
        if (wg_counts) {
            int before = 0, total = 0;
            for (int h = 0; h < G; ++h) {
                const int c = wg_counts[(int64_t)h * E + e];
                before += (h < g) ? c : 0;
                total += c;
            }
            cnt[e] = total;
            gbase[e] = before;
        } else {
            cnt[e] = acc;
            gbase[e] = 0;
        }
    }
    __syncthreads();

    // exclusive scans of counts and of tiles per expert: wave 0, 64 experts
    // at a time, shuffle-based inclusive scans within the wave. The tile list
    // holds the experts in order, each with its full BM-row tiles and then its
    // partial one, except partial tiles of at most BM / 2 rows, which go to
    // the end of the list (in expert order). So every round of GEMM
    // work-groups mixes full and partial (shorter) tiles, and the rounds
    // drift apart: the work-groups do not all store their results and load
    // their next tiles at the same moment (2-3% faster on both grouped GEMMs
    // at the prefill shape than all full tiles first, one long round of equal
    // tiles after another), while the shortest tiles make the last round
    // short (3% faster on a skewed routing whose partial tiles are mostly of
    // one or two row blocks).
    if (wave == 0) {
        int acc = 0, tacc = 0, sacc = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = (e < E) ? cnt[e] : 0;
            const int r = c % BM;
            const bool short_part = r > 0 && r <= BM / 2;     // partial tile of at most half the rows
            const int nt = (c + BM - 1) / BM - (short_part ? 1 : 0);
            const int ns = short_part ? 1 : 0;
            int ic = c, jt = nt, js = ns;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int uc = __shfl_up(ic, d), ut = __shfl_up(jt, d), us = __shfl_up(js, d);
                if (lane >= d) { ic += uc; jt += ut; js += us; }
            }
            if (e < E) {
                off[e] = acc + ic - c;
                tile_base[e] = tacc + jt - nt;
                part_pos[e] = short_part ? sacc + js - 1 : -1;   // rank among short partials, for now
            }
            acc += __shfl(ic, 63);
            tacc += __shfl(jt, 63);
            sacc += __shfl(js, 63);
        }
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            if (e < E && part_pos[e] >= 0) part_pos[e] += tacc;   // after all other tiles
        }
        if (lane == 0) {
            off[E] = acc;
            tile_base[E] = tacc;
            if (g == 0) *num_tiles = tacc + sacc;
        }
    }
    __syncthreads();
    if (g == 0) {
        for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = off[e];
        for (int e = tid; e < E; e += kRouteThreads) {
            counts[e] = cnt[e];
            const int nt = (cnt[e] + BM - 1) / BM;
            for (int i = 0; i < nt; ++i) {
                Tile t;
                t.expert = e;
                t.row_start = off[e] + i * BM;
                t.row_count = min(BM, cnt[e] - i * BM);
                t.pad = 0;
                if (i == nt - 1 && part_pos[e] >= 0) tiles[part_pos[e]] = t;
                else tiles[tile_base[e] + i] = t;
            }
        }
    }

    // stable scatter, wave by wave with no further barrier: 64 slots at a time,
    // a slot's position is its expert's start + this chunk's base + this
    // wave's base + the slots of the same expert before it (earlier batches:
    // the running count in LDS; this batch: lanes below it with the same id,
    // matched bit by bit)
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
            const int pos = off[e] + gbase[e] + run[e] + rank;
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

int64_t route_chunk(int64_t S) {
    const int64_t c = (S + kRouteMaxChunks - 1) / kRouteMaxChunks;
    return c <= kRouteChunk ? kRouteChunk : (c + 1023) / 1024 * 1024;
}

int route_amax_partials(int64_t n) {
    const int64_t b = (n / 8 + kPreThreads - 1) / kPreThreads;
    return (int)(b < kRouteMaxPartials ? b : kRouteMaxPartials);
}

hipError_t launch_route_prepass(const uint16_t* x, int64_t n, uint32_t* partial, const int32_t* ids,
                                int64_t S, int E, int32_t* wg_counts, hipStream_t s) {
    const int n_amax = x ? route_amax_partials(n) : 0;
    const int64_t C = route_chunk(S);
    const int64_t G = (S > kRouteChunk) ? (S + C - 1) / C : 0;
    if (n_amax + G == 0) return hipSuccess;
    route_prepass_kernel<<<(unsigned)(n_amax + G), kPreThreads, sizeof(int32_t) * E, s>>>(
        x, n, n_amax, partial, ids, S, E, C, wg_counts);
    return hipGetLastError();
}


hipError_t launch_route(const int32_t* ids, int64_t S, int topk, int E, int BM, const int32_t* wg_counts,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row, Tile* tiles,
                        int32_t* num_tiles, uint32_t* zero_slots, int n_zero, const SmallQuant* xq,
                        hipStream_t s) {
    (void)topk;
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const size_t lds = sizeof(int32_t) * ((size_t)E * (3 + kWaves) + 1);
    const SmallQuant none = {};
    // one routing work-group per chunk when the pre-pass counted the chunks,
    // else one for everything; then the quantization of the activation, one
    // 16-element block per thread
    const int64_t C = (S > kRouteChunk) ? route_chunk(S) : (S > 0 ? S : 1);
    const int G = (S > kRouteChunk) ? (int)((S + C - 1) / C) : 1;
    const int64_t qgroups = xq ? (xq->M * (xq->K / 16) + kRouteThreads - 1) / kRouteThreads : 0;
    route_kernel<<<(unsigned)(G + qgroups), kRouteThreads, lds, s>>>(
        ids, S, E, BM, nbits, C, G, (S > kRouteChunk) ? wg_counts : nullptr, counts, offsets, sorted_slot,
        slot_row, tiles, num_tiles, zero_slots, n_zero, xq ? *xq : none);
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
