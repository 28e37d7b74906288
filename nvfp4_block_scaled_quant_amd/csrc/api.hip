// C ABI of the NVFP4 expert-layer library: argument validation, workspace
// carving and the launch sequence. Declarations and contracts: include/nvfp4moe.h.
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/nvfp4moe.h"
#include "launch.hpp"

using namespace nvfp4;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// 0 = not checked, 1 = gfx950, 2 = other
std::atomic<int> g_device_ok[kMaxDevices];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NVFP4_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_EDEVICE;
    int st = g_device_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_EHIP;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? NVFP4_OK : NVFP4_EDEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

#define NVFP4_TRY(expr)                      \
    do {                                     \
        hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) return NVFP4_EHIP; \
    } while (0)

struct MoeLayout {
    size_t off[NVFP4_MOE_WS_NUM];
    size_t amax;        // 2 x uint32: x amax, act amax
    size_t partials;    // kRouteMaxPartials x uint32: partial maxima of x
    size_t wg_counts;   // kRouteMaxChunks x E int32: routing chunk counts
    size_t tiles;
    size_t num_tiles;
    size_t total;
    int64_t max_tiles;
};

// Upper bound of sum_e ceil(count_e / BM): floor(S / BM) + number of non-empty experts.
int64_t moe_max_tiles(int64_t S, int64_t E, int64_t BM) {
    if (S <= 0) return 0;
    return S / BM + (E < S ? E : S);
}

// Small batches (at most 16 slots per expert on average) stream the weights
// with 16-row tiles; larger ones use the 256 x 256 MFMA tiles. The streaming
// kernel stages its A rows whole in LDS, so it is also limited to reduction
// lengths (H for L1, I for L2) whose rows fit; beyond that the tiled GEMM,
// whose LDS use does not depend on K, takes small batches too.
bool moe_use_skinny(int64_t S, int64_t E, int64_t H, int64_t I) {
    return S <= (int64_t)kSkinnyBM * E && skinny_lds_bytes(H) <= kSkinnyMaxLds &&
           skinny_lds_bytes(I) <= kSkinnyMaxLds;
}

MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
    MoeLayout L;
    const int64_t S = T * topk;
    // quantized GEMM operands use the padded row pitches pitch_q / pitch_sf;
    // their f16 forms (pitch_h) exist only for the tiled GEMMs
    const bool tiled = !moe_use_skinny(S, E, H, I);
    const size_t sizes[NVFP4_MOE_WS_NUM] = {
        (size_t)(T * pitch_q(H)), (size_t)(T * pitch_sf(H)), 4, 4,
        (size_t)(4 * E),      (size_t)(4 * (E + 1)), (size_t)(4 * S), (size_t)(4 * S),
        (size_t)(2 * S * I),  (size_t)(S * pitch_q(I)), (size_t)(S * pitch_sf(I)), (size_t)(4 * S * H),
        tiled ? (size_t)(T * pitch_h(H)) : 0, tiled ? (size_t)(S * pitch_h(I)) : 0};
    size_t cur = 0;
    for (int i = 0; i < NVFP4_MOE_WS_NUM; ++i) {
        L.off[i] = cur;
        cur = align_up(cur + sizes[i]);
    }
    L.amax = cur;
    cur = align_up(cur + 8);
    L.partials = cur;
    cur = align_up(cur + 4 * kRouteMaxPartials);
    L.wg_counts = cur;
    cur = align_up(cur + 4 * (size_t)kRouteMaxChunks * (size_t)E);
    L.max_tiles = moe_max_tiles(S, E, kSkinnyBM);     // the larger of the two tile lists
    L.tiles = cur;
    cur = align_up(cur + sizeof(Tile) * (size_t)(L.max_tiles > 0 ? L.max_tiles : 1));
    L.num_tiles = cur;
    cur = align_up(cur + 4);
    L.total = cur;
    return L;
}

bool moe_shape_ok(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return false;
    if (H % 16 || I % 16 || topk > E || E > kMaxExperts) return false;
    if (T > (int64_t)1 << 24 || H > (int64_t)1 << 20 || I > (int64_t)1 << 20) return false;
    if (T * topk >= ((int64_t)1 << 31)) return false;
    // 32-bit buffer offsets: every GEMM operand stays below 2 GiB
    if (2 * I * pitch_q(H) >= 0x7FFFFFFF || H * pitch_q(I) >= 0x7FFFFFFF ||
        T * pitch_h(H) >= 0x7FFFFFFF || T * topk * pitch_h(I) >= 0x7FFFFFFF)
        return false;
    return true;
}

// ---------------------------------------------------------------------------
// The allocation-free variant of the layer keeps its workspace in a file-scope
// device array: every GPU the library runs on holds one copy of it (from the
// code object's load until the process ends). On the host `scratch` only
// names the symbol; its device address, which differs per device, comes from
// hipGetSymbolAddress with that device current, taken once per device on the
// entry point's first call there and kept.
static __device__ __align__(256) uint8_t scratch[NVFP4_MOE_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NVFP4_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_EDEVICE;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return NVFP4_EHIP;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_strerror(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_EINVAL: return "invalid argument (null or misaligned pointer, negative size)";
        case NVFP4_ESHAPE: return "unsupported shape (K dimensions must be multiples of 16, 1 <= topk <= E <= 512)";
        case NVFP4_EWORKSPACE: return "workspace missing, misaligned (256 bytes) or too small";
        case NVFP4_EHIP: return "HIP runtime error or kernel launch failure";
        case NVFP4_EDEVICE: return "current device is not an MI355X-class gfx950 GPU";
        case NVFP4_ESCRATCH:
            return "the layer's workspace exceeds the allocation-free entry point's static scratch "
                   "(NVFP4_MOE_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int nvfp4_version(void) { return (5 << 16) | 0; }

// ---------------------------------------------------------------------------
size_t nvfp4_quantize_workspace(int64_t M, int64_t K) {
    (void)M;
    (void)K;
    return kAlign;
}

int nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* sf, float* gs,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (M < 0 || K <= 0) return NVFP4_EINVAL;
    if (K % 16) return NVFP4_ESHAPE;
    if (!gs || (M > 0 && (!x || !q || !sf))) return NVFP4_EINVAL;
    if (M > 0 && (!aligned(x, 16) || !aligned(q, 8))) return NVFP4_EINVAL;
    if (!aligned(gs, 4)) return NVFP4_EINVAL;
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < nvfp4_quantize_workspace(M, K))
        return NVFP4_EWORKSPACE;
    int dv = check_device();
    if (dv) return dv;
    uint32_t* slot = static_cast<uint32_t*>(workspace);
    NVFP4_TRY(launch_zero_u32(slot, 1, stream));
    NVFP4_TRY(launch_amax_bf16(x, M * K, slot, stream));
    NVFP4_TRY(launch_quant_rows(x, M, K, nullptr, slot, q, K / 2, sf, K / 16, gs, stream));
    return NVFP4_OK;
}

int nvfp4_quantize_static(const uint16_t* x, int64_t M, int64_t K, const float* gs, uint8_t* q,
                          uint8_t* sf, hipStream_t stream) {
    if (M < 0 || K <= 0) return NVFP4_EINVAL;
    if (K % 16) return NVFP4_ESHAPE;
    if (M == 0) return NVFP4_OK;
    if (!x || !gs || !q || !sf) return NVFP4_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(gs, 4)) return NVFP4_EINVAL;
    int dv = check_device();
    if (dv) return dv;
    NVFP4_TRY(launch_quant_rows(x, M, K, nullptr, nullptr, q, K / 2, sf, K / 16, nullptr, stream, gs));
    return NVFP4_OK;
}

// ---------------------------------------------------------------------------
size_t nvfp4_quantize_weights_workspace(int64_t E, int64_t K, int64_t N) {
    (void)K;
    (void)N;
    return align_up((size_t)(E > 0 ? E : 1) * 4);
}

size_t nvfp4_quantize_weights_parts_workspace(int64_t E, int64_t K, int64_t N, int64_t parts) {
    (void)K;
    (void)N;
    return align_up((size_t)(E > 0 ? E : 1) * (size_t)(parts > 0 ? parts : 1) * 4);
}

int nvfp4_quantize_weights(const uint16_t* w, int64_t E, int64_t K, int64_t N, uint8_t* q,
                           uint8_t* sf, float* alpha, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (E < 0 || K <= 0 || N <= 0) return NVFP4_EINVAL;
    if (K % 16 || E > 65535) return NVFP4_ESHAPE;
    if (E == 0) return NVFP4_OK;
    if (!w || !q || !sf || !alpha) return NVFP4_EINVAL;
    if (!aligned(w, 16) || !aligned(alpha, 4)) return NVFP4_EINVAL;
    if (!workspace || !aligned(workspace, kAlign) ||
        workspace_bytes < nvfp4_quantize_weights_workspace(E, K, N))
        return NVFP4_EWORKSPACE;
    int dv = check_device();
    if (dv) return dv;
    uint32_t* slots = static_cast<uint32_t*>(workspace);
    NVFP4_TRY(launch_zero_u32(slots, (int)E, stream));
    NVFP4_TRY(launch_amax_bf16_batched(w, E, K * N, slots, stream));
    NVFP4_TRY(launch_quant_cols(w, E, K, N, 1, slots, q, sf, alpha, stream));
    return NVFP4_OK;
}

int nvfp4_quantize_weights_parts(const uint16_t* w, int64_t E, int64_t K, int64_t N, int64_t parts,
                                 uint8_t* q, uint8_t* sf, float* alpha, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (E < 0 || K <= 0 || N <= 0 || parts <= 0) return NVFP4_EINVAL;
    if (K % 16 || E * parts > 65535 || parts > 16 || N % parts || (N / parts) % 8) return NVFP4_ESHAPE;
    if (E == 0) return NVFP4_OK;
    if (!w || !q || !sf || !alpha) return NVFP4_EINVAL;
    if (!aligned(w, 16) || !aligned(alpha, 4)) return NVFP4_EINVAL;
    if (!workspace || !aligned(workspace, kAlign) ||
        workspace_bytes < nvfp4_quantize_weights_parts_workspace(E, K, N, parts))
        return NVFP4_EWORKSPACE;
    int dv = check_device();
    if (dv) return dv;
    uint32_t* slots = static_cast<uint32_t*>(workspace);
    NVFP4_TRY(launch_zero_u32(slots, (int)(E * parts), stream));
    NVFP4_TRY(launch_amax_cols(w, E, K, N, (int)parts, slots, stream));
    NVFP4_TRY(launch_quant_cols(w, E, K, N, (int)parts, slots, q, sf, alpha, stream));
    return NVFP4_OK;
}

// ---------------------------------------------------------------------------
int nvfp4_operand_pitches(int64_t K, int64_t* ldq, int64_t* ldsf, int64_t* ldwsf) {
    if (K <= 0) return NVFP4_EINVAL;
    if (K % 16) return NVFP4_ESHAPE;
    if (!ldq || !ldsf || !ldwsf) return NVFP4_EINVAL;
    *ldq = pitch_q(K);
    *ldsf = pitch_sf(K);
    *ldwsf = pitch_wsf(K);
    return NVFP4_OK;
}

int nvfp4_prepack_weights(const uint8_t* w, const uint8_t* w_sf, int64_t E, int64_t K, int64_t N,
                          uint8_t* w_t, uint8_t* w_sf_t, hipStream_t stream) {
    if (E < 0 || K <= 0 || N <= 0) return NVFP4_EINVAL;
    if (K % 16 || N % 16 || E > 65535) return NVFP4_ESHAPE;
    if (E == 0) return NVFP4_OK;
    if (!w || !w_sf || !w_t || !w_sf_t) return NVFP4_EINVAL;
    if (!aligned(w_t, 16) || !aligned(w_sf_t, 8)) return NVFP4_EINVAL;
    int dv = check_device();
    if (dv) return dv;
    NVFP4_TRY(launch_pack_weights(w, E, K / 2, N, w_t, pitch_q(K), false, stream));
    NVFP4_TRY(launch_pack_weights(w_sf, E, K / 16, N, w_sf_t, pitch_wsf(K), true, stream));
    return NVFP4_OK;
}

// ---------------------------------------------------------------------------
// A's f16 form, then (when K is cut into chunks) the chunks' partial sums
size_t gemm_ws_partial_offset(int64_t M, int64_t K) { return align_up((size_t)((M > 0 ? M : 1) * pitch_h(K))); }

size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0 || K % 16) return 0;
    const int ks = dense_ksplit(M, N, K);
    return gemm_ws_partial_offset(M, K) + (ks > 1 ? align_up((size_t)ks * (size_t)M * (size_t)N * 4) : 0);
}

int nvfp4_gemm(const uint8_t* aq, const uint8_t* asf, const float* a_gs, const uint8_t* bq,
               const uint8_t* bsf, const float* b_alpha, int64_t M, int64_t N, int64_t K,
               uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (M < 0 || N <= 0 || K <= 0) return NVFP4_EINVAL;
    if (K % 16 || N % 16) return NVFP4_ESHAPE;
    if (M * pitch_h(K) >= 0x7FFFFFFF || N * pitch_q(K) >= 0x7FFFFFFF) return NVFP4_ESHAPE;
    if (M == 0) return NVFP4_OK;
    if (!aq || !asf || !a_gs || !bq || !bsf || !b_alpha || !out) return NVFP4_EINVAL;
    if (!aligned(aq, 8) || !aligned(bq, 16) || !aligned(bsf, 8) || !aligned(out, 2) || !aligned(a_gs, 4) ||
        !aligned(b_alpha, 4))
        return NVFP4_EINVAL;
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < nvfp4_gemm_workspace(M, N, K))
        return NVFP4_EWORKSPACE;
    int dv = check_device();
    if (dv) return dv;
    // the A operand in its exact f16 form, rows padded to whole K steps
    uint16_t* ah = static_cast<uint16_t*>(workspace);
    NVFP4_TRY(launch_dequant_rows_f16(aq, asf, M, K, ah, stream));
    GemmParams p = {};
    p.mode = kGemmDense;
    p.aq = aq;
    p.asf = asf;
    p.ah = ah;
    p.M = M;
    p.a_rows = M;
    p.bq = bq;
    p.bsf = bsf;
    p.N = N;
    p.K = K;
    p.a_gs = a_gs;
    p.b_alpha = b_alpha;
    p.out_bf16 = out;
    // too few tiles to fill the GPU: K in chunks, partial sums, then one reduction
    p.ksplit = dense_ksplit(M, N, K);
    p.partial = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + gemm_ws_partial_offset(M, K));
    NVFP4_TRY(launch_gemm(p, stream));
    if (p.ksplit > 1) NVFP4_TRY(launch_splitk_reduce(p.partial, p.ksplit, M, N, a_gs, b_alpha, out, stream));
    return NVFP4_OK;
}

// ---------------------------------------------------------------------------
size_t nvfp4_moe_workspace(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
    if (!moe_shape_ok(T, H, I, E, topk)) return 0;
    return moe_layout(T, H, I, E, topk).total;
}

int nvfp4_moe_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                               size_t* offsets) {
    if (!offsets) return NVFP4_EINVAL;
    if (!moe_shape_ok(T, H, I, E, topk)) return NVFP4_ESHAPE;
    const MoeLayout L = moe_layout(T, H, I, E, topk);
    for (int i = 0; i < NVFP4_MOE_WS_NUM; ++i) offsets[i] = L.off[i];
    return NVFP4_OK;
}

int nvfp4_moe_forward(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                      const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                      const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha, int64_t T,
                      int64_t H, int64_t I, int64_t E, int64_t topk, uint16_t* y, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* stage_events) {
    return nvfp4_moe_forward_ex(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2, w2_sf,
                                w2_alpha, T, H, I, E, topk, y, workspace, workspace_bytes, stream,
                                stage_events, nullptr);
}

int nvfp4_moe_forward_ex(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                         const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha, int64_t T,
                         int64_t H, int64_t I, int64_t E, int64_t topk, uint16_t* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t* stage_events,
                         const nvfp4_moe_options* options) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return NVFP4_EINVAL;
    const int per_half = options ? options->w13_alpha_per_half : 0;
    const float* x_gs = options ? options->x_global_scale : nullptr;
    uint16_t* gu_tap = options ? options->gate_up_tap : nullptr;
    if (per_half != 0 && per_half != 1) return NVFP4_EINVAL;
    if (options && options->reserved != 0) return NVFP4_EINVAL;
    if (x_gs && !aligned(x_gs, 4)) return NVFP4_EINVAL;
    if (gu_tap && !aligned(gu_tap, 4)) return NVFP4_EINVAL;
    if (!moe_shape_ok(T, H, I, E, topk)) return NVFP4_ESHAPE;
    if (!w13 || !w13_sf || !w13_alpha || !w2 || !w2_sf || !w2_alpha) return NVFP4_EINVAL;
    if (T > 0 && (!x || !topk_ids || !topk_weights || !y)) return NVFP4_EINVAL;
    if (T > 0 && (!aligned(x, 16) || !aligned(y, 16) || !aligned(topk_ids, 4) ||
                  !aligned(topk_weights, 4)))
        return NVFP4_EINVAL;
    if (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13_sf, 8) || !aligned(w2_sf, 8) ||
        !aligned(w13_alpha, 4) || !aligned(w2_alpha, 4))
        return NVFP4_EINVAL;
    const MoeLayout L = moe_layout(T, H, I, E, topk);
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < L.total)
        return NVFP4_EWORKSPACE;
    int dv = check_device();
    if (dv) return dv;
    if (T == 0) return NVFP4_OK;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* xq = ws + L.off[NVFP4_MOE_WS_XQ];
    uint8_t* xsf = ws + L.off[NVFP4_MOE_WS_XSF];
    float* gs1 = reinterpret_cast<float*>(ws + L.off[NVFP4_MOE_WS_GS1]);
    float* gs2 = reinterpret_cast<float*>(ws + L.off[NVFP4_MOE_WS_GS2]);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.off[NVFP4_MOE_WS_COUNTS]);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.off[NVFP4_MOE_WS_OFFSETS]);
    int32_t* sorted_slot = reinterpret_cast<int32_t*>(ws + L.off[NVFP4_MOE_WS_SORTED_SLOT]);
    int32_t* slot_row = reinterpret_cast<int32_t*>(ws + L.off[NVFP4_MOE_WS_SLOT_ROW]);
    uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.off[NVFP4_MOE_WS_ACT]);
    uint8_t* aq = ws + L.off[NVFP4_MOE_WS_AQ];
    uint8_t* asf = ws + L.off[NVFP4_MOE_WS_ASF];
    float* o2 = reinterpret_cast<float*>(ws + L.off[NVFP4_MOE_WS_O2]);
    uint16_t* xh = reinterpret_cast<uint16_t*>(ws + L.off[NVFP4_MOE_WS_XH]);
    uint16_t* ah = reinterpret_cast<uint16_t*>(ws + L.off[NVFP4_MOE_WS_AH]);
    uint32_t* amax = reinterpret_cast<uint32_t*>(ws + L.amax);
    Tile* tiles = reinterpret_cast<Tile*>(ws + L.tiles);
    int32_t* num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
    const int64_t S = T * topk;
    const bool skinny = moe_use_skinny(S, E, H, I);
    const int BM = skinny ? kSkinnyBM : kGemmBM;
    const int64_t max_tiles = moe_max_tiles(S, E, BM);

    auto mark = [&](int i) -> hipError_t {
        return stage_events ? hipEventRecord(stage_events[i], stream) : hipSuccess;
    };

    // 1 + 2. routing tables + tile list, and the quantization of x in further
    // work-groups of the same launch, concurrently with the routing (stage 2
    // is then empty). A larger x (and no static scale) first gets its partial
    // maxima from the pre-pass, which also counts the slots of every routing
    // chunk of a larger batch; a small x is reduced by the quantization
    // work-groups themselves, a small batch counted by its one routing
    // work-group. The routing launch zeroes the act amax slot.
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_ROUTE));
    const bool small_x = T * H <= kSmallQuantMax;
    const bool amax_pass = !small_x && !x_gs;
    uint32_t* partials = reinterpret_cast<uint32_t*>(ws + L.partials);
    int32_t* wg_counts = reinterpret_cast<int32_t*>(ws + L.wg_counts);
    NVFP4_TRY(launch_route_prepass(amax_pass ? x : nullptr, T * H, partials, topk_ids, S, (int)E, wg_counts,
                                   stream));
    const SmallQuant sq = {x,
                           x_gs,
                           amax_pass ? partials : nullptr,
                           amax_pass ? route_amax_partials(T * H) : 0,
                           T,
                           H,
                           xq,
                           pitch_q(H),
                           xsf,
                           pitch_sf(H),
                           gs1,
                           skinny ? nullptr : xh};
    NVFP4_TRY(launch_route(topk_ids, S, (int)topk, (int)E, BM, wg_counts, counts, offsets, sorted_slot,
                           slot_row, tiles, num_tiles, amax + 1, 1, &sq, stream));
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_QUANT_X));
    // 3. L1 grouped GEMM with fused SiLU(gate) * up
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_L1));
    GemmParams p1 = {};
    p1.mode = kGemmL1;
    p1.ksplit = 1;
    p1.aq = xq;
    p1.asf = xsf;
    p1.ah = xh;
    p1.a_rows = T;
    p1.a_gather = sorted_slot;
    p1.topk = (int)topk;
    p1.bq = w13;
    p1.bsf = w13_sf;
    p1.N = 2 * I;
    p1.K = H;
    p1.a_gs = gs1;
    p1.b_alpha = w13_alpha;
    p1.alpha_stride = per_half ? 2 : 1;
    p1.tiles = tiles;
    p1.num_tiles = num_tiles;
    p1.max_tiles = max_tiles;
    p1.out_bf16 = act;
    p1.I = I;
    p1.amax_slot = amax + 1;
    p1.gu_tap = gu_tap;
    NVFP4_TRY(skinny ? launch_skinny(p1, stream) : launch_gemm(p1, stream));
    // 4. requantize act (rows of valid slots only: offsets[E])
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_REQUANT));
    NVFP4_TRY(launch_quant_rows(act, S, I, offsets + E, amax + 1, aq, pitch_q(I), asf, pitch_sf(I), gs2,
                                stream, nullptr, skinny ? nullptr : ah));
    // 5a. L2 grouped GEMM
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_L2));
    GemmParams p2 = {};
    p2.mode = kGemmL2;
    p2.ksplit = 1;
    p2.aq = aq;
    p2.asf = asf;
    p2.ah = ah;
    p2.a_rows = S;
    p2.bq = w2;
    p2.bsf = w2_sf;
    p2.N = H;
    p2.K = I;
    p2.a_gs = gs2;
    p2.b_alpha = w2_alpha;
    p2.tiles = tiles;
    p2.num_tiles = num_tiles;
    p2.max_tiles = max_tiles;
    p2.out_f32 = o2;
    NVFP4_TRY(skinny ? launch_skinny(p2, stream) : launch_gemm(p2, stream));
    // 5b. weighted combine
    NVFP4_TRY(mark(NVFP4_MOE_STAGE_COMBINE));
    NVFP4_TRY(launch_combine(o2, slot_row, topk_weights, T, (int)topk, H, y, stream));
    NVFP4_TRY(mark(NVFP4_MOE_NUM_STAGES));
    return NVFP4_OK;
}

int nvfp4_moe_forward_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                              const uint8_t* w13, const uint8_t* w13_sf, const float* w13_alpha,
                              const uint8_t* w2, const uint8_t* w2_sf, const float* w2_alpha,
                              int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, uint16_t* y,
                              hipStream_t stream, hipEvent_t* stage_events,
                              const nvfp4_moe_options* options) {
    // the shape checks of nvfp4_moe_forward_ex first, so that a bad shape is
    // reported as such and not as a scratch overflow
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return NVFP4_EINVAL;
    if (!moe_shape_ok(T, H, I, E, topk)) return NVFP4_ESHAPE;
    if (moe_layout(T, H, I, E, topk).total > (size_t)NVFP4_MOE_SCRATCH_BYTES) return NVFP4_ESCRATCH;
    int dv = check_device();
    if (dv) return dv;
    void* ws = nullptr;
    const int st = scratch_address(&ws);
    if (st) return st;
    return nvfp4_moe_forward_ex(x, topk_ids, topk_weights, w13, w13_sf, w13_alpha, w2, w2_sf, w2_alpha, T,
                                H, I, E, topk, y, ws, (size_t)NVFP4_MOE_SCRATCH_BYTES, stream,
                                stage_events, options);
}

// ---------------------------------------------------------------------------
int nvfp4_route_topk(const float* logits, int64_t T, int64_t E, int64_t topk, int32_t* topk_ids,
                     float* topk_weights, hipStream_t stream) {
    if (T < 0 || E <= 0 || topk <= 0) return NVFP4_EINVAL;
    if (topk > E || E > kMaxExperts || T >= ((int64_t)1 << 31) / E) return NVFP4_ESHAPE;
    if (T == 0) return NVFP4_OK;
    if (!logits || !topk_ids || !topk_weights) return NVFP4_EINVAL;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4)) return NVFP4_EINVAL;
    int dv = check_device();
    if (dv) return dv;
    return hip_status(launch_route_topk(logits, T, (int)E, (int)topk, topk_ids, topk_weights, stream));
}

}  // extern "C"
