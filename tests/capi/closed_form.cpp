// The expert layer driven through the C ABI alone (no Python, no torch): the
// constant layer whose output is known by hand (the case of
// tests/test_oracle_closed_form.py), built from bf16 weights with the
// library's own weight quantizer and prepack, then run through
// nvfp4_moe_forward and nvfp4_moe_forward_noalloc.
//
//   x = 3.0 (T x H); expert 0: gate 0.5, up 0.25, w2 2^-10; expert 1: gate
//   0.5, up 0.125, w2 2^-10; every token to (expert 0, expert 1) with
//   routing weights (0.25, 0.75)  =>  y = 5760 everywhere (bf16 0x45B4).
//
// Exit status 0 when every output element is 0x45B4 on both entry points,
// 1 on a wrong value, 2 on an API or HIP error (each printed).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "nvfp4moe.h"

namespace {

constexpr int64_t T = 4, H = 256, I = 128, E = 2, K = 2;

#define HIP_OK(expr)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "%s: %s\n", #expr, hipGetErrorString(e_));               \
            std::exit(2);                                                                 \
        }                                                                                 \
    } while (0)

#define API_OK(expr)                                                                      \
    do {                                                                                  \
        int s_ = (expr);                                                                  \
        if (s_ != NVFP4_OK) {                                                             \
            std::fprintf(stderr, "%s: %s\n", #expr, nvfp4_strerror(s_));                 \
            std::exit(2);                                                                 \
        }                                                                                 \
    } while (0)

template <typename T_>
T_* upload(const std::vector<T_>& h) {
    T_* d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T_)));
    HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T_), hipMemcpyHostToDevice));
    return d;
}

void* device_bytes(size_t n) {
    void* d = nullptr;
    HIP_OK(hipMalloc(&d, n ? n : 1));
    return d;
}

// bf16 bit patterns of the constants (all exact)
constexpr uint16_t kThree = 0x4040, kHalf = 0x3F00, kQuarter = 0x3E80, kEighth = 0x3E00;
constexpr uint16_t kTwoPowMinus10 = 0x3A80, kExpected = 0x45B4;   // 2^-10, 5760

// canonical quantized weights (E, Kd/2, N) + (E, Kd/16, N) + alpha (E) of bf16 w (E, Kd, N), then packed
struct Packed {
    uint8_t* q;
    uint8_t* sf;
    float* alpha;
};

Packed quantize_and_pack(const std::vector<uint16_t>& w, int64_t Kd, int64_t N, hipStream_t s) {
    uint16_t* dw = upload(w);
    uint8_t* q = static_cast<uint8_t*>(device_bytes(E * Kd / 2 * N));
    uint8_t* sf = static_cast<uint8_t*>(device_bytes(E * Kd / 16 * N));
    Packed p;
    p.alpha = static_cast<float*>(device_bytes(E * sizeof(float)));
    const size_t nws = nvfp4_quantize_weights_workspace(E, Kd, N);
    void* ws = device_bytes(nws);
    API_OK(nvfp4_quantize_weights(dw, E, Kd, N, q, sf, p.alpha, ws, nws, s));
    int64_t ldq = 0, ldsf = 0, ldwsf = 0;
    API_OK(nvfp4_operand_pitches(Kd, &ldq, &ldsf, &ldwsf));
    p.q = static_cast<uint8_t*>(device_bytes(E * N * ldq));
    p.sf = static_cast<uint8_t*>(device_bytes(E * N * ldwsf));
    API_OK(nvfp4_prepack_weights(q, sf, E, Kd, N, p.q, p.sf, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipFree(dw));
    HIP_OK(hipFree(q));
    HIP_OK(hipFree(sf));
    HIP_OK(hipFree(ws));
    return p;
}

int check(const char* what, const uint16_t* dy) {
    std::vector<uint16_t> y(T * H);
    HIP_OK(hipMemcpy(y.data(), dy, y.size() * sizeof(uint16_t), hipMemcpyDeviceToHost));
    int bad = 0;
    for (size_t i = 0; i < y.size(); ++i)
        if (y[i] != kExpected) {
            if (bad < 4) std::fprintf(stderr, "%s: y[%zu] = 0x%04x, expected 0x%04x\n", what, i, y[i], kExpected);
            ++bad;
        }
    std::printf("%s: %d of %zu elements differ from 5760\n", what, bad, y.size());
    return bad;
}

}  // namespace

int main() {
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    std::printf("library version %d.%d\n", nvfp4_version() >> 16, nvfp4_version() & 0xFFFF);

    // w13[e] (H, 2I): gate columns [0, I), up columns [I, 2I); w2[e] (I, H)
    std::vector<uint16_t> w13(E * H * 2 * I), w2(E * I * H, kTwoPowMinus10);
    for (int64_t e = 0; e < E; ++e)
        for (int64_t k = 0; k < H; ++k)
            for (int64_t n = 0; n < 2 * I; ++n)
                w13[(e * H + k) * 2 * I + n] = n < I ? kHalf : (e == 0 ? kQuarter : kEighth);
    const Packed p13 = quantize_and_pack(w13, H, 2 * I, s);
    const Packed p2 = quantize_and_pack(w2, I, H, s);

    const std::vector<uint16_t> x(T * H, kThree);
    std::vector<int32_t> ids(T * K);
    std::vector<float> wts(T * K);
    for (int64_t t = 0; t < T; ++t) {
        ids[t * K] = 0, ids[t * K + 1] = 1;
        wts[t * K] = 0.25f, wts[t * K + 1] = 0.75f;
    }
    uint16_t* dx = upload(x);
    int32_t* dids = upload(ids);
    float* dwts = upload(wts);
    uint16_t* dy = static_cast<uint16_t*>(device_bytes(T * H * sizeof(uint16_t)));

    const size_t nws = nvfp4_moe_workspace(T, H, I, E, K);
    void* ws = device_bytes(nws);
    API_OK(nvfp4_moe_forward(dx, dids, dwts, p13.q, p13.sf, p13.alpha, p2.q, p2.sf, p2.alpha, T, H, I, E, K,
                             dy, ws, nws, s, nullptr));
    HIP_OK(hipStreamSynchronize(s));
    int bad = check("nvfp4_moe_forward", dy);

    HIP_OK(hipMemset(dy, 0, T * H * sizeof(uint16_t)));
    API_OK(nvfp4_moe_forward_noalloc(dx, dids, dwts, p13.q, p13.sf, p13.alpha, p2.q, p2.sf, p2.alpha, T, H, I,
                                     E, K, dy, s, nullptr, nullptr));
    HIP_OK(hipStreamSynchronize(s));
    bad += check("nvfp4_moe_forward_noalloc", dy);

    for (void* d : {static_cast<void*>(p13.q), static_cast<void*>(p13.sf), static_cast<void*>(p13.alpha),
                    static_cast<void*>(p2.q), static_cast<void*>(p2.sf), static_cast<void*>(p2.alpha),
                    static_cast<void*>(dx), static_cast<void*>(dids), static_cast<void*>(dwts),
                    static_cast<void*>(dy), ws})
        HIP_OK(hipFree(d));
    HIP_OK(hipStreamDestroy(s));
    return bad ? 1 : 0;
}
