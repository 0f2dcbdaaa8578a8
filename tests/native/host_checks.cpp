// Host-side checks of libqerl's C++ code, built for the CPU only (no kernel
// is launched) under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_native_sanitize.py:
//  * every launch plan's workspace use against the size query the caller
//    sizes the workspace by (decode_plan_check / gemm_plan_check), for the
//    projections of the Qwen2.5-7B and -32B decoder layers at every decode
//    batch, the rollout and prefill batches, the multi-segment calls with and
//    without the RMSNorm, and a sweep of small and ragged shapes;
//  * the argument checks of every entry point, fed rejected arguments (they
//    return before anything touches a device).
#include <stdint.h>
#include <stdio.h>

#include "../../include/qerl.h"
#include "../../nvfp4_weight_only_quantize_amd/csrc/qerl_internal.h"

static long g_checks = 0, g_bad = 0;

static void plan(int64_t m, int64_t n, int64_t k, int r) {
    char msg[256];
    ++g_checks;
    const size_t size = qerl_w4a16_lora_gemm_workspace_size(m, n, k, r);
    if (qerl::gemm_plan_check(m, n, k, r, (int64_t)size, msg, sizeof msg)) {
        if (g_bad++ < 20) printf("plan: %s\n", msg);
    }
}

static void plan_multi(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg) {
    char msg[256];
    for (int norm = 0; norm < 2; ++norm) {
        if (norm && k > QERL_MAX_NORM_WIDTH) continue;
        ++g_checks;
        if (qerl::gemm_multi_plan_check(m, k, n, r, nseg, norm != 0, msg, sizeof msg)) {
            if (g_bad++ < 20) printf("plan_multi norm=%d: %s\n", norm, msg);
        }
    }
}

static void expect(qerl_status got, qerl_status want, const char *what) {
    ++g_checks;
    if (got != want) {
        if (g_bad++ < 20) printf("status: %s: got %d want %d (%s)\n", what, got, want, qerl_last_error());
    }
}

int main() {
    // projections of one decoder layer (N, K): q, k, v, o, gate, up, down
    const int64_t layers[2][7][2] = {
        {{3584, 3584}, {512, 3584}, {512, 3584}, {3584, 3584}, {18944, 3584}, {18944, 3584}, {3584, 18944}},
        {{5120, 5120}, {1024, 5120}, {1024, 5120}, {5120, 5120}, {27648, 5120}, {27648, 5120}, {5120, 27648}}};
    const int ranks[] = {0, 8, 16, 32, 64, 128};
    const int64_t big_m[] = {65, 100, 128, 129, 192, 200, 256, 257, 300, 1000, 2048, 8192};
    for (const auto &layer : layers) {
        for (const int r : ranks) {
            for (int64_t m = 1; m <= 64; ++m)
                for (const auto &p : layer) plan(m, p[0], p[1], r);
            for (const int64_t m : big_m)
                for (const auto &p : layer) plan(m, p[0], p[1], r);
            // q|k|v and gate|up of one x, fused gate|up as one tensor
            const int64_t qkv[3] = {layer[0][0], layer[1][0], layer[2][0]};
            const int64_t gu[2] = {layer[4][0], layer[5][0]};
            const int rr[4] = {r, r, r, r};
            for (int64_t m = 1; m <= 64; ++m) {
                plan_multi(m, layer[0][1], qkv, rr, 3);
                plan_multi(m, layer[4][1], gu, rr, 2);
            }
            for (const int64_t m : big_m) {
                plan_multi(m, layer[0][1], qkv, rr, 3);
                plan_multi(m, layer[4][1], gu, rr, 2);
                plan(m, 2 * layer[4][0], layer[4][1], 2 * r > 128 ? 128 : 2 * r);
            }
        }
    }
    // small and ragged shapes
    const int64_t ns[] = {1, 15, 16, 17, 63, 64, 65, 100, 257, 1000, 4097};
    const int64_t ks[] = {16, 32, 48, 112, 128, 144, 512, 528, 1040, 4112};
    const int64_t ms[] = {1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 129, 700};
    const int rs[] = {0, 1, 5, 16, 33, 128};
    for (const int64_t n : ns)
        for (const int64_t k : ks)
            for (const int64_t m : ms)
                for (const int r : rs) plan(m, n, k, r);
    for (const int64_t k : ks)
        for (const int64_t m : ms)
            for (const int r : rs) {
                const int64_t n3[4] = {17, 1000, 64, 4097};
                const int r4[4] = {r, r == 0 ? 5 : 0, r, 1};
                plan_multi(m, k, n3, r4, 4);
                plan_multi(m, k, n3, r4, 1);
            }

    // rejected arguments: nothing is touched, so fake (aligned) addresses do
    void *const F = reinterpret_cast<void *>((uintptr_t)1 << 20);
    const uint8_t *FB = static_cast<const uint8_t *>(F);
    const float *FF = static_cast<const float *>(F);
    uint8_t *FW = static_cast<uint8_t *>(F);
    float *FO = static_cast<float *>(F);
    void *const MIS = reinterpret_cast<void *>(((uintptr_t)1 << 20) + 2);
    expect(qerl_nvfp4_quantize(nullptr, 4, 32, 32, FW, FW, FO, nullptr, 0, F, 4096, nullptr), QERL_ERR_NULL, "quantize null");
    expect(qerl_nvfp4_quantize(F, 4, 24, 24, FW, FW, FO, nullptr, 0, F, 4096, nullptr), QERL_ERR_SHAPE, "quantize k%16");
    expect(qerl_nvfp4_quantize(F, 0, 32, 32, FW, FW, FO, nullptr, 0, F, 4096, nullptr), QERL_ERR_SHAPE, "quantize n=0");
    expect(qerl_nvfp4_quantize(MIS, 4, 32, 32, FW, FW, FO, nullptr, 0, F, 4096, nullptr), QERL_ERR_ALIGN, "quantize align");
    expect(qerl_nvfp4_quantize(F, 4, 32, 32, FW, FW, FO, nullptr, 7, F, 4096, nullptr), QERL_ERR_ARG, "quantize flags");
    expect(qerl_nvfp4_quantize(F, 4, 32, 32, FW, FW, FO, nullptr, 0, nullptr, 0, nullptr), QERL_ERR_WORKSPACE, "quantize ws");
    expect(qerl_nvfp4_quantize(F, (int64_t)1 << 40, (int64_t)1 << 40, (int64_t)1 << 40, FW, FW, FO, nullptr, 0, F,
                               4096, nullptr), QERL_ERR_SHAPE, "quantize huge");
    expect(qerl_mxfp4_quantize(F, 4, 48, 48, FW, FW, nullptr), QERL_ERR_SHAPE, "mxfp4 k%32");
    expect(qerl_nvfp4_dequantize(FB, FB, FF, 4, 24, F, 24, nullptr), QERL_ERR_SHAPE, "dequant k%16");
    expect(qerl_nvfp4_dequantize(nullptr, FB, FF, 4, 32, F, 32, nullptr), QERL_ERR_NULL, "dequant null");
    expect(qerl_w4a16_lora_gemm(F, 1, 16, 16, FB, FB, FF, 1, nullptr, nullptr, 4, 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_NULL, "gemm lora null");
    expect(qerl_w4a16_lora_gemm(F, 1, 16, 16, FB, FB, FF, 1, F, F, 129, 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_ARG, "gemm rank");
    expect(qerl_w4a16_lora_gemm(F, 1, 16, 16, FB, FB, FF, 1, F, F, 4, 1.0f / 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_ARG, "gemm lora_scale inf");
    expect(qerl_w4a16_lora_gemm(F, 1, 20, 20, FB, FB, FF, 1, nullptr, nullptr, 0, 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_SHAPE, "gemm k%16");
    expect(qerl_w4a16_lora_gemm(F, 1, 16, 12, FB, FB, FF, 1, nullptr, nullptr, 0, 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_SHAPE, "gemm ldx<k");
    expect(qerl_w4a16_lora_gemm(MIS, 1, 16, 16, FB, FB, FF, 1, nullptr, nullptr, 0, 0.0f, F, 1, F, 1 << 20, nullptr),
           QERL_ERR_ALIGN, "gemm align");
    expect(qerl_w4a16_lora_gemm(F, 64, 3584, 3584, FB, FB, FF, 18944, F, F, 32, 2.0f, F, 18944, F, 16, nullptr),
           QERL_ERR_WORKSPACE, "gemm ws");
    expect(qerl_w4a16_lora_gemm_noalloc(F, 128, 5120, 5120, FB, FB, FF, 27648, F, F, 32, 2.0f, F, 27648, nullptr),
           QERL_ERR_WORKSPACE, "noalloc above scratch");
    qerl_gemm_segment seg{FB, FB, FF, 64, F, F, 8, 2.0f, F, 64};
    expect(qerl_w4a16_lora_gemm_multi(F, 8, 64, 64, &seg, 0, F, 1 << 20, nullptr), QERL_ERR_ARG, "multi nseg 0");
    expect(qerl_w4a16_lora_gemm_multi(F, 8, 64, 64, &seg, 5, F, 1 << 20, nullptr), QERL_ERR_ARG, "multi nseg 5");
    expect(qerl_w4a16_lora_gemm_multi(F, 8, 64, 64, nullptr, 1, F, 1 << 20, nullptr), QERL_ERR_NULL, "multi null");
    expect(qerl_rmsnorm_w4a16_lora_gemm_multi(F, 8, 64, 64, FF, 0.0f, &seg, 1, F, 1 << 20, nullptr), QERL_ERR_ARG,
           "norm eps");
    expect(qerl_rmsnorm_w4a16_lora_gemm_multi(F, 8, 32768, 32768, FF, 1e-6f, &seg, 1, F, 1 << 20, nullptr),
           QERL_ERR_SHAPE, "norm width");
    expect(qerl_w4a16_lora_backward(nullptr, 4, 64, 64, F, 64, 64, FB, FB, FF, F, F, 8, 2.0f, F, 64, FO, FO, F,
                                    1 << 20, nullptr),
           QERL_ERR_NULL, "backward null");
    expect(qerl_aqn_rmsnorm(F, 4, 64, 64, FF, -1.0f, 0.0f, 0, 0, 0, FO, nullptr, 64, nullptr, nullptr),
           QERL_ERR_ARG, "aqn eps");
    expect(qerl_aqn_rmsnorm(F, 4, 20000, 20000, FF, 1e-6f, 0.0f, 0, 0, 0, FO, nullptr, 20000, nullptr, nullptr),
           QERL_ERR_SHAPE, "aqn width");
    for (long s = 0; s < 8; ++s) (void)qerl_status_string((qerl_status)s);
    printf("%ld checks, %ld failed\n", g_checks, g_bad);
    return g_bad == 0 ? 0 : 1;
}
