// api.cpp -- the C ABI of libqerl (declared in include/qerl.h): argument
// validation on the host, then dispatch to the HIP launchers.  Nothing is
// enqueued when validation fails.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/qerl.h"
#include "qerl_internal.h"

namespace {

thread_local char g_last_error[512] = "";

qerl_status fail(qerl_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
qerl_status fail(qerl_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

qerl_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return QERL_OK;
    return fail(QERL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// QERL_DEBUG set (and not "0"): every GEMM call first checks its launch plan's
// workspace use against the size query on the host (decode_plan_check and
// the prefill plan's check) and fails with QERL_ERR_WORKSPACE instead of
// launching a plan that would address past it.
bool debug_checks() {
    static const bool on = [] {
        const char *v = getenv("QERL_DEBUG");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

// Largest element count a single tensor may have (keeps 64-bit index math far
// from overflow and every grid dimension in range).
constexpr int64_t kMaxElems = (int64_t)1 << 40;

}  // namespace

extern "C" {

const char *qerl_status_string(qerl_status s) {
    switch (s) {
        case QERL_OK: return "ok";
        case QERL_ERR_NULL: return "a required pointer is NULL";
        case QERL_ERR_SHAPE: return "a size is out of range";
        case QERL_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
        case QERL_ERR_ARG: return "a scalar argument is out of range";
        case QERL_ERR_WORKSPACE: return "workspace missing or too small";
        case QERL_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *qerl_last_error(void) { return g_last_error; }

const char *qerl_last_hip_error(void) { return g_last_error; }

size_t qerl_nvfp4_quantize_workspace_size(int64_t n, int64_t k) {
    return qerl::quantize_workspace_bytes(n, k);
}

qerl_status qerl_nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                  int64_t n, int64_t k, void *out_bf16, int64_t ldo, void *stream) {
    g_last_error[0] = '\0';
    if (!packed || !scales || !tensor_scale || !out_bf16)
        return fail(QERL_ERR_NULL, "nvfp4_dequantize: packed, scales, tensor_scale and out are required");
    if (n < 1 || k < 16 || k % 16 != 0 || ldo < k || ldo > kMaxElems || n > kMaxElems / ldo)
        return fail(QERL_ERR_SHAPE, "nvfp4_dequantize: need n >= 1, k >= 16, k %% 16 == 0, ldo >= k "
                    "(got n=%lld k=%lld ldo=%lld)", (long long)n, (long long)k, (long long)ldo);
    if (((uintptr_t)packed & 7u) || !aligned16(out_bf16) || ldo % 8 != 0 || ((uintptr_t)tensor_scale & 3u))
        return fail(QERL_ERR_ALIGN, "nvfp4_dequantize: packed must be 8-byte aligned, out 16-byte aligned with "
                    "ldo %% 8 == 0");
    return hip_status(qerl::launch_nvfp4_dequantize(packed, scales, tensor_scale, n, k,
                                                    static_cast<uint16_t *>(out_bf16), ldo,
                                                    static_cast<hipStream_t>(stream)),
                      "nvfp4_dequantize launch");
}

static qerl_status quantize_common(const char *what, const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                   uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                   const float *tensor_scale_in, uint32_t flags, void *workspace,
                                   size_t workspace_bytes, void *stream, bool stochastic, uint64_t seed);

qerl_status qerl_nvfp4_quantize(const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                const float *tensor_scale_in, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return quantize_common("nvfp4_quantize", w_bf16, n, k, ldw, packed, scales, tensor_scale, tensor_scale_in,
                           flags, workspace, workspace_bytes, stream, false, 0);
}

qerl_status qerl_nvfp4_quantize_stochastic(const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                           uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                           const float *tensor_scale_in, uint32_t flags, uint64_t seed,
                                           void *workspace, size_t workspace_bytes, void *stream) {
    return quantize_common("nvfp4_quantize_stochastic", w_bf16, n, k, ldw, packed, scales, tensor_scale,
                           tensor_scale_in, flags, workspace, workspace_bytes, stream, true, seed);
}

qerl_status qerl_mxfp4_quantize(const void *w_bf16, int64_t n, int64_t k, int64_t ldw, uint8_t *packed,
                                uint8_t *scales, void *stream) {
    g_last_error[0] = '\0';
    if (!w_bf16 || !packed || !scales) return fail(QERL_ERR_NULL, "mxfp4_quantize: w, packed and scales are required");
    if (n < 1 || k < 32 || k % 32 != 0 || ldw < k || n > kMaxElems / k || ldw > kMaxElems)
        return fail(QERL_ERR_SHAPE, "mxfp4_quantize: need n >= 1, k >= 32, k %% 32 == 0, ldw >= k "
                    "(got n=%lld k=%lld ldw=%lld)", (long long)n, (long long)k, (long long)ldw);
    if (!aligned16(w_bf16) || !aligned16(packed) || ldw % 8 != 0)
        return fail(QERL_ERR_ALIGN, "mxfp4_quantize: w and packed must be 16-byte aligned and ldw %% 8 == 0");
    return hip_status(qerl::launch_mxfp4_quantize(static_cast<const uint16_t *>(w_bf16), n, k, ldw, packed, scales,
                                                  static_cast<hipStream_t>(stream)),
                      "mxfp4_quantize launch");
}

static qerl_status quantize_common(const char *what, const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                   uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                   const float *tensor_scale_in, uint32_t flags, void *workspace,
                                   size_t workspace_bytes, void *stream, bool stochastic, uint64_t seed) {
    g_last_error[0] = '\0';
    if (!w_bf16 || !packed || !scales || !tensor_scale)
        return fail(QERL_ERR_NULL, "%s: w, packed, scales and tensor_scale are required", what);
    if (n < 1 || k < 16 || k % 16 != 0 || ldw < k || n > kMaxElems / k || ldw > kMaxElems)
        return fail(QERL_ERR_SHAPE, "%s: need n >= 1, k >= 16, k %% 16 == 0, ldw >= k "
                    "(got n=%lld k=%lld ldw=%lld)", what, (long long)n, (long long)k, (long long)ldw);
    if (!aligned16(w_bf16) || !aligned16(packed) || !aligned16(scales) || ldw % 8 != 0 ||
        ((uintptr_t)tensor_scale & 3u) || ((uintptr_t)tensor_scale_in & 3u))
        return fail(QERL_ERR_ALIGN, "%s: pointers must be 16-byte aligned and ldw %% 8 == 0", what);
    if (flags & ~1u) return fail(QERL_ERR_ARG, "%s: unknown flag bits 0x%x", what, flags);
    if (!tensor_scale_in && (!workspace || workspace_bytes < qerl::quantize_workspace_bytes(n, k)))
        return fail(QERL_ERR_WORKSPACE, "%s: workspace of %zu bytes needed",
                    what, qerl::quantize_workspace_bytes(n, k));
    if (workspace && !aligned16(workspace))
        return fail(QERL_ERR_ALIGN, "%s: workspace must be 16-byte aligned", what);
    return hip_status(qerl::launch_nvfp4_quantize(static_cast<const uint16_t *>(w_bf16), n, k, ldw,
                                                  packed, scales, tensor_scale, tensor_scale_in,
                                                  flags, workspace, static_cast<hipStream_t>(stream),
                                                  stochastic, seed),
                      "nvfp4_quantize launch");
}

size_t qerl_w4a16_lora_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t r) {
    return qerl::gemm_workspace_bytes(m, n, k, r);
}

}  // extern "C"

namespace {

// Validation shared by the single and multi-segment GEMM calls; fills *a.
qerl_status check_gemm(const char *what, const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                       const uint8_t *packed, const uint8_t *scales, const float *tensor_scale, int64_t n,
                       const void *lora_a_bf16, const void *lora_b_bf16, int32_t r, float lora_scale,
                       void *y_bf16, int64_t ldy, qerl::GemmArgs *a) {
    if (!x_bf16 || !packed || !scales || !tensor_scale || !y_bf16)
        return fail(QERL_ERR_NULL, "%s: x, packed, scales, tensor_scale and y are required", what);
    if (r < 0 || r > QERL_MAX_LORA_RANK)
        return fail(QERL_ERR_ARG, "%s: LoRA rank %d outside [0, %d]", what, r, QERL_MAX_LORA_RANK);
    if (r > 0 && (!lora_a_bf16 || !lora_b_bf16))
        return fail(QERL_ERR_NULL, "%s: lora_a and lora_b are required when r > 0", what);
    if (!isfinite(lora_scale)) return fail(QERL_ERR_ARG, "%s: lora_scale must be finite", what);
    if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || ldx < k || ldy < n || m > kMaxElems / k ||
        n > kMaxElems / k || m > kMaxElems / ldy || ldx > kMaxElems || m > ((int64_t)1 << 24) ||
        n > ((int64_t)1 << 28))
        return fail(QERL_ERR_SHAPE, "%s: need m, n >= 1, k >= 16, k %% 16 == 0, ldx >= k, "
                    "ldy >= n (got m=%lld n=%lld k=%lld ldx=%lld ldy=%lld)", what, (long long)m,
                    (long long)n, (long long)k, (long long)ldx, (long long)ldy);
    if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(scales) || ((uintptr_t)y_bf16 & 1u) ||
        ((uintptr_t)tensor_scale & 3u) || ldx % 8 != 0 ||
        (r > 0 && (!aligned16(lora_a_bf16) || !aligned16(lora_b_bf16))))
        return fail(QERL_ERR_ALIGN, "%s: x, packed, scales, lora_a, lora_b must be 16-byte "
                    "aligned, y 2-byte aligned, ldx %% 8 == 0", what);
    a->x = static_cast<const uint16_t *>(x_bf16);
    a->m = m;
    a->k = k;
    a->ldx = ldx;
    a->packed = packed;
    a->scales = scales;
    a->tensor_scale = tensor_scale;
    a->n = n;
    a->lora_a = static_cast<const uint16_t *>(lora_a_bf16);
    a->lora_b = static_cast<const uint16_t *>(lora_b_bf16);
    a->r = r;
    a->lora_scale = lora_scale;
    a->y = static_cast<uint16_t *>(y_bf16);
    a->ldy = ldy;
    a->workspace = nullptr;
    return QERL_OK;
}

static_assert(QERL_MAX_SEGMENTS == 4, "the header's segment limit is the launcher's");

}  // namespace

extern "C" {

qerl_status qerl_w4a16_lora_gemm(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                 const uint8_t *packed, const uint8_t *scales,
                                 const float *tensor_scale, int64_t n,
                                 const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                 float lora_scale, void *y_bf16, int64_t ldy,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    qerl::GemmArgs a;
    const qerl_status st = check_gemm("w4a16_lora_gemm", x_bf16, m, k, ldx, packed, scales, tensor_scale, n,
                                      lora_a_bf16, lora_b_bf16, r, lora_scale, y_bf16, ldy, &a);
    if (st != QERL_OK) return st;
    const size_t need = qerl::gemm_workspace_bytes(m, n, k, r);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm: workspace of %zu bytes needed", need);
    if (workspace && !aligned16(workspace))
        return fail(QERL_ERR_ALIGN, "w4a16_lora_gemm: workspace must be 16-byte aligned");
    a.workspace = workspace;
    if (debug_checks()) {
        char msg[200];
        if (qerl::gemm_plan_check(m, n, k, r, (int64_t)need, msg, sizeof msg))
            return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm: plan check: %s", msg);
    }
    return hip_status(qerl::launch_w4a16_lora_gemm(a, static_cast<hipStream_t>(stream)),
                      "w4a16_lora_gemm launch");
}

qerl_status qerl_w4a16_lora_gemm_noalloc(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                         const uint8_t *packed, const uint8_t *scales,
                                         const float *tensor_scale, int64_t n,
                                         const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                         float lora_scale, void *y_bf16, int64_t ldy, void *stream) {
    g_last_error[0] = '\0';
    qerl::GemmArgs a;
    const qerl_status st = check_gemm("w4a16_lora_gemm_noalloc", x_bf16, m, k, ldx, packed, scales, tensor_scale,
                                      n, lora_a_bf16, lora_b_bf16, r, lora_scale, y_bf16, ldy, &a);
    if (st != QERL_OK) return st;
    const size_t need = qerl::gemm_workspace_bytes(m, n, k, r);
    if (need > QERL_NOALLOC_SCRATCH_BYTES)
        return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm_noalloc: m=%lld n=%lld k=%lld r=%d needs %zu bytes of "
                    "scratch, above the static scratch of %zu bytes (use qerl_w4a16_lora_gemm with a workspace)",
                    (long long)m, (long long)n, (long long)k, r, need, (size_t)QERL_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const qerl_status sst = hip_status(qerl::noalloc_scratch(&ws), "w4a16_lora_gemm_noalloc: scratch address");
    if (sst != QERL_OK) return sst;
    a.workspace = ws;
    if (debug_checks()) {
        char msg[200];
        if (qerl::gemm_plan_check(m, n, k, r, (int64_t)need, msg, sizeof msg))
            return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm_noalloc: plan check: %s", msg);
    }
    return hip_status(qerl::launch_w4a16_lora_gemm(a, static_cast<hipStream_t>(stream)),
                      "w4a16_lora_gemm_noalloc launch");
}

size_t qerl_w4a16_lora_gemm_multi_workspace_size(int64_t m, int64_t k, const qerl_gemm_segment *segs,
                                                 int32_t nseg) {
    if (!segs || nseg < 1 || nseg > QERL_MAX_SEGMENTS) return 0;
    int64_t n[QERL_MAX_SEGMENTS];
    int r[QERL_MAX_SEGMENTS];
    for (int i = 0; i < nseg; ++i) {
        n[i] = segs[i].n;
        r[i] = segs[i].r;
    }
    return qerl::gemm_multi_workspace_bytes(m, k, n, r, nseg);
}

qerl_status qerl_w4a16_lora_gemm_multi(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                       const qerl_gemm_segment *segs, int32_t nseg, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    if (!segs) return fail(QERL_ERR_NULL, "w4a16_lora_gemm_multi: segs is required");
    if (nseg < 1 || nseg > QERL_MAX_SEGMENTS)
        return fail(QERL_ERR_ARG, "w4a16_lora_gemm_multi: nseg %d outside [1, %d]", nseg, QERL_MAX_SEGMENTS);
    qerl::GemmArgs a[QERL_MAX_SEGMENTS];
    int64_t n[QERL_MAX_SEGMENTS];
    int r[QERL_MAX_SEGMENTS];
    char what[48];
    for (int i = 0; i < nseg; ++i) {
        snprintf(what, sizeof what, "w4a16_lora_gemm_multi segment %d", i);
        const qerl_gemm_segment &g = segs[i];
        const qerl_status st = check_gemm(what, x_bf16, m, k, ldx, g.packed, g.scales, g.tensor_scale, g.n,
                                          g.lora_a_bf16, g.lora_b_bf16, g.r, g.lora_scale, g.y_bf16, g.ldy, &a[i]);
        if (st != QERL_OK) return st;
        n[i] = g.n;
        r[i] = g.r;
    }
    const size_t need = qerl::gemm_multi_workspace_bytes(m, k, n, r, nseg);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm_multi: workspace of %zu bytes needed", need);
    if (workspace && !aligned16(workspace))
        return fail(QERL_ERR_ALIGN, "w4a16_lora_gemm_multi: workspace must be 16-byte aligned");
    for (int i = 0; i < nseg; ++i) a[i].workspace = workspace;
    if (debug_checks()) {
        char msg[200];
        if (qerl::gemm_multi_plan_check(m, k, n, r, nseg, false, msg, sizeof msg))
            return fail(QERL_ERR_WORKSPACE, "w4a16_lora_gemm_multi: plan check: %s", msg);
    }
    return hip_status(qerl::launch_w4a16_lora_gemm_multi(a, nseg, static_cast<hipStream_t>(stream)),
                      "w4a16_lora_gemm_multi launch");
}

size_t qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size(int64_t m, int64_t k, const qerl_gemm_segment *segs,
                                                         int32_t nseg) {
    if (!segs || nseg < 1 || nseg > QERL_MAX_SEGMENTS) return 0;
    int64_t n[QERL_MAX_SEGMENTS];
    int r[QERL_MAX_SEGMENTS];
    for (int i = 0; i < nseg; ++i) {
        n[i] = segs[i].n;
        r[i] = segs[i].r;
    }
    return qerl::norm_gemm_multi_workspace_bytes(m, k, n, r, nseg);
}

qerl_status qerl_rmsnorm_w4a16_lora_gemm_multi(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                               const float *norm_weight, float eps,
                                               const qerl_gemm_segment *segs, int32_t nseg,
                                               void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    if (!segs || !norm_weight) return fail(QERL_ERR_NULL, "rmsnorm_w4a16_lora_gemm_multi: segs and norm_weight are required");
    if (nseg < 1 || nseg > QERL_MAX_SEGMENTS)
        return fail(QERL_ERR_ARG, "rmsnorm_w4a16_lora_gemm_multi: nseg %d outside [1, %d]", nseg, QERL_MAX_SEGMENTS);
    if (!(eps > 0.0f) || !isfinite(eps))
        return fail(QERL_ERR_ARG, "rmsnorm_w4a16_lora_gemm_multi: eps must be positive and finite");
    if (k > QERL_MAX_NORM_WIDTH)
        return fail(QERL_ERR_SHAPE, "rmsnorm_w4a16_lora_gemm_multi: k=%lld above %d", (long long)k, QERL_MAX_NORM_WIDTH);
    if (!aligned16(norm_weight))
        return fail(QERL_ERR_ALIGN, "rmsnorm_w4a16_lora_gemm_multi: norm_weight must be 16-byte aligned");
    qerl::GemmArgs a[QERL_MAX_SEGMENTS];
    int64_t n[QERL_MAX_SEGMENTS];
    int r[QERL_MAX_SEGMENTS];
    char what[56];
    for (int i = 0; i < nseg; ++i) {
        snprintf(what, sizeof what, "rmsnorm_w4a16_lora_gemm_multi segment %d", i);
        const qerl_gemm_segment &g = segs[i];
        const qerl_status st = check_gemm(what, x_bf16, m, k, ldx, g.packed, g.scales, g.tensor_scale, g.n,
                                          g.lora_a_bf16, g.lora_b_bf16, g.r, g.lora_scale, g.y_bf16, g.ldy, &a[i]);
        if (st != QERL_OK) return st;
        n[i] = g.n;
        r[i] = g.r;
    }
    const size_t need = qerl::norm_gemm_multi_workspace_bytes(m, k, n, r, nseg);
    if (!workspace || workspace_bytes < need)
        return fail(QERL_ERR_WORKSPACE, "rmsnorm_w4a16_lora_gemm_multi: workspace of %zu bytes needed", need);
    if (!aligned16(workspace))
        return fail(QERL_ERR_ALIGN, "rmsnorm_w4a16_lora_gemm_multi: workspace must be 16-byte aligned");
    for (int i = 0; i < nseg; ++i) {
        a[i].workspace = workspace;
        a[i].norm_w = norm_weight;
        a[i].norm_eps = eps;
    }
    if (debug_checks()) {
        char msg[200];
        if (qerl::gemm_multi_plan_check(m, k, n, r, nseg, true, msg, sizeof msg))
            return fail(QERL_ERR_WORKSPACE, "rmsnorm_w4a16_lora_gemm_multi: plan check: %s", msg);
    }
    return hip_status(qerl::launch_norm_gemm_multi(a, nseg, static_cast<hipStream_t>(stream)),
                      "rmsnorm_w4a16_lora_gemm_multi launch");
}

qerl_status qerl_aqn_noisy_weight(const float *weight, int64_t h, float sigma, uint64_t seed, uint64_t step,
                                  uint32_t layer_id, float *noisy_weight_out, void *stream) {
    g_last_error[0] = '\0';
    if (!weight || !noisy_weight_out) return fail(QERL_ERR_NULL, "aqn_noisy_weight: weight and noisy_weight_out are required");
    if (h < 1 || h > QERL_MAX_NORM_WIDTH)
        return fail(QERL_ERR_SHAPE, "aqn_noisy_weight: need 1 <= h <= %d (got %lld)", QERL_MAX_NORM_WIDTH, (long long)h);
    if (((uintptr_t)weight & 3u) || ((uintptr_t)noisy_weight_out & 3u))
        return fail(QERL_ERR_ALIGN, "aqn_noisy_weight: pointers must be 4-byte aligned");
    if (!(sigma >= 0.0f) || !isfinite(sigma))
        return fail(QERL_ERR_ARG, "aqn_noisy_weight: sigma must be non-negative and finite");
    qerl::AqnArgs a{};
    a.h = h;
    a.weight = weight;
    a.sigma = sigma;
    a.seed = seed;
    a.step = step;
    a.layer = layer_id;
    a.noisy_out = noisy_weight_out;
    return hip_status(qerl::launch_aqn_noisy_weight(a, static_cast<hipStream_t>(stream)), "aqn_noisy_weight launch");
}

size_t qerl_w4a16_lora_backward_workspace_size(int64_t m, int64_t n, int64_t k, int32_t r) {
    if (m < 1 || n < 1 || k < 1 || r < 0) return 0;
    return qerl::backward_workspace_bytes(m, n, k, r);
}

qerl_status qerl_w4a16_lora_backward(const void *dy_bf16, int64_t m, int64_t n, int64_t ldy,
                                     const void *x_bf16, int64_t k, int64_t ldx,
                                     const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                     const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                     float lora_scale, void *dx_bf16, int64_t lddx, float *da_f32,
                                     float *db_f32, void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    if (!dy_bf16 || !x_bf16 || !packed || !scales || !tensor_scale)
        return fail(QERL_ERR_NULL, "w4a16_lora_backward: dy, x, packed, scales and tensor_scale are required");
    if (r < 0 || r > QERL_MAX_LORA_RANK)
        return fail(QERL_ERR_ARG, "w4a16_lora_backward: LoRA rank %d outside [0, %d]", r, QERL_MAX_LORA_RANK);
    if (r > 0 && (!lora_a_bf16 || !lora_b_bf16))
        return fail(QERL_ERR_NULL, "w4a16_lora_backward: lora_a and lora_b are required when r > 0");
    if (!isfinite(lora_scale)) return fail(QERL_ERR_ARG, "w4a16_lora_backward: lora_scale must be finite");
    if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || ldy < n || ldx < k || (dx_bf16 && lddx < k) ||
        m > kMaxElems / k || m > kMaxElems / ldy || m > kMaxElems / ldx || n > kMaxElems / k ||
        (dx_bf16 && m > kMaxElems / lddx) || m > ((int64_t)1 << 22) * 64)
        return fail(QERL_ERR_SHAPE, "w4a16_lora_backward: need m, n >= 1, k >= 16, k %% 16 == 0, ldy >= n, "
                    "ldx >= k, lddx >= k (got m=%lld n=%lld k=%lld)", (long long)m, (long long)n, (long long)k);
    if (!aligned16(dy_bf16) || !aligned16(x_bf16) || !aligned16(packed) || ldx % 8 != 0 ||
        ((uintptr_t)dx_bf16 & 1u) || ((uintptr_t)tensor_scale & 3u) || ((uintptr_t)da_f32 & 3u) ||
        ((uintptr_t)db_f32 & 3u) || (r > 0 && (!aligned16(lora_a_bf16) || ((uintptr_t)lora_b_bf16 & 1u))))
        return fail(QERL_ERR_ALIGN, "w4a16_lora_backward: dy, x, packed, lora_a must be 16-byte aligned, "
                    "ldx %% 8 == 0");
    const size_t need = qerl::backward_workspace_bytes(m, n, k, r);
    if (!workspace || workspace_bytes < need)
        return fail(QERL_ERR_WORKSPACE, "w4a16_lora_backward: workspace of %zu bytes needed", need);
    if (!aligned16(workspace)) return fail(QERL_ERR_ALIGN, "w4a16_lora_backward: workspace must be 16-byte aligned");
    qerl::BackwardArgs b{};
    b.dy = static_cast<const uint16_t *>(dy_bf16);
    b.x = static_cast<const uint16_t *>(x_bf16);
    b.m = m;
    b.n = n;
    b.k = k;
    b.ldy = ldy;
    b.ldx = ldx;
    b.packed = packed;
    b.scales = scales;
    b.tensor_scale = tensor_scale;
    b.lora_a = static_cast<const uint16_t *>(lora_a_bf16);
    b.lora_b = static_cast<const uint16_t *>(lora_b_bf16);
    b.r = r;
    b.lora_scale = lora_scale;
    b.dx = static_cast<uint16_t *>(dx_bf16);
    b.lddx = lddx;
    b.da = r > 0 ? da_f32 : nullptr;
    b.db = r > 0 ? db_f32 : nullptr;
    b.workspace = workspace;
    return hip_status(qerl::launch_backward(b, static_cast<hipStream_t>(stream)), "w4a16_lora_backward launch");
}

float qerl_aqn_sigma(int32_t stage, int32_t num_stages, float sigma_start, float sigma_end) {
    if (!(sigma_start > 0.0f) || !(sigma_end > 0.0f) || !isfinite(sigma_start) || !isfinite(sigma_end))
        return NAN;
    if (num_stages <= 1) return sigma_start;
    if (stage < 0) stage = 0;
    if (stage > num_stages - 1) stage = num_stages - 1;
    const double ratio = (double)sigma_end / (double)sigma_start;
    return (float)((double)sigma_start * pow(ratio, (double)stage / (double)(num_stages - 1)));
}

qerl_status qerl_aqn_rmsnorm(const void *x_bf16, int64_t m, int64_t h, int64_t ldx,
                             const float *weight, float eps, float sigma,
                             uint64_t seed, uint64_t step, uint32_t layer_id,
                             float *y_f32, void *y_bf16, int64_t ldy,
                             float *noisy_weight_out, void *stream) {
    g_last_error[0] = '\0';
    if (!x_bf16 || !weight) return fail(QERL_ERR_NULL, "aqn_rmsnorm: x and weight are required");
    if (!y_f32 && !y_bf16) return fail(QERL_ERR_NULL, "aqn_rmsnorm: give y_f32, y_bf16 or both");
    if (m < 1 || h < 1 || h > QERL_MAX_NORM_WIDTH || ldx < h || ldy < h || m > kMaxElems / ldx ||
        m > kMaxElems / ldy)
        return fail(QERL_ERR_SHAPE, "aqn_rmsnorm: need m >= 1, 1 <= h <= %d, ldx >= h, ldy >= h "
                    "(got m=%lld h=%lld ldx=%lld ldy=%lld)", QERL_MAX_NORM_WIDTH, (long long)m,
                    (long long)h, (long long)ldx, (long long)ldy);
    if (((uintptr_t)x_bf16 & 1u) || ((uintptr_t)weight & 3u) || ((uintptr_t)y_f32 & 3u) ||
        ((uintptr_t)y_bf16 & 1u) || ((uintptr_t)noisy_weight_out & 3u))
        return fail(QERL_ERR_ALIGN, "aqn_rmsnorm: pointers must be aligned to their element size");
    if (!(eps > 0.0f) || !isfinite(eps)) return fail(QERL_ERR_ARG, "aqn_rmsnorm: eps must be positive and finite");
    if (!(sigma >= 0.0f) || !isfinite(sigma))
        return fail(QERL_ERR_ARG, "aqn_rmsnorm: sigma must be non-negative and finite");
    qerl::AqnArgs a;
    a.x = static_cast<const uint16_t *>(x_bf16);
    a.m = m;
    a.h = h;
    a.ldx = ldx;
    a.weight = weight;
    a.eps = eps;
    a.sigma = sigma;
    a.seed = seed;
    a.step = step;
    a.layer = layer_id;
    a.y_f32 = y_f32;
    a.y_bf16 = static_cast<uint16_t *>(y_bf16);
    a.ldy = ldy;
    a.noisy_out = noisy_weight_out;
    return hip_status(qerl::launch_aqn_rmsnorm(a, static_cast<hipStream_t>(stream)), "aqn_rmsnorm launch");
}

}  // extern "C"
