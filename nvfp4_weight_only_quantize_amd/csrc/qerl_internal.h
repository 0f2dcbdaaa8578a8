// qerl_internal.h -- launchers behind the C ABI.  Arguments reaching these
// functions have already been validated by api.cpp (shapes, alignment,
// workspace size), so the launchers only choose a kernel and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qerl {

// ---- quantizer ----
constexpr int kAmaxMaxBlocks = 1024;  // per-workgroup partial maxima kept in the workspace
size_t quantize_workspace_bytes(int64_t n, int64_t k);
// stochastic: stochastic element rounding with stream `seed`
hipError_t launch_nvfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                                 uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                 const float *tensor_scale_in, uint32_t flags, void *workspace,
                                 hipStream_t stream, bool stochastic = false, uint64_t seed = 0);
// BF16 -> MXFP4 (k % 32 == 0): packed [n, k/2], E8M0 scales [n, k/32]; no workspace
hipError_t launch_mxfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw, uint8_t *packed,
                                 uint8_t *scales, hipStream_t stream);
// NVFP4 -> BF16 [n, k] (row stride ldo): e2m1 * e4m3 * s_t rounded once to BF16
hipError_t launch_nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                   int64_t n, int64_t k, uint16_t *out, int64_t ldo, hipStream_t stream);

// ---- W4A16 + LoRA ----
struct GemmArgs {
    const uint16_t *x;
    int64_t m, k, ldx;
    const uint8_t *packed;
    const uint8_t *scales;
    const float *tensor_scale;
    int64_t n;
    const uint16_t *lora_a;
    const uint16_t *lora_b;
    int r;
    float lora_scale;
    uint16_t *y;
    int64_t ldy;
    void *workspace;
    // RMSNorm prologue (decode path, m <= 16): x is the norm's input and each
    // row is normed with scale vector norm_w [k] and norm_eps before the
    // product; nullptr: x is used as it is
    const float *norm_w = nullptr;
    float norm_eps = 0.0f;
};
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
#define QERL_MAX_SEGMENTS 4
hipError_t launch_w4a16_lora_gemm(const GemmArgs &a, hipStream_t stream);
// device address of the current device's copy of the static scratch array
// (QERL_NOALLOC_SCRATCH_BYTES), looked up on the first call on each device
hipError_t noalloc_scratch(void **ptr);
// decode batches (m <= kDecodeMaxM): HBM-streaming path in decode.hip
constexpr int64_t kDecodeMaxM = 256;
size_t decode_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
hipError_t launch_decode(const GemmArgs &a, hipStream_t stream);
// Several GEMMs sharing x (m, k, ldx) in one launch: segs[i] differ only in
// the weight, LoRA and output fields and all carry the same workspace.
size_t gemm_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg);
hipError_t launch_w4a16_lora_gemm_multi(const GemmArgs *segs, int nseg, hipStream_t stream);
size_t decode_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg,
                                    bool norm = false);
hipError_t launch_decode_multi(const GemmArgs *segs, int nseg, hipStream_t stream);
// RMSNorm + GEMMs: the norm fused into the decode launch when m <= kNormFuseMaxM
// and k % 32 == 0 (segs carry norm_w), else a norm launch into the workspace
// and then launch_w4a16_lora_gemm_multi
constexpr int64_t kNormFuseMaxM = 16;
size_t norm_gemm_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg);
hipError_t launch_norm_gemm_multi(const GemmArgs *segs, int nseg, hipStream_t stream);
// Host checks of a launch's workspace use against its size query (0: in
// bounds; else a message in msg): decode (m <= 256) launches over segments of
// one x, one projection's launch for a workspace of `size` bytes, and the
// multi-segment calls with or without the RMSNorm.
int decode_plan_check(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm, char *msg,
                      size_t len);
int gemm_plan_check(int64_t m, int64_t n, int64_t k, int r, int64_t size, char *msg, size_t len);
int gemm_multi_plan_check(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm, char *msg,
                          size_t len);

// ---- backward of the layer (LoRA trained, W frozen) ----
constexpr int kMaxRankBwd = 128;  // QERL_MAX_LORA_RANK
struct BackwardArgs {
    const uint16_t *dy;  // [m, n], row stride ldy
    const uint16_t *x;   // [m, k], row stride ldx
    int64_t m, n, k, ldy, ldx;
    const uint8_t *packed;
    const uint8_t *scales;
    const float *tensor_scale;
    const uint16_t *lora_a;  // [r, k]
    const uint16_t *lora_b;  // [n, r]
    int r;
    float lora_scale;
    uint16_t *dx;  // [m, k], row stride lddx (nullable)
    int64_t lddx;
    float *da;  // [r, k] (nullable)
    float *db;  // [n, r] (nullable)
    void *workspace;
};
size_t backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
hipError_t launch_backward(const BackwardArgs &b, hipStream_t stream);

// ---- AQN RMSNorm ----
struct AqnArgs {
    const uint16_t *x;
    int64_t m, h, ldx;
    const float *weight;
    float eps, sigma;
    uint64_t seed, step;
    uint32_t layer;
    float *y_f32;
    uint16_t *y_bf16;
    int64_t ldy;
    float *noisy_out;
};
hipError_t launch_aqn_rmsnorm(const AqnArgs &a, hipStream_t stream);
// w + sigma z alone (a.x, a.m and the outputs unused; a.noisy_out required)
hipError_t launch_aqn_noisy_weight(const AqnArgs &a, hipStream_t stream);

}  // namespace qerl
