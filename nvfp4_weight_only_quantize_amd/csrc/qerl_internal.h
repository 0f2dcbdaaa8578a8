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
hipError_t launch_nvfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                                 uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                 const float *tensor_scale_in, uint32_t flags, void *workspace,
                                 hipStream_t stream);

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
};
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
// Every GEMM workspace starts with this many bytes of counters for the decode
// path's in-kernel split-K reduction: zero before first use, left zero by
// every call (the other path never writes them).
constexpr int64_t kGemmCtrBytes = 64 * 1024;
hipError_t launch_w4a16_lora_gemm(const GemmArgs &a, hipStream_t stream);
// decode batches (m <= kDecodeMaxM): HBM-streaming path in decode.hip
constexpr int64_t kDecodeMaxM = 64;
size_t decode_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);
hipError_t launch_decode(const GemmArgs &a, hipStream_t stream);

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

}  // namespace qerl
