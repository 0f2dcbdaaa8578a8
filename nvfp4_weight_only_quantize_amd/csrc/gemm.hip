// gemm.hip -- W4A16 (NVFP4 weight x BF16 activation) linear layer with a
// BF16 LoRA update, for gfx950.
//
//   y[m, n] = s_t * sum_k x[m,k] e2m1(q[n,k]) e4m3(sb[n,k/16])
//           + lora_scale * sum_j t[m,j] B[n,j],      t = x A^T
//
// The frozen NVFP4 base times BF16 activations is the rollout kernel of the
// "NVlabs/QeRL" README ("Acknowledgement"); the LoRA sum is the low-rank
// update of the bitsofall page ("LoRA (Low-Rank Adaptation)"), fused into the
// same kernel as its "Implementation and Practical Details" section asks
// ("NVFP4 + LoRA summation").
//
// Kernels:
//   lora_down_kernel  t = x A^T in FP32 (one wave per output), written to the
//                     workspace either as FP32 (GEMV path) or pre-multiplied by
//                     lora_scale / s_t and split into BF16 hi + lo halves (MFMA
//                     path, where the LoRA product becomes 2r extra K columns).
//   gemv_kernel       small m: HBM-streaming; groups of LPR lanes own one weight
//                     row, 16-byte loads of 32 nibbles, E2M1 -> BF16 decode in
//                     registers, v_dot2_f32_bf16 against x, one FP32 FMA per
//                     16-element block for the E4M3 scale, lane-group reduction.
//   mfma_kernel       larger m: 64x64 output tiles, x and dequantized weight
//                     tiles (e2m1 * e4m3 is exact in BF16) staged in LDS, BF16
//                     MFMA 16x16x32 with FP32 accumulation; s_t applied once.
#include "device_common.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// LoRA down-projection
// ---------------------------------------------------------------------------
enum LoraOut { kLoraF32 = 0, kLoraSplitBf16 = 1 };

// One wave per (row m, rank j).  Output:
//   kLoraF32:       t32[m * r + j] = t
//   kLoraSplitBf16: t16[m * 2r + j] = bf16(u), t16[m * 2r + r + j] = bf16(u - bf16(u)),
//                   with u = t * lora_scale / s_t
template <int MODE>
__global__ __launch_bounds__(kThreads) void lora_down_kernel(GemmArgs a) {
    const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t total = a.m * a.r;
    if (wave_id >= total) return;
    const int64_t m = wave_id / a.r;
    const int j = (int)(wave_id - m * a.r);
    const uint16_t *xr = a.x + m * a.ldx;
    const uint16_t *ar = a.lora_a + (int64_t)j * a.k;
    float acc = 0.0f;
    // 8 elements (16 B) per lane per step; k % 16 == 0 so vectors never straddle the end
    for (int64_t kk = (int64_t)lane * 8; kk < a.k; kk += 64 * 8) {
        const uint4 xv = *reinterpret_cast<const uint4 *>(xr + kk);
        const uint4 av = *reinterpret_cast<const uint4 *>(ar + kk);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.x), as_bf16x2(av.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.y), as_bf16x2(av.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.z), as_bf16x2(av.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.w), as_bf16x2(av.w), acc, false);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        if (MODE == kLoraF32) {
            static_cast<float *>(a.workspace)[m * a.r + j] = acc;
        } else {
            const float u = acc * (a.lora_scale / *a.tensor_scale);
            const uint16_t hi = f32_to_bf16_bits(u);
            const uint16_t lo = f32_to_bf16_bits(u - __uint_as_float((uint32_t)hi << 16));
            uint16_t *t16 = static_cast<uint16_t *>(a.workspace);
            t16[m * 2 * a.r + j] = hi;
            t16[m * 2 * a.r + a.r + j] = lo;
        }
    }
}

// ---------------------------------------------------------------------------
// GEMV path (m <= 4)
// ---------------------------------------------------------------------------
// Dot of 16 decoded weights (two 32-bit words of packed nibbles) with 16 BF16
// activations (two 16-byte vectors), FP32 result.
__device__ __forceinline__ float dot16(uint32_t q0, uint32_t q1, const uint4 &x0, const uint4 &x1) {
    float p = 0.0f;
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q0, 0), as_bf16x2(x0.x), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q0, 1), as_bf16x2(x0.y), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q0, 2), as_bf16x2(x0.z), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q0, 3), as_bf16x2(x0.w), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q1, 0), as_bf16x2(x1.x), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q1, 1), as_bf16x2(x1.y), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q1, 2), as_bf16x2(x1.z), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(QERL_FP4_PAIR_BF16(q1, 3), as_bf16x2(x1.w), p, false);
    return p;
}

// Requires k % 32 == 0 (one 16-byte packed vector = 32 elements = two blocks).
template <int MT, int LPR>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemmArgs a) {
    constexpr int kGroups = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const int group = threadIdx.x / LPR;
    const int64_t chunks = a.k >> 5;
    const float st = *a.tensor_scale;
    const float *t32 = static_cast<const float *>(a.workspace);
    for (int64_t n = (int64_t)blockIdx.x * kGroups + group; n < a.n; n += (int64_t)gridDim.x * kGroups) {
        const uint4 *wrow = reinterpret_cast<const uint4 *>(a.packed + n * (a.k >> 1));
        const uint16_t *srow = reinterpret_cast<const uint16_t *>(a.scales + n * (a.k >> 4));
        float acc[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = 0.0f;
#pragma unroll 2
        for (int64_t c = sub; c < chunks; c += LPR) {
            const uint4 q = wrow[c];
            const uint32_t sc = srow[c];
            const float s0 = QERL_E4M3_F32(sc, 0), s1 = QERL_E4M3_F32(sc, 1);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const uint4 *xv = reinterpret_cast<const uint4 *>(a.x + i * a.ldx + c * 32);
                const uint4 x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
                acc[i] = __builtin_fmaf(dot16(q.x, q.y, x0, x1), s0, acc[i]);
                acc[i] = __builtin_fmaf(dot16(q.z, q.w, x2, x3), s1, acc[i]);
            }
        }
        float v[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            float lora = 0.0f;
            for (int j = sub; j < a.r; j += LPR)
                lora = __builtin_fmaf(t32[i * a.r + j], bf16lo_to_f32(a.lora_b[n * a.r + j]), lora);
            v[i] = st * acc[i] + a.lora_scale * lora;
        }
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) {
#pragma unroll
            for (int i = 0; i < MT; ++i) v[i] += __shfl_xor(v[i], off, kWave);
        }
        if (sub == 0) {
#pragma unroll
            for (int i = 0; i < MT; ++i) a.y[i * a.ldy + n] = f32_to_bf16_bits(v[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------
constexpr int BM = 64, BN = 64, BK = 32, LDS_PITCH = BK + 8;  // pitch in BF16 elements

// Fill one 8-element (16-byte) piece of the weight tile: row n, columns
// [kk, kk + 8) of the main range (dequantized e2m1 * e4m3, exact in BF16) or
// of the LoRA range (B[n, j] for j = kk mod r, which pairs with the hi and lo
// halves of the scaled t).
__device__ __forceinline__ uint4 load_w_piece(const GemmArgs &a, int64_t n, int64_t kk, int64_t klora) {
    uint4 o = make_uint4(0, 0, 0, 0);
    if (n >= a.n) return o;
    if (kk < a.k) {
        const uint32_t q = *reinterpret_cast<const uint32_t *>(a.packed + n * (a.k >> 1) + (kk >> 1));
        const float sc = QERL_E4M3_F32(a.scales[n * (a.k >> 4) + (kk >> 4)], 0);
        const f32x2_t f0 = QERL_FP4_PAIR_F32(q, 0), f1 = QERL_FP4_PAIR_F32(q, 1);
        const f32x2_t f2 = QERL_FP4_PAIR_F32(q, 2), f3 = QERL_FP4_PAIR_F32(q, 3);
        o.x = pack_bf16x2(f0.x * sc, f0.y * sc);
        o.y = pack_bf16x2(f1.x * sc, f1.y * sc);
        o.z = pack_bf16x2(f2.x * sc, f2.y * sc);
        o.w = pack_bf16x2(f3.x * sc, f3.y * sc);
        return o;
    }
    const int64_t j0 = kk - a.k;  // column inside the LoRA range [0, 2r)
    if (j0 >= klora) return o;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t j = j0 + i;
        e[i] = j < klora ? a.lora_b[n * a.r + (j % a.r)] : (uint16_t)0;
    }
    o.x = e[0] | ((uint32_t)e[1] << 16);
    o.y = e[2] | ((uint32_t)e[3] << 16);
    o.z = e[4] | ((uint32_t)e[5] << 16);
    o.w = e[6] | ((uint32_t)e[7] << 16);
    return o;
}

// 8 activations of row m at column kk (main range from x, LoRA range from the
// split t in the workspace, row stride 2r).
__device__ __forceinline__ uint4 load_x_piece(const GemmArgs &a, int64_t m, int64_t kk, int64_t klora) {
    uint4 o = make_uint4(0, 0, 0, 0);
    if (m >= a.m) return o;
    if (kk < a.k) return *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + kk);
    const int64_t j0 = kk - a.k;
    if (j0 >= klora) return o;
    const uint16_t *t16 = static_cast<const uint16_t *>(a.workspace) + m * klora;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (j0 + i < klora) ? t16[j0 + i] : (uint16_t)0;
    o.x = e[0] | ((uint32_t)e[1] << 16);
    o.y = e[2] | ((uint32_t)e[3] << 16);
    o.z = e[4] | ((uint32_t)e[5] << 16);
    o.w = e[6] | ((uint32_t)e[7] << 16);
    return o;
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sx[BM * LDS_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sw[BN * LDS_PITCH];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t tiles_n = (a.n + BN - 1) / BN;
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    const int64_t klora = 2 * (int64_t)a.r;
    const int64_t ktot = a.k + klora;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int lr = tid >> 2, lc = (tid & 3) * 8;  // loader: row and 8-column piece
    for (int64_t k0 = 0; k0 < ktot; k0 += BK) {
        *reinterpret_cast<uint4 *>(&sx[lr * LDS_PITCH + lc]) = load_x_piece(a, m0 + lr, k0 + lc, klora);
        *reinterpret_cast<uint4 *>(&sw[lr * LDS_PITCH + lc]) = load_w_piece(a, n0 + lr, k0 + lc, klora);
        __syncthreads();
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t *>(&sx[(wm + 16 * i + (lane & 15)) * LDS_PITCH + 8 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8_t *>(&sw[(wn + 16 * j + (lane & 15)) * LDS_PITCH + 8 * (lane >> 4)]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        __syncthreads();
    }
    const float st = *a.tensor_scale;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
                const int64_t n = n0 + wn + 16 * j + (lane & 15);
                if (m < a.m && n < a.n) a.y[m * a.ldy + n] = f32_to_bf16_bits(st * acc[i][j][v]);
            }
}

constexpr int64_t kGemvMaxM = 4;

int num_cus() {
    static int cus = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess) return 256;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            return 256;
        return v;
    }();
    return cus;
}

template <int MT>
hipError_t launch_gemv(const GemmArgs &a, hipStream_t stream) {
    // enough lanes per row that the grid covers the chip several times over
    const int64_t cus = num_cus();
    const int64_t target_waves = cus * 16;
    int lpr = 16;
    if (a.n * 16 / 64 < target_waves) lpr = 64;
    const int groups = kThreads / lpr;
    int64_t grid = (a.n + groups - 1) / groups;
    if (grid > cus * 64) grid = cus * 64;
    if (lpr == 64)
        hipLaunchKernelGGL((gemv_kernel<MT, 64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemv_kernel<MT, 16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t, int64_t, int r) {
    // FP32 t [m, r] (GEMV path) or BF16 hi/lo t [m, 2r] (MFMA path): same size
    const size_t bytes = (size_t)m * (size_t)(r > 0 ? r : 0) * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_w4a16_lora_gemm(const GemmArgs &a, hipStream_t stream) {
    const bool gemv = a.m <= kGemvMaxM && (a.k % 32) == 0;
    if (a.r > 0) {
        const int64_t waves = a.m * a.r;
        const int64_t grid = (waves * 64 + kThreads - 1) / kThreads;
        if (gemv)
            hipLaunchKernelGGL((lora_down_kernel<kLoraF32>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((lora_down_kernel<kLoraSplitBf16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (gemv) {
        switch (a.m) {
            case 1: return launch_gemv<1>(a, stream);
            case 2: return launch_gemv<2>(a, stream);
            case 3: return launch_gemv<3>(a, stream);
            default: return launch_gemv<4>(a, stream);
        }
    }
    const int64_t tiles = ((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qerl
