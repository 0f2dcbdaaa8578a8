// aqn.hip -- RMSNorm with adaptive quantization noise (AQN) for gfx950.
//
// AQN injects channel-wise Gaussian noise through the normalization layer
// ("Paper 2510.11696 -- QeRL: Beyond Efficiency", "Summary"); the noise sits in
// the norm's scale parameters, so no extra weights are needed (dataforcee
// page, findings section).  Here the FP32 scale vector becomes w + sigma * z
// with one z ~ N(0, 1) per channel, shared by all rows, and
//   y[i, c] = x[i, c] / sqrt(mean_c x[i, c]^2 + eps) * (w[c] + sigma z[c]).
//
// z is a pure function of (seed, step, layer): counter-based Philox4x64-10
// (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed, layer) and counter
// (c/4, step, 0, 0), then Box-Muller (1958) on word pairs (r0, r1), (r2, r3).
//
// Launch: a 2-D grid.  blockIdx.x picks 1024 channels (4 per thread: one
// Philox block), blockIdx.y a group of rows (one row for m <= 512, else
// kRows).  Every workgroup reads the whole of its rows for the sum of squares
// (L2-resident, a few KB per row), so no workgroup waits for another; the
// noise of a channel is drawn once per row group.
#include "device_common.h"
#include "../../include/qerl.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;
constexpr int kChanPerWg = 4 * kThreads;
constexpr int kRows = 4;           // rows per workgroup (m > kOneRowMaxM)
constexpr int64_t kOneRowMaxM = 512;
constexpr int kMaxRowGroups = 8192;

// compute units of the current device (queried once)
int64_t aqn_cus() {
    static const int64_t cus = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        return (int64_t)v;
    }();
    return cus;
}

__device__ __forceinline__ void box_muller(uint64_t ra, uint64_t rb, float &z0, float &z1) {
    const float u1 = (float)((ra >> 40) + 1) * 0x1p-24f;  // (0, 1]
    const float u2 = (float)(rb >> 40) * 0x1p-24f;        // [0, 1)
    const float rad = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincospif(2.0f * u2, &s, &c);
    z0 = rad * c;
    z1 = rad * s;
}

// VEC: x rows 16-byte aligned (x % 16 == 0, ldx % 8 == 0, h % 8 == 0) and
// outputs vector-aligned (y_f32 % 16, y_bf16 % 8, ldy % 4 == 0).
// ROWS: rows per workgroup and row group.  Each row's loads -- its 16-byte
// pieces for the sum of squares (at most kMaxPieces per thread) and this
// thread's 4 output channels -- are issued together, and the noise is drawn
// while they travel, so a row group costs one round trip.
constexpr int kMaxPieces = (QERL_MAX_NORM_WIDTH / 8 + kThreads - 1) / kThreads;
template <bool VEC, int ROWS>
__global__ __launch_bounds__(kThreads) void aqn_rmsnorm_kernel(AqnArgs a) {
    __shared__ float s_red[ROWS][4];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t g = (int64_t)blockIdx.x * kThreads + tid;  // Philox block: channels 4g .. 4g+3
    const int64_t c0 = 4 * g;
    const float inv_h = 1.0f / (float)a.h;
    bool drawn = false;
    float wn[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t rg = blockIdx.y; rg * ROWS < a.m; rg += gridDim.y) {
        const int64_t row0 = rg * ROWS;
        float ss[ROWS];
        uint2 xo[ROWS];  // this thread's output channels of each row (VEC)
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            ss[i] = 0.0f;
            xo[i] = make_uint2(0, 0);
            if (row0 + i >= a.m) continue;
            const uint16_t *xr = a.x + (row0 + i) * a.ldx;
            if (VEC) {
                uint4 v[kMaxPieces];
#pragma unroll
                for (int u = 0; u < kMaxPieces; ++u) {
                    const int64_t pc = tid + (int64_t)u * kThreads;
                    v[u] = pc * 8 < a.h ? *reinterpret_cast<const uint4 *>(xr + pc * 8) : make_uint4(0, 0, 0, 0);
                }
                if (c0 < a.h) xo[i] = *reinterpret_cast<const uint2 *>(xr + c0);
                if (!drawn) {  // (first row only) the noise while the loads travel
                    drawn = true;
                    if (c0 < a.h) {
                        float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // sigma == 0: w + 0 z is w
                        if (a.sigma != 0.0f) {
                            const U64x4 r = philox4x64_10((uint64_t)g, a.step, 0, 0, a.seed, (uint64_t)a.layer);
                            box_muller(r.v[0], r.v[1], z[0], z[1]);
                            box_muller(r.v[2], r.v[3], z[2], z[3]);
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (c0 + j < a.h) {
                                wn[j] = __builtin_fmaf(a.sigma, z[j], a.weight[c0 + j]);
                                if (blockIdx.y == 0 && a.noisy_out) a.noisy_out[c0 + j] = wn[j];
                            }
                    }
                }
#pragma unroll
                for (int u = 0; u < kMaxPieces; ++u) {
                    const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float lo = bf16lo_to_f32(w4[j]), hi = bf16hi_to_f32(w4[j]);
                        ss[i] = __builtin_fmaf(lo, lo, ss[i]);
                        ss[i] = __builtin_fmaf(hi, hi, ss[i]);
                    }
                }
            } else {
                for (int64_t c = tid; c < a.h; c += kThreads) {
                    const float v = bf16lo_to_f32(xr[c]);
                    ss[i] = __builtin_fmaf(v, v, ss[i]);
                }
            }
        }
        if (!drawn) {  // (no row drawn the noise yet: the scalar path, or a short row group)
            drawn = true;
            if (c0 < a.h) {
                float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (a.sigma != 0.0f) {
                    const U64x4 r = philox4x64_10((uint64_t)g, a.step, 0, 0, a.seed, (uint64_t)a.layer);
                    box_muller(r.v[0], r.v[1], z[0], z[1]);
                    box_muller(r.v[2], r.v[3], z[2], z[3]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (c0 + j < a.h) {
                        wn[j] = __builtin_fmaf(a.sigma, z[j], a.weight[c0 + j]);
                        if (blockIdx.y == 0 && a.noisy_out) a.noisy_out[c0 + j] = wn[j];
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < ROWS; ++i) ss[i] = wave_sum(ss[i]);
        __syncthreads();  // s_red may still be read for the previous row group
        if ((tid & 63) == 0)
#pragma unroll
            for (int i = 0; i < ROWS; ++i) s_red[i][wave] = ss[i];
        __syncthreads();
        if (c0 >= a.h) continue;
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const int64_t row = row0 + i;
            if (row >= a.m) break;
            const float tot = (s_red[i][0] + s_red[i][1]) + (s_red[i][2] + s_red[i][3]);
            const float inv = 1.0f / sqrtf(tot * inv_h + a.eps);
            if (VEC) {
                const uint2 xv = xo[i];
                const float y0 = bf16lo_to_f32(xv.x) * inv * wn[0], y1 = bf16hi_to_f32(xv.x) * inv * wn[1];
                const float y2 = bf16lo_to_f32(xv.y) * inv * wn[2], y3 = bf16hi_to_f32(xv.y) * inv * wn[3];
                if (a.y_f32) *reinterpret_cast<float4 *>(a.y_f32 + row * a.ldy + c0) = make_float4(y0, y1, y2, y3);
                if (a.y_bf16)
                    *reinterpret_cast<uint2 *>(a.y_bf16 + row * a.ldy + c0) =
                        make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            } else {
                const uint16_t *xr = a.x + row * a.ldx;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t c = c0 + j;
                    if (c >= a.h) break;
                    const float y = bf16lo_to_f32(xr[c]) * inv * wn[j];
                    if (a.y_f32) a.y_f32[row * a.ldy + c] = y;
                    if (a.y_bf16) a.y_bf16[row * a.ldy + c] = f32_to_bf16_bits(y);
                }
            }
        }
    }
}

// m > kOneRowMaxM, vector-aligned rows: a workgroup takes ROWS whole rows at
// a time (grid-stride over row groups) and reads each row once.  Thread tid
// holds the 16-byte pieces tid + kThreads u of every row, the same pieces and
// summation order as aqn_rmsnorm_kernel, so the sums of squares and outputs
// are the same bits; the row's outputs come from the pieces already in
// registers, and the scale w + sigma z of the thread's channels is drawn once
// per workgroup.  NP: pieces per thread (h <= 8 kThreads NP).
template <int ROWS, int NP>
__global__ __launch_bounds__(kThreads) void aqn_rmsnorm_rows_kernel(AqnArgs a) {
    __shared__ float s_red[ROWS][4];
    const int tid = threadIdx.x, wave = tid >> 6;
    const float inv_h = 1.0f / (float)a.h;
    float wn[NP][8];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int64_t pc = tid + (int64_t)u * kThreads;  // channels 8 pc .. 8 pc + 7 (h % 8 == 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) wn[u][j] = 0.0f;
        if (pc * 8 >= a.h) continue;
#pragma unroll
        for (int b = 0; b < 2; ++b) {  // Philox blocks 2 pc, 2 pc + 1: channels 4 g .. 4 g + 3
            const int64_t g = 2 * pc + b;
            float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // sigma == 0: w + 0 z is w
            if (a.sigma != 0.0f) {
                const U64x4 r = philox4x64_10((uint64_t)g, a.step, 0, 0, a.seed, (uint64_t)a.layer);
                box_muller(r.v[0], r.v[1], z[0], z[1]);
                box_muller(r.v[2], r.v[3], z[2], z[3]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wn[u][4 * b + j] = __builtin_fmaf(a.sigma, z[j], a.weight[4 * g + j]);
                if (blockIdx.x == 0 && a.noisy_out) a.noisy_out[4 * g + j] = wn[u][4 * b + j];
            }
        }
    }
    for (int64_t rg = blockIdx.x; rg * ROWS < a.m; rg += gridDim.x) {
        const int64_t row0 = rg * ROWS;
        uint4 v[ROWS][NP];
        float ss[ROWS];
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const uint16_t *xr = a.x + (row0 + i) * a.ldx;
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const int64_t pc = tid + (int64_t)u * kThreads;
                v[i][u] = row0 + i < a.m && pc * 8 < a.h ? *reinterpret_cast<const uint4 *>(xr + pc * 8)
                                                          : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            ss[i] = 0.0f;
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const uint32_t w4[4] = {v[i][u].x, v[i][u].y, v[i][u].z, v[i][u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = bf16lo_to_f32(w4[j]), hi = bf16hi_to_f32(w4[j]);
                    ss[i] = __builtin_fmaf(lo, lo, ss[i]);
                    ss[i] = __builtin_fmaf(hi, hi, ss[i]);
                }
            }
            ss[i] = wave_sum(ss[i]);
        }
        __syncthreads();  // s_red may still be read for the previous row group
        if ((tid & 63) == 0)
#pragma unroll
            for (int i = 0; i < ROWS; ++i) s_red[i][wave] = ss[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const int64_t row = row0 + i;
            if (row >= a.m) break;
            const float tot = (s_red[i][0] + s_red[i][1]) + (s_red[i][2] + s_red[i][3]);
            const float inv = 1.0f / sqrtf(tot * inv_h + a.eps);
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const int64_t pc = tid + (int64_t)u * kThreads;
                if (pc * 8 >= a.h) continue;
                const uint32_t w4[4] = {v[i][u].x, v[i][u].y, v[i][u].z, v[i][u].w};
                float y[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    y[2 * j] = bf16lo_to_f32(w4[j]) * inv * wn[u][2 * j];
                    y[2 * j + 1] = bf16hi_to_f32(w4[j]) * inv * wn[u][2 * j + 1];
                }
                if (a.y_f32) {
                    float4 *yo = reinterpret_cast<float4 *>(a.y_f32 + row * a.ldy + pc * 8);
                    yo[0] = make_float4(y[0], y[1], y[2], y[3]);
                    yo[1] = make_float4(y[4], y[5], y[6], y[7]);
                }
                if (a.y_bf16)
                    *reinterpret_cast<uint4 *>(a.y_bf16 + row * a.ldy + pc * 8) =
                        make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                   pack_bf16x2(y[6], y[7]));
            }
        }
    }
}

// w + sigma z alone: the scale vector every norm call of one (seed, step,
// layer) uses, for callers that apply it themselves (the RMSNorm prologue of
// the decode GEMM).  Thread g draws channels 4g .. 4g + 3, as above.
__global__ __launch_bounds__(kThreads) void aqn_noisy_weight_kernel(AqnArgs a) {
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t c0 = 4 * g;
    if (c0 >= a.h) return;
    const U64x4 r = philox4x64_10((uint64_t)g, a.step, 0, 0, a.seed, (uint64_t)a.layer);
    float z[4];
    box_muller(r.v[0], r.v[1], z[0], z[1]);
    box_muller(r.v[2], r.v[3], z[2], z[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (c0 + i < a.h) a.noisy_out[c0 + i] = __builtin_fmaf(a.sigma, z[i], a.weight[c0 + i]);
}

}  // namespace

hipError_t launch_aqn_noisy_weight(const AqnArgs &a, hipStream_t stream) {
    const int64_t blocks = (a.h + kChanPerWg - 1) / kChanPerWg;
    hipLaunchKernelGGL(aqn_noisy_weight_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_aqn_rmsnorm(const AqnArgs &a, hipStream_t stream) {
    const bool vec = ((uintptr_t)a.x & 15u) == 0 && a.ldx % 8 == 0 && a.h % 8 == 0 &&
                     ((uintptr_t)a.y_f32 & 15u) == 0 && ((uintptr_t)a.y_bf16 & 7u) == 0 && a.ldy % 4 == 0;
    // one row per workgroup while that gives few enough workgroups (each
    // draws its channels' noise once); kRows rows per group above
    const int rows = a.m <= kOneRowMaxM ? 1 : kRows;
    const int64_t row_groups = (a.m + rows - 1) / rows;
    const dim3 grid((unsigned)((a.h + kChanPerWg - 1) / kChanPerWg),
                    (unsigned)(row_groups < kMaxRowGroups ? row_groups : kMaxRowGroups));
    if (vec && rows > 1 && ((uintptr_t)a.y_bf16 & 15u) == 0 && ((uintptr_t)a.y_f32 & 15u) == 0 && a.ldy % 8 == 0) {
        // whole rows per workgroup: a few row groups each, so the noise is drawn
        // once per few rows rather than once per row group; two workgroups per CU
        // (M = 8192, H = 5120: 37 us, against 43-45 us with one, three or four
        // per CU, 38 us with two rows a group and 76 us with eight)
        const int64_t wgs = row_groups < 2 * aqn_cus() ? row_groups : 2 * aqn_cus();
        if (a.h <= 8 * kThreads * 4)
            hipLaunchKernelGGL((aqn_rmsnorm_rows_kernel<kRows, 4>), dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((aqn_rmsnorm_rows_kernel<kRows / 2, kMaxPieces>), dim3((unsigned)wgs), dim3(kThreads), 0,
                               stream, a);
        return hipGetLastError();
    }
    if (vec) {
        if (rows == 1)
            hipLaunchKernelGGL((aqn_rmsnorm_kernel<true, 1>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((aqn_rmsnorm_kernel<true, kRows>), grid, dim3(kThreads), 0, stream, a);
    } else {
        if (rows == 1)
            hipLaunchKernelGGL((aqn_rmsnorm_kernel<false, 1>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((aqn_rmsnorm_kernel<false, kRows>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace qerl
