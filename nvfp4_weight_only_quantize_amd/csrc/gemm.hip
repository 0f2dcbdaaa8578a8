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
// Larger m (m > 64; m <= 64 is the decode path of decode.hip):
//   prologue_kernel  t = x A^T in FP32, pre-multiplied by lora_scale / s_t and
//                    split into BF16 hi + lo halves, so that the LoRA product
//                    becomes 2r extra K columns of the same MFMA accumulation.
//   tiled_kernel     64x64 output tiles, x and dequantized weight tiles
//                    (e2m1 * e4m3 is exact in BF16) staged in LDS, BF16 MFMA
//                    16x16x32 with FP32 accumulation; s_t applied once.
#include "device_common.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Launch plan and workspace layout
// ---------------------------------------------------------------------------
// The workspace starts with the decode path's counter region, which this path
// never touches, then holds the BF16 hi/lo t [m, 2r].
struct Plan {
    int64_t t_off, bytes;
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

Plan make_plan(int64_t m, int64_t n, int64_t k, int r) {
    (void)n;
    (void)k;
    Plan p{};
    p.t_off = kGemmCtrBytes;
    p.bytes = p.t_off + align256(m * (int64_t)r * 4);
    return p;
}

struct Gemm {
    GemmArgs a;
    Plan p;
    __device__ uint16_t *t16() const { return reinterpret_cast<uint16_t *>(static_cast<char *>(a.workspace) + p.t_off); }
};

// ---------------------------------------------------------------------------
// Prologue: LoRA down-projection t = x A^T
// ---------------------------------------------------------------------------
// One workgroup per (row m, rank j); its 256 lanes split K (16 bytes per lane
// per step, four steps in flight).  Output, with u = t * lora_scale / s_t:
//   t16[m * 2r + j] = bf16(u), t16[m * 2r + r + j] = bf16(u - bf16(u))
__global__ __launch_bounds__(kThreads) void prologue_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    const int64_t pair = blockIdx.x;
    const int64_t m = pair / a.r;
    const int j = (int)(pair - m * a.r);
    const uint16_t *xr = a.x + m * a.ldx;
    const uint16_t *ar = a.lora_a + (int64_t)j * a.k;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t step = (int64_t)kThreads * 8;
    int64_t kk = (int64_t)threadIdx.x * 8;
    for (; kk + 3 * step < a.k; kk += 4 * step) {
        uint4 xv[4], av[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xv[u] = *reinterpret_cast<const uint4 *>(xr + kk + u * step);
            av[u] = *reinterpret_cast<const uint4 *>(ar + kk + u * step);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc[u] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u].x), as_bf16x2(av[u].x), acc[u], false);
            acc[u] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u].y), as_bf16x2(av[u].y), acc[u], false);
            acc[u] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u].z), as_bf16x2(av[u].z), acc[u], false);
            acc[u] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u].w), as_bf16x2(av[u].w), acc[u], false);
        }
    }
    for (; kk < a.k; kk += step) {  // k % 16 == 0: a vector never straddles the end
        const uint4 xv = *reinterpret_cast<const uint4 *>(xr + kk);
        const uint4 av = *reinterpret_cast<const uint4 *>(ar + kk);
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.x), as_bf16x2(av.x), acc[0], false);
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.y), as_bf16x2(av.y), acc[0], false);
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.z), as_bf16x2(av.z), acc[0], false);
        acc[0] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.w), as_bf16x2(av.w), acc[0], false);
    }
    __shared__ float red[4];
    const float t = block_sum_256((acc[0] + acc[1]) + (acc[2] + acc[3]), red);
    if (threadIdx.x == 0) {
        const float u = t * (a.lora_scale / *a.tensor_scale);
        const uint16_t hi = f32_to_bf16_bits(u);
        const uint16_t lo = f32_to_bf16_bits(u - __uint_as_float((uint32_t)hi << 16));
        uint16_t *t16 = g.t16();
        t16[m * 2 * a.r + j] = hi;
        t16[m * 2 * a.r + a.r + j] = lo;
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
        e[i] = j < klora ? a.lora_b[n * a.r + (j < a.r ? j : j - a.r)] : (uint16_t)0;
    }
    o.x = e[0] | ((uint32_t)e[1] << 16);
    o.y = e[2] | ((uint32_t)e[3] << 16);
    o.z = e[4] | ((uint32_t)e[5] << 16);
    o.w = e[6] | ((uint32_t)e[7] << 16);
    return o;
}

// 8 activations of row m at column kk (main range from x, LoRA range from the
// split t in the workspace, row stride 2r).
__device__ __forceinline__ uint4 load_x_piece(const Gemm &g, int64_t m, int64_t kk, int64_t klora) {
    const GemmArgs &a = g.a;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (m >= a.m) return o;
    if (kk < a.k) return *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + kk);
    const int64_t j0 = kk - a.k;
    if (j0 >= klora) return o;
    const uint16_t *t16 = g.t16() + m * klora;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (j0 + i < klora) ? t16[j0 + i] : (uint16_t)0;
    o.x = e[0] | ((uint32_t)e[1] << 16);
    o.y = e[2] | ((uint32_t)e[3] << 16);
    o.z = e[4] | ((uint32_t)e[5] << 16);
    o.w = e[6] | ((uint32_t)e[7] << 16);
    return o;
}

__global__ __launch_bounds__(kThreads) void tiled_kernel(Gemm g) {
    const GemmArgs &a = g.a;
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
        *reinterpret_cast<uint4 *>(&sx[lr * LDS_PITCH + lc]) = load_x_piece(g, m0 + lr, k0 + lc, klora);
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

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    if (m <= kDecodeMaxM) return decode_workspace_bytes(m, n, k, r);
    return (size_t)make_plan(m, n, k, r).bytes;
}

hipError_t launch_w4a16_lora_gemm(const GemmArgs &a, hipStream_t stream) {
    if (a.m <= kDecodeMaxM) return launch_decode(a, stream);
    const Gemm g{a, make_plan(a.m, a.n, a.k, a.r)};
    if (a.r > 0) {
        const int64_t grid = a.m * a.r;
        if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t tiles = ((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(tiled_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

}  // namespace qerl
