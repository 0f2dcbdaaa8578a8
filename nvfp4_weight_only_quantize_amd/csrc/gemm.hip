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
//   prefill_kernel   256 x 128 output tiles, x and dequantized weight tiles
//                    (e2m1 * e4m3 is exact in BF16) double-buffered in LDS,
//                    BF16 MFMA 16x16x32 with FP32 accumulation; s_t applied
//                    once.
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
// MFMA path (m > 64)
// ---------------------------------------------------------------------------
// Workgroup tile 256 (rows of x) x 128 (weight rows), K in steps of 32; four
// waves, each a 128 x 64 sub-tile (8 x 4 MFMA 16x16x32 tiles, 128 FP32
// accumulators per lane).  x and dequantized weight tiles are double-buffered
// in LDS; the global loads of step s+1 are in flight while step s multiplies.
// The LoRA product rides along as 2r extra K columns (t hi/lo x B twice).
constexpr int PBM = 256, PBN = 128, PBK = 32, PPITCH = PBK + 8;  // LDS row pitch in BF16 elements
constexpr int PA_STAGE = PBM * PPITCH, PB_STAGE = PBN * PPITCH;  // elements per LDS stage

// 8 elements of the extended K range [0, k + 2r) for x row m at column kk:
// x itself, then the BF16 hi/lo halves of t * lora_scale / s_t; zero past
// the end and for rows past m.
__device__ __forceinline__ uint4 x_piece_ext(const Gemm &g, int64_t m, int64_t kk, int64_t klora) {
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
    __builtin_memcpy(&o, e, 16);
    return o;
}

// 16 weights of row n at columns [kk, kk + 16) of the extended K range:
// dequantized NVFP4 (exact in BF16), then B [n, j] for j = column - k mod r;
// zero past the end and for rows past n.
__device__ __forceinline__ void w_piece_ext(const GemmArgs &a, int64_t n, int64_t kk, int64_t klora, uint4 &lo,
                                            uint4 &hi) {
    lo = hi = make_uint4(0, 0, 0, 0);
    if (n >= a.n) return;
    if (kk < a.k) {  // k % 16 == 0: a 16-element block is inside or outside
        const uint2 q = *reinterpret_cast<const uint2 *>(a.packed + n * (a.k >> 1) + (kk >> 1));
        const float sc = QERL_E4M3_F32(a.scales[n * (a.k >> 4) + (kk >> 4)], 0);
        const f32x2_t f0 = QERL_FP4_PAIR_F32(q.x, 0), f1 = QERL_FP4_PAIR_F32(q.x, 1);
        const f32x2_t f2 = QERL_FP4_PAIR_F32(q.x, 2), f3 = QERL_FP4_PAIR_F32(q.x, 3);
        const f32x2_t f4 = QERL_FP4_PAIR_F32(q.y, 0), f5 = QERL_FP4_PAIR_F32(q.y, 1);
        const f32x2_t f6 = QERL_FP4_PAIR_F32(q.y, 2), f7 = QERL_FP4_PAIR_F32(q.y, 3);
        lo = make_uint4(pack_bf16x2(f0.x * sc, f0.y * sc), pack_bf16x2(f1.x * sc, f1.y * sc),
                        pack_bf16x2(f2.x * sc, f2.y * sc), pack_bf16x2(f3.x * sc, f3.y * sc));
        hi = make_uint4(pack_bf16x2(f4.x * sc, f4.y * sc), pack_bf16x2(f5.x * sc, f5.y * sc),
                        pack_bf16x2(f6.x * sc, f6.y * sc), pack_bf16x2(f7.x * sc, f7.y * sc));
        return;
    }
    const int64_t j0 = kk - a.k;
    uint16_t e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t j = j0 + i;
        e[i] = j < klora ? a.lora_b[n * a.r + (j < a.r ? j : j - a.r)] : (uint16_t)0;
    }
    __builtin_memcpy(&lo, e, 16);
    __builtin_memcpy(&hi, e + 8, 16);
}

__global__ __launch_bounds__(256, 2) void prefill_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    extern __shared__ __attribute__((aligned(16))) uint16_t plds[];
    uint16_t *sa = plds;                   // [2][PBM][PPITCH]
    uint16_t *sb = plds + 2 * PA_STAGE;    // [2][PBN][PPITCH]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous range of tiles (n fastest), so the workgroups sharing an x
    // row block also share that XCD's L2
    const int64_t tiles_n = (a.n + PBN - 1) / PBN, tiles = tiles_n * ((a.m + PBM - 1) / PBM);
    const int64_t b = blockIdx.x, x8 = b % 8, q8 = tiles / 8, r8 = tiles % 8;
    const int64_t tile = x8 * q8 + (x8 < r8 ? x8 : r8) + b / 8;
    const int64_t m0 = (tile / tiles_n) * PBM, n0 = (tile % tiles_n) * PBN;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t klora = 2 * (int64_t)a.r;
    const int64_t ktot = a.k + klora;
    const int64_t steps = (ktot + PBK - 1) / PBK;
    const bool fast_k = (a.k & 31) == 0;

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // this thread's loads: x rows tid/4 + 64u, 8-column piece tid % 4; weight
    // row tid / 2, 16-column half tid % 2
    const int xr = tid >> 2, xc = (tid & 3) * 8;
    const int wr = tid >> 1, wc = (tid & 1) * 16;
    const int64_t wn_row = n0 + wr < a.n ? n0 + wr : a.n - 1;
    // x rows past m are clamped (their outputs are discarded); named
    // registers, not arrays (an array here ends up in scratch memory)
    auto xrow = [&](int u) {
        const int64_t m = m0 + xr + 64 * u < a.m ? m0 + xr + 64 * u : a.m - 1;
        return a.x + m * a.ldx + xc;
    };
    const uint16_t *xr0 = xrow(0), *xr1 = xrow(1), *xr2 = xrow(2), *xr3 = xrow(3);
    const uint8_t *wq_row = a.packed + wn_row * (a.k >> 1) + (wc >> 1);
    const uint8_t *ws_row = a.scales + wn_row * (a.k >> 4) + (wc >> 4);

    // compute one K step from LDS buffer buf
    auto mma_step = [&](int buf) {
        const uint16_t *pa = sa + buf * PA_STAGE + (wm * 128 + lr) * PPITCH + 8 * lq;
        const uint16_t *pb = sb + buf * PB_STAGE + (wn * 64 + lr) * PPITCH + 8 * lq;
        bf16x8_t bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const bf16x8_t *>(pb + 16 * j * PPITCH);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(pa + 16 * i * PPITCH);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- the main K range in full 32-column steps (k % 32 == 0): plain
    // vector loads of step s+1 in flight while step s multiplies ----
    const int64_t fast_steps = fast_k ? a.k / PBK : 0;
    uint4 xp0, xp1, xp2, xp3;
    uint2 wq;
    uint32_t wsb;
    auto issue = [&](int64_t s) {
        const int64_t k0 = s * PBK;
        xp0 = *reinterpret_cast<const uint4 *>(xr0 + k0);
        xp1 = *reinterpret_cast<const uint4 *>(xr1 + k0);
        xp2 = *reinterpret_cast<const uint4 *>(xr2 + k0);
        xp3 = *reinterpret_cast<const uint4 *>(xr3 + k0);
        wq = *reinterpret_cast<const uint2 *>(wq_row + (k0 >> 1));
        wsb = ws_row[k0 >> 4];
    };
    auto commit = [&](int buf) {
        uint16_t *pa = sa + buf * PA_STAGE + xr * PPITCH + xc, *pb = sb + buf * PB_STAGE;
        *reinterpret_cast<uint4 *>(pa) = xp0;
        *reinterpret_cast<uint4 *>(pa + 64 * PPITCH) = xp1;
        *reinterpret_cast<uint4 *>(pa + 128 * PPITCH) = xp2;
        *reinterpret_cast<uint4 *>(pa + 192 * PPITCH) = xp3;
        const float sc = QERL_E4M3_F32(wsb, 0);
        const f32x2_t f0 = QERL_FP4_PAIR_F32(wq.x, 0), f1 = QERL_FP4_PAIR_F32(wq.x, 1);
        const f32x2_t f2 = QERL_FP4_PAIR_F32(wq.x, 2), f3 = QERL_FP4_PAIR_F32(wq.x, 3);
        const f32x2_t f4 = QERL_FP4_PAIR_F32(wq.y, 0), f5 = QERL_FP4_PAIR_F32(wq.y, 1);
        const f32x2_t f6 = QERL_FP4_PAIR_F32(wq.y, 2), f7 = QERL_FP4_PAIR_F32(wq.y, 3);
        *reinterpret_cast<uint4 *>(pb + wr * PPITCH + wc) =
            make_uint4(pack_bf16x2(f0.x * sc, f0.y * sc), pack_bf16x2(f1.x * sc, f1.y * sc),
                       pack_bf16x2(f2.x * sc, f2.y * sc), pack_bf16x2(f3.x * sc, f3.y * sc));
        *reinterpret_cast<uint4 *>(pb + wr * PPITCH + wc + 8) =
            make_uint4(pack_bf16x2(f4.x * sc, f4.y * sc), pack_bf16x2(f5.x * sc, f5.y * sc),
                       pack_bf16x2(f6.x * sc, f6.y * sc), pack_bf16x2(f7.x * sc, f7.y * sc));
    };
    if (fast_steps > 0) {
        issue(0);
        commit(0);
        __syncthreads();
        for (int64_t s = 0; s < fast_steps; ++s) {
            const int buf = (int)(s & 1);
            if (s + 1 < fast_steps) issue(s + 1);  // uniform
            mma_step(buf);
            if (s + 1 < fast_steps) commit(buf ^ 1);
            __syncthreads();
        }
    }
    // ---- the rest: a partial last K step and the LoRA columns, one buffer ----
    for (int64_t s = fast_steps; s < steps; ++s) {
        const int64_t k0 = s * PBK;
        uint4 lo, hi;
        w_piece_ext(a, n0 + wr, k0 + wc, klora, lo, hi);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<uint4 *>(sa + (xr + 64 * u) * PPITCH + xc) = x_piece_ext(g, m0 + xr + 64 * u, k0 + xc, klora);
        *reinterpret_cast<uint4 *>(sb + wr * PPITCH + wc) = lo;
        *reinterpret_cast<uint4 *>(sb + wr * PPITCH + wc + 8) = hi;
        __syncthreads();
        mma_step(0);
        __syncthreads();
    }
    const float st_scale = *a.tensor_scale;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + wm * 128 + 16 * i + 4 * lq + v;
                const int64_t n = n0 + wn * 64 + 16 * j + lr;
                if (m < a.m && n < a.n) a.y[m * a.ldy + n] = f32_to_bf16_bits(st_scale * acc[i][j][v]);
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
    const int64_t tiles = ((a.n + PBN - 1) / PBN) * ((a.m + PBM - 1) / PBM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)(2 * PA_STAGE + 2 * PB_STAGE) * 2;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)tiles), dim3(256), lds, stream, g);
    return hipGetLastError();
}

}  // namespace qerl
