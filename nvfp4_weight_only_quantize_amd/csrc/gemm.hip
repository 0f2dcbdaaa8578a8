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
// Launch plan and workspace layout
// ---------------------------------------------------------------------------
enum Path { kGemv = 0, kSkinny = 1, kTiled = 2 };
enum LoraOut { kLoraF32 = 0, kLoraSplitBf16 = 1 };

constexpr int64_t kGemvMaxM = 4;
constexpr int64_t kSkinnyMaxM = 64;
constexpr int64_t kChunk = 128;          // K elements per skinny-kernel chunk

// Everything a GEMM kernel needs beyond the caller's arguments.  The plan is a
// pure function of (m, n, k, r), so the workspace size query and the launch
// always agree.
struct Plan {
    int path;
    int mt, nw, waves;          // skinny: 16-row m-tiles, 16-column groups, waves per workgroup
    int64_t tiles;              // skinny: workgroups (column tiles)
    int64_t t_off, bytes;
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

Plan make_plan(int64_t m, int64_t n, int64_t k, int r) {
    Plan p{};
    if (m <= kGemvMaxM && k % 32 == 0) p.path = kGemv;
    else if (m <= kSkinnyMaxM) p.path = kSkinny;
    else p.path = kTiled;
    p.t_off = 0;
    p.bytes = align256(m * (int64_t)r * 4);  // FP32 t [m, r] or BF16 hi/lo t [m, 2r]
    if (p.path == kSkinny) {
        p.mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
        p.nw = p.mt;                      // x fragments reused over nw column groups
        p.waves = p.mt == 1 ? 16 : 8;     // waves splitting K inside the workgroup
        p.tiles = (n + 16 * p.nw - 1) / (16 * p.nw);
    }
    return p;
}

struct Gemm {
    GemmArgs a;
    Plan p;
    __device__ float *t32() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.t_off); }
    __device__ uint16_t *t16() const { return reinterpret_cast<uint16_t *>(static_cast<char *>(a.workspace) + p.t_off); }
};

// ---------------------------------------------------------------------------
// Prologue: LoRA down-projection t = x A^T
// ---------------------------------------------------------------------------
// One workgroup per (row m, rank j); its 256 lanes split K (16 bytes per lane
// per step, four steps in flight).  Output:
//   kLoraF32:       t32[m * r + j] = t
//   kLoraSplitBf16: t16[m * 2r + j] = bf16(u), t16[m * 2r + r + j] = bf16(u - bf16(u)),
//                   with u = t * lora_scale / s_t
template <int MODE>
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
        if (MODE == kLoraF32) {
            g.t32()[m * a.r + j] = t;
        } else {
            const float u = t * (a.lora_scale / *a.tensor_scale);
            const uint16_t hi = f32_to_bf16_bits(u);
            const uint16_t lo = f32_to_bf16_bits(u - __uint_as_float((uint32_t)hi << 16));
            uint16_t *t16 = g.t16();
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
__global__ __launch_bounds__(kThreads) void gemv_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    constexpr int kGroups = kThreads / LPR;
    const int sub = threadIdx.x % LPR;
    const int group = threadIdx.x / LPR;
    const int64_t chunks = a.k >> 5;
    const float st = *a.tensor_scale;
    const float *t32 = g.t32();
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

// ---------------------------------------------------------------------------
// Skinny MFMA path (4 < m <= 64): split-K, weights streamed once
// ---------------------------------------------------------------------------
// Workgroup = 4 waves on the same 16*NW weight rows and the same K slice; wave
// w takes the slice's 128-element chunks w, w+4, ...  Lane (lr = lane%16,
// lq = lane/16) owns row n0 + 16g + lr of column group g and elements
// 32lq .. 32lq+31 of a chunk: 16 packed bytes and 2 scale bytes, prefetched
// one chunk ahead.  Step j of a chunk feeds elements 32lq + 8j .. +8 of the
// weights (B operand) and of the x rows (A operand) to one 16x16x32 MFMA per
// (m-tile, column group): the K order inside a chunk is permuted the same way
// on both operands, which leaves the dot products unchanged.  Weights are
// dequantized to BF16 as e2m1 * e4m3 (exact); s_t is applied in the epilogue.
// The LoRA product rides along as 2r extra K columns (t split into BF16 hi/lo,
// pre-scaled by lora_scale / s_t, against B repeated twice) in the last slice.
// Split-K partials go to the workspace; the last workgroup to arrive at a
// column tile (atomic counter, no waiting) sums them in slice order and writes y.

__device__ __forceinline__ bf16x8_t dequant8(uint32_t q, float s) {
    const f32x2_t f0 = QERL_FP4_PAIR_F32(q, 0), f1 = QERL_FP4_PAIR_F32(q, 1);
    const f32x2_t f2 = QERL_FP4_PAIR_F32(q, 2), f3 = QERL_FP4_PAIR_F32(q, 3);
    const uint4 o = make_uint4(pack_bf16x2(f0.x * s, f0.y * s), pack_bf16x2(f1.x * s, f1.y * s),
                               pack_bf16x2(f2.x * s, f2.y * s), pack_bf16x2(f3.x * s, f3.y * s));
    bf16x8_t v;
    __builtin_memcpy(&v, &o, 16);
    return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &u) {
    bf16x8_t v;
    __builtin_memcpy(&v, &u, 16);
    return v;
}

template <int NW>
__device__ __forceinline__ void load_w_chunk(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq,
                                             uint4 (&w)[NW], uint32_t (&sc)[NW]) {
    const int64_t e0 = c * kChunk + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        const int64_t n = n0 + 16 * g + lr;
        w[g] = make_uint4(0, 0, 0, 0);
        sc[g] = 0;
        if (n < a.n && e0 < a.k) {
            const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
            const uint8_t *srow = a.scales + n * (a.k >> 4) + (e0 >> 4);
            if (e0 + 32 <= a.k) {
                if ((a.k & 31) == 0) {
                    w[g] = *reinterpret_cast<const uint4 *>(prow);
                } else {  // rows are only 8-byte aligned
                    const uint2 lo = reinterpret_cast<const uint2 *>(prow)[0];
                    const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
                    w[g] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
                sc[g] = (uint32_t)srow[0] | ((uint32_t)srow[1] << 8);
            } else {  // k % 16 == 0: the last 16 elements of a row
                const uint2 lo = *reinterpret_cast<const uint2 *>(prow);
                w[g] = make_uint4(lo.x, lo.y, 0, 0);
                sc[g] = srow[0];
            }
        }
    }
}

// 8 BF16 values v(i), i < 8, with out-of-range entries zero
template <typename F>
__device__ __forceinline__ uint4 gather8(F v) {
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = v(i);
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

// Weights of one full chunk (all 32 elements of every lane in range): rows
// past n are clamped to the last row -- they only feed output columns that
// the epilogue discards -- so the loads need no branches.
template <int NW>
__device__ __forceinline__ void load_w_full(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq,
                                            uint4 (&w)[NW], uint32_t (&sc)[NW]) {
    const int64_t e0 = c * kChunk + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        int64_t n = n0 + 16 * g + lr;
        n = n < a.n ? n : a.n - 1;
        const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
        const uint8_t *srow = a.scales + n * (a.k >> 4) + (e0 >> 4);
        if ((a.k & 31) == 0) {
            w[g] = *reinterpret_cast<const uint4 *>(prow);
        } else {  // rows are only 8-byte aligned
            const uint2 lo = reinterpret_cast<const uint2 *>(prow)[0];
            const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
            w[g] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        sc[g] = (uint32_t)srow[0] | ((uint32_t)srow[1] << 8);
    }
}

template <int MT>
__device__ __forceinline__ void load_x_full(const GemmArgs &a, int64_t c, int lr, int lq, uint4 (&xa)[MT][4]) {
    const int64_t e0 = c * kChunk + 32 * lq;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int64_t m = 16 * mt + lr;
        m = m < a.m ? m : a.m - 1;  // rows past m feed discarded outputs only
        const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + m * a.ldx + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[mt][j] = xr[j];
    }
}

template <int MT, int NW>
__device__ __forceinline__ void mma_chunk(const uint4 (&w)[NW], const uint32_t (&sc)[NW],
                                          const uint4 (&xa)[MT][4], f32x4_t (&acc)[MT][NW]) {
    float sv[NW][2];
#pragma unroll
    for (int gi = 0; gi < NW; ++gi) {
        sv[gi][0] = QERL_E4M3_F32(sc[gi], 0);
        sv[gi][1] = QERL_E4M3_F32(sc[gi], 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int gi = 0; gi < NW; ++gi) {
            const uint32_t q = j == 0 ? w[gi].x : j == 1 ? w[gi].y : j == 2 ? w[gi].z : w[gi].w;
            const bf16x8_t b = dequant8(q, sv[gi][j >> 1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mt][j]), b, acc[mt][gi], 0, 0, 0);
        }
    }
}

template <int MT, int NW, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    constexpr int V = MT * NW * 4;  // accumulator floats per lane
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NW;
    const int64_t chunks = (a.k + kChunk - 1) / kChunk;
    const int64_t full_chunks = a.k / kChunk;

    f32x4_t acc[MT][NW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Full chunks, round-robin over the waves (at any moment the workgroup
    // streams WAVES consecutive 64-byte pieces of each of its rows).  Each wave
    // keeps DEPTH chunks in flight in a register ring: the weights and x of
    // chunk c + DEPTH*WAVES are issued together right after chunk c is consumed,
    // so the in-order wait for chunk c never waits for later chunks.  Chunk
    // indices past the end are clamped to a valid chunk (loaded, not used), so
    // every load is unconditional.
    {
        constexpr int DEPTH = 1;
        uint4 w[DEPTH][NW];
        uint32_t sc[DEPTH][NW];
        uint4 xa[DEPTH][MT][4];
        const int64_t last = full_chunks - 1;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (full_chunks == 0) break;
            int64_t c = wave + (int64_t)d * WAVES;
            c = c < last ? c : last;
            load_w_full<NW>(a, n0, c, lr, lq, w[d], sc[d]);
            load_x_full<MT>(a, c, lr, lq, xa[d]);
        }
        for (int64_t c0 = wave; c0 < full_chunks; c0 += (int64_t)DEPTH * WAVES) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int64_t c = c0 + (int64_t)d * WAVES;
                if (c < full_chunks) mma_chunk<MT, NW>(w[d], sc[d], xa[d], acc);
                int64_t cn = c + (int64_t)DEPTH * WAVES;
                if (cn < full_chunks + (int64_t)DEPTH * WAVES) {  // uniform: ring refill
                    cn = cn < last ? cn : last;
                    load_w_full<NW>(a, n0, cn, lr, lq, w[d], sc[d]);
                    load_x_full<MT>(a, cn, lr, lq, xa[d]);
                }
            }
        }
    }
    // the last, partial chunk of K (k % 128 != 0): guarded loads, zero fill
    if (chunks > full_chunks && full_chunks % WAVES == wave) {
        const int64_t c = full_chunks;
        uint4 w[NW];
        uint32_t sc[NW];
        load_w_chunk<NW>(a, n0, c, lr, lq, w, sc);
        const int64_t e0 = c * kChunk + 32 * lq;
        uint4 xa[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int64_t m = 16 * mt + lr;
            m = m < a.m ? m : a.m - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xa[mt][j] = e0 + 8 * j < a.k ? *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + e0 + 8 * j)
                                             : make_uint4(0, 0, 0, 0);
        }
        mma_chunk<MT, NW>(w, sc, xa, acc);
    }

    // LoRA columns: A = split t [m, 2r] (hi then lo), B = lora_b[n, j mod r];
    // taken by the waves after the one holding the last K chunk
    if (a.r > 0) {
        const int64_t klora = 2 * (int64_t)a.r;
        const int64_t lchunks = (klora + kChunk - 1) / kChunk;
        const uint16_t *t16 = g.t16();
        for (int64_t l = (wave - chunks % WAVES + WAVES) % WAVES; l < lchunks; l += WAVES) {
            const int64_t e0 = l * kChunk + 32 * lq;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t jj = e0 + 8 * j;  // lanes past 2r gather zeros: the MFMA needs every lane
                bf16x8_t b[NW];
#pragma unroll
                for (int gi = 0; gi < NW; ++gi) {
                    const int64_t n = n0 + 16 * gi + lr;
                    b[gi] = as_bf16x8(gather8([&](int i) -> uint32_t {
                        const int64_t col = jj + i;  // < 2r: col mod r is one conditional subtract
                        return (n < a.n && col < klora) ? a.lora_b[n * a.r + (col < a.r ? col : col - a.r)] : 0u;
                    }));
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int64_t m = 16 * mt + lr;
                    const bf16x8_t xv = as_bf16x8(gather8([&](int i) -> uint32_t {
                        return (m < a.m && jj + i < klora) ? t16[m * klora + jj + i] : 0u;
                    }));
#pragma unroll
                    for (int gi = 0; gi < NW; ++gi)
                        acc[mt][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, b[gi], acc[mt][gi], 0, 0, 0);
                }
            }
        }
    }

    // tree reduction of the waves' accumulators through LDS
    __shared__ float red[(WAVES / 2) * V * 64];
#pragma unroll
    for (int half = WAVES / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int gi = 0; gi < NW; ++gi)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[((wave - half) * V + (mt * NW + gi) * 4 + v) * 64 + lane] = acc[mt][gi][v];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int gi = 0; gi < NW; ++gi)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[mt][gi][v] += red[(wave * V + (mt * NW + gi) * 4 + v) * 64 + lane];
        }
        __syncthreads();
    }
    if (wave != 0) return;
    const float st = *a.tensor_scale;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int gi = 0; gi < NW; ++gi)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = 16 * mt + 4 * lq + v;
                const int64_t n = n0 + 16 * gi + lr;
                if (m < a.m && n < a.n) a.y[m * a.ldy + n] = f32_to_bf16_bits(st * acc[mt][gi][v]);
            }
}

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
hipError_t launch_gemv(const Gemm &g, hipStream_t stream) {
    // enough lanes per row that the grid covers the chip several times over
    const int64_t cus = num_cus();
    const int64_t target_waves = cus * 16;
    int lpr = 16;
    if (g.a.n * 16 / 64 < target_waves) lpr = 64;
    const int groups = kThreads / lpr;
    int64_t grid = (g.a.n + groups - 1) / groups;
    if (grid > cus * 64) grid = cus * 64;
    if (lpr == 64)
        hipLaunchKernelGGL((gemv_kernel<MT, 64>), dim3((unsigned)grid), dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL((gemv_kernel<MT, 16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
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
        if (g.p.path == kGemv)
            hipLaunchKernelGGL((prologue_kernel<kLoraF32>), dim3((unsigned)grid), dim3(kThreads), 0, stream, g);
        else
            hipLaunchKernelGGL((prologue_kernel<kLoraSplitBf16>), dim3((unsigned)grid), dim3(kThreads), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g.p.path == kGemv) {
        switch (a.m) {
            case 1: return launch_gemv<1>(g, stream);
            case 2: return launch_gemv<2>(g, stream);
            case 3: return launch_gemv<3>(g, stream);
            default: return launch_gemv<4>(g, stream);
        }
    }
    if (g.p.path == kSkinny) {
        if (g.p.tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)g.p.tiles);
        if (g.p.mt == 1)
            hipLaunchKernelGGL((skinny_kernel<1, 1, 16>), grid, dim3(16 * 64), 0, stream, g);
        else if (g.p.mt == 2)
            hipLaunchKernelGGL((skinny_kernel<2, 2, 8>), grid, dim3(8 * 64), 0, stream, g);
        else
            hipLaunchKernelGGL((skinny_kernel<4, 4, 8>), grid, dim3(8 * 64), 0, stream, g);
        return hipGetLastError();
    }
    const int64_t tiles = ((a.n + BN - 1) / BN) * ((a.m + BM - 1) / BM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(tiled_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

}  // namespace qerl
