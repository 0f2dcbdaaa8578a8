// backward.hip -- backward of the W4A16 + LoRA layer for gfx950.
//
// The update phase trains the low-rank matrices with the NVFP4 base frozen
// ("QeRL: NVFP4-Quantized Reinforcement Learning -- Redefining Efficiency in
// AI Training and Inference", "LoRA (Low-Rank Adaptation)").  For
//   y = x what^T + lambda (x A^T) B^T,   t = x A^T,   g = dy B   ([M, r])
// the gradients are
//   dx = dy what + lambda g A   [M, K]  BF16   dx_kernel
//   dA = lambda g^T x           [r, K]  FP32   mprod_kernel
//   dB = lambda dy^T t          [N, r]  FP32   mprod_kernel
//
// dx contracts over N, along which the packed weight is strided: a workgroup
// owns a 128 x 128 tile of dx and walks N in steps of 64 rows, decoding each
// 64 x 128 weight block (exact BF16 e2m1 * e4m3) into LDS transposed, so that
// every MFMA B fragment (8 consecutive n of one column) is one 16-byte LDS
// read; the tile is double-buffered (the next block is decoded while this
// one multiplies), one barrier per step.  The LoRA term continues the same accumulation: the ranks act as 2r
// more rows, A as their weights and g * lambda / s_t split into BF16 hi + lo
// as their activations; s_t is applied once at the end.
//
// t and g (contractions over K and N, both operands contiguous along them,
// B transposed first) and dA, dB (contractions over M, along which x and dy
// are strided: transposed LDS tiles, the FP32 side as BF16 hi + lo) run on the
// MFMA over chunks of the contraction; the chunks' partial sums are added in
// chunk order.
#include "device_common.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;

// out[p * osp + j * osj] = scale * sum over chunks (in order) of part[c][p][j]
__global__ __launch_bounds__(kThreads) void chunk_reduce_kernel(const float *part, int64_t chunks, int64_t P, int r,
                                                                 float scale, float *out, int64_t osp, int64_t osj) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= P * r) return;
    const int64_t p = i / r, j = i - p * r;
    float acc = 0.0f;
    for (int64_t c = 0; c < chunks; ++c) acc += part[c * P * r + i];
    out[p * osp + j * osj] = scale * acc;
}

// ---- rank products on the MFMA: part[c][i][j] = sum over q in chunk c of
// L[i][q] R[j][q], with both L [M, Q] and R [r, Q] contiguous along q (t = x A^T
// with R = A; g = dy B with R = B^T formed first).  A workgroup takes 16 rows
// of L and every rank; its 4 waves take interleaved 32-column steps of the
// chunk and their tiles are summed in wave order through LDS.
constexpr int kRpChunk = 1024;
__device__ __forceinline__ bf16x8_t as_bf16x8_b(const uint4 &u) {
    bf16x8_t v;
    __builtin_memcpy(&v, &u, 16);
    return v;
}
struct RankProd {
    const uint16_t *L;
    int64_t ldl;
    const uint16_t *R;
    int64_t ldr;
    int64_t M, Q;
    int r;
    float *part;  // [chunks][M][r]
};

// 8 BF16 of row `row` at columns q .. q + 7 (zeros past rows or Q)
__device__ __forceinline__ uint4 load_row8(const uint16_t *base, int64_t ld, int64_t rows, int64_t row, int64_t Q,
                                           int64_t q) {
    if (row >= rows || q >= Q) return make_uint4(0, 0, 0, 0);
    const uint16_t *p = base + row * ld + q;
    if (q + 8 <= Q && (ld & 7) == 0) return *reinterpret_cast<const uint4 *>(p);
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = q + i < Q ? p[i] : (uint16_t)0;
    uint4 v;
    __builtin_memcpy(&v, e, 16);
    return v;
}

__global__ __launch_bounds__(kThreads) void rank_prod_kernel(RankProd a) {
    constexpr int JT = kMaxRankBwd / 16;
    __shared__ f32x4_t red[4][JT][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t i0 = (int64_t)blockIdx.x * 16, c = blockIdx.y;
    const int64_t q0 = c * kRpChunk, q1 = q0 + kRpChunk < a.Q ? q0 + kRpChunk : a.Q;
    const int jt_n = (a.r + 15) / 16;
    f32x4_t acc[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t q = q0 + 32 * wave; q < q1; q += 128) {
        const uint4 af = load_row8(a.L, a.ldl, a.M, i0 + lr, q1, q + 8 * lq);
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            if (j >= jt_n) break;  // (uniform)
            const uint4 bf = load_row8(a.R, a.ldr, a.r, 16 * j + lr, q1, q + 8 * lq);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_b(af), as_bf16x8_b(bf), acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < JT; ++j)
        if (j < jt_n) red[wave][j][lane] = acc[j];
    __syncthreads();
    // tile j, lane l: rows 4 (l / 16) + v, rank 16 j + l % 16; one wave per tile group
    for (int j = wave; j < jt_n; j += 4) {
        f32x4_t t = red[0][j][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) t = t + red[w][j][lane];
        const int64_t jj = 16 * j + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = i0 + 4 * lq + v;
            if (i < a.M && jj < a.r) a.part[(c * a.M + i) * a.r + jj] = t[v];
        }
    }
}

// ---- products over M on the MFMA: part[c][p][j] = sum over m in chunk c of
// X[m][p] Y[m][j], X BF16 [M, P] (row stride ldx), Y FP32 [M, r] (dA with
// X = x, Y = g; dB with X = dy, Y = t).  Both are strided along M, the
// contraction: each 32-row step stages X's 128 columns and Y transposed into
// LDS (Y as BF16 hi + lo, two MFMAs), so every fragment is one 16-byte read.
// A workgroup covers 128 values of p x every rank over one chunk of M.
constexpr int kMpChunk = 512, kMpP = 128, kMpStep = 32;
constexpr int kMpPitch = kMpStep + 8;  // BF16 per transposed LDS row
struct MProd {
    const uint16_t *X;
    int64_t ldx;
    const float *Y;
    int64_t M, P;
    int r;
    float *part;  // [chunks][P][r]
};

__global__ __launch_bounds__(kThreads) void mprod_kernel(MProd a) {
    constexpr int JT = kMaxRankBwd / 16;
    __shared__ __attribute__((aligned(16))) uint16_t xt[kMpP * kMpPitch];           // [p][m]
    __shared__ __attribute__((aligned(16))) uint16_t yt[2][kMaxRankBwd * kMpPitch];  // hi, lo: [j][m]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t p0 = (int64_t)blockIdx.x * kMpP, c = blockIdx.y;
    const int64_t m0 = c * kMpChunk, m1 = m0 + kMpChunk < a.M ? m0 + kMpChunk : a.M;
    const int jt_n = (a.r + 15) / 16;
    // wave w: p-tiles 2 w, 2 w + 1 x every rank tile
    f32x4_t acc[2][JT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t ms = m0; ms < m1; ms += kMpStep) {
        __syncthreads();  // the previous step's tiles have been read
        // X rows ms .. ms + 31, columns p0 .. p0 + 127 -> xt[p][m]: a thread
        // takes one row and 16 columns (two 8-column loads)
        {
            const int ml = tid >> 3, pc = 16 * (tid & 7);
            const int64_t mm = ms + ml;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t pp = p0 + pc + 8 * h;
                uint16_t e[8];
                if (mm < m1 && pp + 8 <= a.P && (a.ldx & 7) == 0) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(a.X + mm * a.ldx + pp);
                    __builtin_memcpy(e, &v, 16);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) e[i] = (mm < m1 && pp + i < a.P) ? a.X[mm * a.ldx + pp + i] : (uint16_t)0;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) xt[(pc + 8 * h + i) * kMpPitch + ml] = e[i];
            }
        }
        // Y rows ms .. ms + 31, all ranks -> yt[hi/lo][j][m]
        for (int e = tid; e < kMpStep * a.r; e += kThreads) {
            const int ml = e / a.r, j = e - ml * a.r;
            const int64_t mm = ms + ml;
            const float v = mm < m1 ? a.Y[mm * a.r + j] : 0.0f;
            const uint16_t hi = f32_to_bf16_bits(v);
            yt[0][j * kMpPitch + ml] = hi;
            yt[1][j * kMpPitch + ml] = f32_to_bf16_bits(v - __uint_as_float((uint32_t)hi << 16));
        }
        // ranks past r (to the tile edge) are zero
        for (int e = tid; e < kMpStep * (16 * jt_n - a.r); e += kThreads) {
            const int ml = e % kMpStep, j = a.r + e / kMpStep;
            yt[0][j * kMpPitch + ml] = 0;
            yt[1][j * kMpPitch + ml] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(xt + (32 * wave + 16 * i + lr) * kMpPitch + 8 * lq);
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                if (j >= jt_n) break;  // (uniform)
                const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(yt[0] + (16 * j + lr) * kMpPitch + 8 * lq);
                const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(yt[1] + (16 * j + lr) * kMpPitch + 8 * lq);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[i][j], 0, 0, 0);
            }
        }
    }
    // tile (i, j), lane l: p = p0 + 32 w + 16 i + 4 (l / 16) + v, rank 16 j + l % 16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            if (j >= jt_n) break;
            const int64_t jj = 16 * j + lr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t pp = p0 + 32 * wave + 16 * i + 4 * lq + v;
                if (pp < a.P && jj < a.r) a.part[(c * a.P + pp) * a.r + jj] = acc[i][j][v];
            }
        }
}

// B [n, r] -> B^T [r, ldt] (BF16, rows padded to ldt >= n with zeros)
__global__ __launch_bounds__(kThreads) void transpose_b_kernel(const uint16_t *b, int64_t n, int r, uint16_t *bt,
                                                               int64_t ldt) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (int64_t)r * ldt) return;
    const int64_t j = i / ldt, nn = i - j * ldt;
    bt[i] = nn < n ? b[nn * r + j] : (uint16_t)0;
}

// ---- dx = dy what + lambda g A ---------------------------------------------
constexpr int kMT = 8;  // 16-row m-tiles per workgroup
constexpr int kBM = 16 * kMT, kBK = 128, kBN = 64;  // dx tile (rows x columns), N per step
constexpr int kTPitch = kBN + 8;  // BF16 elements per transposed LDS row (16-byte aligned rows)
// element offset of transposed row kk: the four column segments a wave writes
// at once lie 32 rows apart, and 32 pitches are a whole number of bank
// rounds, so each 32-row group is skewed by 8 more dwords (a fragment read
// stays inside one group); 3.03 -> 2.99 ms on the 7B backward
constexpr int kTSkew = 16;
__device__ __forceinline__ int trow(int kk) { return kk * kTPitch + (kk >> 5) * kTSkew; }
constexpr int kTTile = kBK * kTPitch + (kBK / 32 - 1) * kTSkew;  // elements of one buffer

struct DxArgs {
    const uint16_t *dy;
    int64_t m, n, ldy;
    const uint8_t *packed;
    const uint8_t *scales;
    const float *tensor_scale;
    int64_t k;
    const uint16_t *lora_a;
    int r;
    float lora_scale;
    const float *g;  // [m, r] FP32
    uint16_t *dx;
    int64_t lddx;
};

// 8 BF16 of dy row `row`, columns c0 .. c0 + 7 (zeros past m or n)
__device__ __forceinline__ uint4 load_dy8(const DxArgs &a, int64_t row, int64_t c0) {
    if (row >= a.m || c0 >= a.n) return make_uint4(0, 0, 0, 0);
    const uint16_t *p = a.dy + row * a.ldy + c0;
    if (c0 + 8 <= a.n && (a.ldy & 7) == 0) return *reinterpret_cast<const uint4 *>(p);
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = c0 + i < a.n ? p[i] : (uint16_t)0;
    uint4 v;
    __builtin_memcpy(&v, e, 16);
    return v;
}

// The 32 weights of row nrow, columns kcol .. kcol + 31 (two 16-blocks), as
// packed bytes and their two scale bytes (zeros past n or k)
struct WPiece {
    uint4 q;
    uint32_t s0, s1;
};
__device__ __forceinline__ WPiece load_wpiece(const DxArgs &a, int64_t nrow, int64_t kcol) {
    WPiece w{make_uint4(0, 0, 0, 0), 0, 0};
    if (nrow < a.n && kcol < a.k) {
        const uint8_t *pr = a.packed + nrow * (a.k >> 1) + (kcol >> 1);
        const uint8_t *sr = a.scales + nrow * (a.k >> 4) + (kcol >> 4);
        // rows start 8-byte aligned (k % 16 == 0), 16-byte aligned when k % 32 == 0
        const uint2 h0 = *reinterpret_cast<const uint2 *>(pr);
        w.q.x = h0.x;
        w.q.y = h0.y;
        w.s0 = sr[0];
        if (kcol + 32 <= a.k) {  // (else the last 16-block of a row with k % 32 == 16)
            const uint2 h1 = reinterpret_cast<const uint2 *>(pr)[1];
            w.q.z = h1.x;
            w.q.w = h1.y;
            w.s1 = sr[1];
        }
    }
    return w;
}

// decode (exact BF16 e2m1 * e4m3) and store transposed: column kl + e of the
// tile gets row nl
__device__ __forceinline__ void store_wpiece(uint16_t *t, const WPiece &w, int nl, int kl) {
    const float s0 = QERL_E4M3_F32(w.s0, 0), s1 = QERL_E4M3_F32(w.s1, 0);
    const uint32_t qq[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float sc = h < 2 ? s0 : s1;
        const f32x2_t f0 = QERL_FP4_PAIR_F32(qq[h], 0), f1 = QERL_FP4_PAIR_F32(qq[h], 1);
        const f32x2_t f2 = QERL_FP4_PAIR_F32(qq[h], 2), f3 = QERL_FP4_PAIR_F32(qq[h], 3);
        const float v[8] = {f0.x, f0.y, f1.x, f1.y, f2.x, f2.y, f3.x, f3.y};
#pragma unroll
        for (int e = 0; e < 8; ++e) t[trow(kl + 8 * h + e) + nl] = f32_to_bf16_bits(v[e] * sc);
    }
}

__global__ __launch_bounds__(kThreads) void dx_kernel(DxArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tt[2][kTTile];  // tile^T: [kk][n], double-buffered
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t i0 = (int64_t)blockIdx.y * kBM, kk0 = (int64_t)blockIdx.x * kBK;
    // wave w: m-tiles kMW w .. kMW w + kMW - 1 (its own dy rows) x all 8 column tiles
    constexpr int kMW = kMT / 4, kNT = kBK / 16;
    f32x4_t acc[kMW][kNT];
#pragma unroll
    for (int i = 0; i < kMW; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // a thread's decode share per step: weight row nl (of 64), 32 columns at 32 seg
    const int nl = tid >> 2, seg = tid & 3;
    const int64_t kcol = kk0 + 32 * seg;
    auto mfma_k32 = [&](const uint16_t *t, int koff, const uint4 (&af)[kMW]) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(t + trow(16 * j + lr) + koff + 8 * lq);
#pragma unroll
            for (int i = 0; i < kMW; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_b(af[i]), b, acc[i][j], 0, 0, 0);
        }
    };
    const int64_t mrow0 = i0 + 16 * kMW * wave;  // this wave's first dy row
    const int64_t steps = (a.n + kBN - 1) / kBN;
    if (steps > 0) {
        store_wpiece(tt[0], load_wpiece(a, nl, kcol), nl, 32 * seg);
        __syncthreads();
    }
    for (int64_t s = 0; s < steps; ++s) {
        const int64_t n0 = s * kBN;
        // A fragments of this step (dy rows i0 + 16 i + lr, two 32-column halves)
        // and the next step's weights, all issued before the products
        uint4 af[2][kMW];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < kMW; ++i) af[h][i] = load_dy8(a, mrow0 + 16 * i + lr, n0 + 32 * h + 8 * lq);
        const bool more = s + 1 < steps;
        WPiece nxt{make_uint4(0, 0, 0, 0), 0, 0};
        if (more) nxt = load_wpiece(a, n0 + kBN + nl, kcol);
        const uint16_t *cur = tt[s & 1];
        mfma_k32(cur, 0, af[0]);
        mfma_k32(cur, 32, af[1]);
        if (more) store_wpiece(tt[(s + 1) & 1], nxt, nl, 32 * seg);
        __syncthreads();  // next tile written; this one read by every wave
    }
    // LoRA: ranks as 2r more rows (hi, lo) with weights A and activations
    // g * lambda / s_t, 64 ranks per step (rows of the tile past r are zero)
    const float st = *a.tensor_scale;
    const float gs = a.lora_scale / st;
    // lambda / s_t finite and moderate: the ranks ride in the accumulation;
    // else (tiny s_t) the epilogue adds lambda sum_j g[i, j] A[j, kk] itself
    const bool fold = __builtin_isfinite(gs) && __builtin_fabsf(gs) <= 0x1p64f;  // (uniform)
    for (int64_t j0 = 0; fold && j0 < a.r; j0 += kBN) {
        // A row j0 + nl, 32 columns at kcol (BF16 as it is), transposed into the tile
        uint4 av[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                       make_uint4(0, 0, 0, 0)};
        if (j0 + nl < a.r && kcol < a.k) {
            const uint4 *pa = reinterpret_cast<const uint4 *>(a.lora_a + (j0 + nl) * a.k + kcol);
            av[0] = pa[0];
            av[1] = pa[1];
            if (kcol + 32 <= a.k) {
                av[2] = pa[2];
                av[3] = pa[3];
            }
        }
        uint16_t *t = tt[0];
        const uint32_t aw[16] = {av[0].x, av[0].y, av[0].z, av[0].w, av[1].x, av[1].y, av[1].z, av[1].w,
                                 av[2].x, av[2].y, av[2].z, av[2].w, av[3].x, av[3].y, av[3].z, av[3].w};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            t[trow(32 * seg + 2 * e) + nl] = (uint16_t)(aw[e] & 0xFFFFu);
            t[trow(32 * seg + 2 * e + 1) + nl] = (uint16_t)(aw[e] >> 16);
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 ah[kMW], al[kMW];
#pragma unroll
            for (int i = 0; i < kMW; ++i) {
                const int64_t row = mrow0 + 16 * i + lr;
                float gv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t j = j0 + 32 * h + 8 * lq + e;
                    gv[e] = (row < a.m && j < a.r) ? a.g[row * a.r + j] * gs : 0.0f;
                }
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hw[e] = pack_bf16x2(gv[2 * e], gv[2 * e + 1]);
                    lw[e] = pack_bf16x2(gv[2 * e] - bf16lo_to_f32(hw[e]), gv[2 * e + 1] - bf16hi_to_f32(hw[e]));
                }
                ah[i] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                al[i] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            }
            mfma_k32(t, 32 * h, ah);
            mfma_k32(t, 32 * h, al);
        }
        __syncthreads();  // the tile is read before the next ranks overwrite it
    }
    // dx[i][kk] = bf16(s_t * acc): lane holds rows 4 lq + v of column lr
#pragma unroll
    for (int i = 0; i < kMW; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = mrow0 + 16 * i + 4 * lq + v, col = kk0 + 16 * j + lr;
                if (row < a.m && col < a.k) {
                    float d = st * acc[i][j][v];
                    if (!fold) {
                        float l = 0.0f;
                        for (int jr = 0; jr < a.r; ++jr)
                            l = __builtin_fmaf(a.g[row * a.r + jr], bf16lo_to_f32(a.lora_a[jr * a.k + col]), l);
                        d = __builtin_fmaf(a.lora_scale, l, d);
                    }
                    a.dx[row * a.lddx + col] = f32_to_bf16_bits(d);
                }
            }
}

}  // namespace

size_t backward_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    // t and g [m, r], then the largest chunk partials (one product at a time)
    int64_t part = 0;
    const int64_t rp_k = (k + kRpChunk - 1) / kRpChunk, rp_n = (n + kRpChunk - 1) / kRpChunk;
    const int64_t mp = (m + kMpChunk - 1) / kMpChunk;
    const int64_t cand[4] = {rp_k * m * r, rp_n * m * r, mp * k * r, mp * n * r};
    for (int64_t c : cand) part = c > part ? c : part;
    const int64_t ldt = (n + 7) / 8 * 8;  // B^T rows, 16-byte aligned
    return (size_t)(2 * m * r + part) * 4 + (size_t)(r * ldt) * 2 + 512;
}

hipError_t launch_backward(const BackwardArgs &b, hipStream_t stream) {
    float *t = static_cast<float *>(b.workspace);
    float *g = t + b.m * b.r;
    float *part = g + b.m * b.r;
    hipError_t e = hipSuccess;
    if (b.r > 0) {
        int64_t part_floats = 0;
        {
            const int64_t rp_k = (b.k + kRpChunk - 1) / kRpChunk, rp_n = (b.n + kRpChunk - 1) / kRpChunk;
            const int64_t mp = (b.m + kMpChunk - 1) / kMpChunk;
            const int64_t cand[4] = {rp_k * b.m * b.r, rp_n * b.m * b.r, mp * b.k * b.r, mp * b.n * b.r};
            for (int64_t c : cand) part_floats = c > part_floats ? c : part_floats;
        }
        const int64_t ldt = (b.n + 7) / 8 * 8;
        // B^T after t, g and the partials, 256-byte aligned from the (16-byte aligned) workspace
        uint16_t *bt = reinterpret_cast<uint16_t *>(static_cast<char *>(b.workspace) +
                                                    (((2 * b.m * b.r + part_floats) * 4 + 255) & ~(int64_t)255));
        auto rank_prod = [&](const uint16_t *L, int64_t ldl, const uint16_t *R, int64_t ldr, int64_t Q, float *out) {
            const int64_t chunks = (Q + kRpChunk - 1) / kRpChunk;
            hipLaunchKernelGGL(rank_prod_kernel, dim3((unsigned)((b.m + 15) / 16), (unsigned)chunks), dim3(kThreads),
                               0, stream, RankProd{L, ldl, R, ldr, b.m, Q, b.r, part});
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            const int64_t total = b.m * b.r;
            hipLaunchKernelGGL(chunk_reduce_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                               dim3(kThreads), 0, stream, part, chunks, b.m, b.r, 1.0f, out, (int64_t)b.r, (int64_t)1);
            return hipGetLastError();
        };
        // t = x A^T (A rows contiguous along k)
        e = rank_prod(b.x, b.ldx, b.lora_a, b.k, b.k, t);
        if (e != hipSuccess) return e;
        // g = dy B = dy (B^T)^T: B^T formed first, rows padded to a multiple of 8
        hipLaunchKernelGGL(transpose_b_kernel, dim3((unsigned)((b.r * ldt + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, b.lora_b, b.n, b.r, bt, ldt);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = rank_prod(b.dy, b.ldy, bt, ldt, b.n, g);
        if (e != hipSuccess) return e;
        auto mprod = [&](const uint16_t *X, int64_t ldx, const float *Y, int64_t P, float *out, int64_t osp,
                         int64_t osj) {
            const int64_t chunks = (b.m + kMpChunk - 1) / kMpChunk;
            hipLaunchKernelGGL(mprod_kernel, dim3((unsigned)((P + kMpP - 1) / kMpP), (unsigned)chunks),
                               dim3(kThreads), 0, stream, MProd{X, ldx, Y, b.m, P, b.r, part});
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            const int64_t total = P * b.r;
            hipLaunchKernelGGL(chunk_reduce_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                               dim3(kThreads), 0, stream, part, chunks, P, b.r, b.lora_scale, out, osp, osj);
            return hipGetLastError();
        };
        if (b.da) {  // dA[j][kk] = lambda sum_i x[i][kk] g[i][j]
            e = mprod(b.x, b.ldx, g, b.k, b.da, 1, b.k);
            if (e != hipSuccess) return e;
        }
        if (b.db) {  // dB[n][j] = lambda sum_i dy[i][n] t[i][j]
            e = mprod(b.dy, b.ldy, t, b.n, b.db, b.r, 1);
            if (e != hipSuccess) return e;
        }
    }
    if (b.dx) {
        const DxArgs d{b.dy, b.m, b.n, b.ldy, b.packed, b.scales, b.tensor_scale, b.k, b.lora_a, b.r, b.lora_scale,
                       g, b.dx, b.lddx};
        const dim3 grid((unsigned)((b.k + kBK - 1) / kBK), (unsigned)((b.m + kBM - 1) / kBM));
        hipLaunchKernelGGL(dx_kernel, grid, dim3(kThreads), 0, stream, d);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace qerl
