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
// Larger m (m > 256; m <= 256 is the decode path of decode.hip):
//   prologue_kernel  t = x A^T in FP32 (MFMA, 16 rows of x per workgroup),
//                    pre-multiplied by lora_scale / s_t and split into BF16
//                    hi + lo halves, so that the LoRA product becomes 2r extra
//                    K columns of the same MFMA accumulation.
//   prefill_kernel   128 x 256 output tiles over the K loops of mfma_tile.h
//                    (x by LDS DMA, weights decoded to exact BF16 in
//                    registers, BF16 MFMA 16x16x32 with FP32 accumulation);
//                    s_t applied once; with K a multiple of 256 the scales
//                    arrive by LDS DMA, four blocks at a time.  Grids of few
//                    tiles split K (even block counts per split): every
//                    split stores its FP32 tile and the last to arrive at
//                    the tile sums them in split order and writes y, or
//   reduce_kernel    does, over the whole chip, when a tile has many splits.
#include <stdio.h>

#include "device_common.h"
#include "mfma_tile.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Launch plan and workspace layout
// ---------------------------------------------------------------------------
// The workspace holds the BF16 hi/lo t [m, 2r] (with the prologue's K-range
// partials of t when it splits K) and, when the main loop splits K, one
// counter per output tile and the FP32 partial tiles [splits][tiles][PBM PBN]
// in lane order.
#ifndef QERL_PF_WAVES
#define QERL_PF_WAVES 4
#endif
constexpr int kPfWaves = QERL_PF_WAVES;  // waves of a prefill workgroup, 64 weight rows each
constexpr int PBM = 128, PBN = 64 * kPfWaves;  // output tile: rows of x x weight rows
constexpr int64_t kPartTileBytes = (int64_t)PBM * PBN * 4;  // one split's FP32 tile
// below this many tiles (two resident workgroups per CU) K may be split: the
// split count is the one with the least modeled time, rounds of resident
// workgroups x (blocks per split + kSplitOverhead) plus the reduce's FP32
// traffic.  A grid of 256-511 tiles leaves a quarter to half of the slots idle
// (32B layer at M = 2048: q, o and down have 320 tiles and take three splits,
// two rounds); a count that spills a few workgroups into another round costs
// a whole round (k and v there: 64 tiles, seven splits in one round of 448
// workgroups rather than ten in two).
constexpr int64_t kSplitTiles = 512;
constexpr double kSplitOverhead = 2.0;     // per workgroup, in K blocks: x tile start, epilogue
constexpr double kReduceBytesPerBlock = 1.9e7;  // partial-tile bytes moved in the time of one K block
// where the splits of a tile meet: inside the launch, the last split reading
// every split's 128 KB tile alone (about kMeetUsPerSplit each), or in
// reduce_kernel over the whole chip (a launch plus the partial tiles' traffic)
constexpr double kMeetUsPerSplit = 2.0, kReduceLaunchUs = 4.0, kReduceBytesPerUs = 4.4e6;
constexpr int64_t kPrologueWgs = 512;  // below this many prologue workgroups its K is split
constexpr int64_t kMaxSplits = 16;

struct Plan {
    int64_t tiles, splits, bps;  // output tiles, K splits, 128-column blocks per split
    bool meet;                   // split K: the splits meet in the launch, else in reduce_kernel
    int64_t ksplit, kchunk;      // prologue: K ranges (FP32 partial t each when > 1), columns per range
    int64_t t_off, tpart_off, cnt_off, part_off, bytes;
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

Plan make_plan(int64_t m, int64_t n, int64_t k, int r) {
    Plan p{};
    p.tiles = ((m + PBM - 1) / PBM) * ((n + PBN - 1) / PBN);
    const int64_t blocks = k / 128;
    p.splits = 1;
    p.bps = blocks;
    if (p.tiles < kSplitTiles && blocks >= 8) {
        double best = 0.0;
        for (int64_t s = 1; s <= blocks / 4 && s <= kMaxSplits; ++s) {  // at least four blocks per split
            int64_t bps = (blocks + s - 1) / s;
            if (s > 1 && blocks % 2 == 0) bps += bps & 1;  // even split starts: aligned scale chunks
            const int64_t sp = (blocks + bps - 1) / bps;  // no empty split
            const int64_t rounds = (p.tiles * sp + kSplitTiles - 1) / kSplitTiles;
            const double t = (double)rounds * ((double)bps + kSplitOverhead) +
                             (sp > 1 ? (double)m * (double)n * (4.0 * (double)sp + 2.0) / kReduceBytesPerBlock : 0.0);
            if (s == 1 || t < best) {
                best = t;
                p.splits = sp;
                p.bps = bps;
            }
        }
    }
    // the prologue: one workgroup per 16 rows of x; with fewer than
    // kPrologueWgs of them, K is split too (ranges of at least 512 columns,
    // a multiple of 128) and t_reduce_kernel adds the ranges' FP32 partials
    const int64_t row_groups = (m + 15) / 16;
    p.ksplit = 1;
    p.kchunk = k;
    if (r > 0 && row_groups < kPrologueWgs) {
        int64_t ks = (2 * kPrologueWgs + row_groups - 1) / row_groups;
        if (ks > k / 512) ks = k / 512;
        if (ks > 1) {
            p.kchunk = ((k + ks - 1) / ks + 127) / 128 * 128;
            p.ksplit = (k + p.kchunk - 1) / p.kchunk;
        }
    }
    p.t_off = 0;
    p.tpart_off = align256(p.t_off + m * (int64_t)r * 4);
    p.meet = p.splits > 1 && (double)p.splits * kMeetUsPerSplit <
                                 kReduceLaunchUs + (double)m * (double)n * (4.0 * (double)p.splits + 2.0) / kReduceBytesPerUs;
    p.cnt_off = align256(p.tpart_off + (p.ksplit > 1 ? p.ksplit * m * (int64_t)r * 4 : 0));
    p.part_off = align256(p.cnt_off + (p.splits > 1 ? p.tiles * 4 : 0));
    p.bytes = p.part_off + (p.splits > 1 ? align256(p.splits * p.tiles * kPartTileBytes) : 0);
    return p;
}

struct Gemm {
    GemmArgs a;
    Plan p;
    __device__ uint16_t *t16() const { return reinterpret_cast<uint16_t *>(static_cast<char *>(a.workspace) + p.t_off); }
    __device__ float *part() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.part_off); }
    __device__ float *tpart() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.tpart_off); }
    __device__ uint32_t *cnt() const { return reinterpret_cast<uint32_t *>(static_cast<char *>(a.workspace) + p.cnt_off); }
};

// The K splits of one output tile meet inside the launch: each stores its FP32
// tile (lane order, 16 bytes a lane per MFMA tile) and adds one to the tile's
// counter; the split that brings it to `splits` sums the tiles in split order
// and writes y, and sets the counter back to zero.  No workgroup waits for
// another.  The splits may run on different XCDs, whose L2 caches are not
// coherent with each other, so the tiles and the counter use the SC1 cache
// policy (the agent-scope coherent accesses that relaxed agent-scope atomics
// compile to), and a split's stores have completed before it arrives.  The
// counters are cleared by the launch before (the prologue, or
// cnt_zero_kernel without LoRA), so nothing needs to be zero beforehand.
constexpr int kSC1 = 16;  // cache-policy operand of the buffer builtins: SC1

// The LoRA product rides in the MFMA accumulation as t * lora_scale / s_t,
// which needs that factor finite and moderate; for tiny s_t (a subnormal or
// a caller's tensor scale far below lora_scale) it is not, and then the
// prologue stores lora_scale * t in FP32 in the same region, the extra K
// columns read as zeros, and the epilogue adds sum_j (lora_scale t[m, j])
// B[n, j] to s_t * acc.  Every kernel decides the same way from the same two
// floats.
__device__ __forceinline__ bool lora_fold_ok(float lora_scale, float st) {
    const float mul = lora_scale / st;
    return __builtin_isfinite(mul) && __builtin_fabsf(mul) <= 0x1p64f;
}

// sum_j t32[m, j] B[n, j] in rank order (the unfolded LoRA term)
__device__ __forceinline__ float lora_term(const GemmArgs &a, const float *t32, int64_t m, int64_t n) {
    float s = 0.0f;
    for (int j = 0; j < a.r; ++j) s = __builtin_fmaf(t32[m * a.r + j], bf16lo_to_f32(a.lora_b[n * a.r + j]), s);
    return s;
}

// ---------------------------------------------------------------------------
// Prologue: LoRA down-projection t = x A^T
// ---------------------------------------------------------------------------
// One workgroup per 16 rows of x, all ranks: MFMA 16x16x32 with x as the A
// operand (lane l: row l % 16, columns 8 (l / 16) .. +8 of a 32-column step)
// and a 16-rank tile of the LoRA A matrix as the B operand, so tile j holds
// t[m0 + 4 (l / 16) + v][16 j + l % 16] in element v.  The four waves take
// interleaved 32-column steps, U at a time with every load issued before the
// products, and are summed in wave order through LDS.  x is read once; the
// LoRA A matrix is re-read per workgroup from L2.  Output, with
// u = t * lora_scale / s_t:
//   t16[m * 2r + j] = bf16(u), t16[m * 2r + r + j] = bf16(u - bf16(u))
// t[m, j] (FP32) into the region the main kernel reads: the BF16 hi/lo halves
// of t * lora_scale / s_t, or lora_scale * t in FP32 when that factor does
// not fold (fold and mul as lora_fold_ok and lora_scale / s_t give them)
__device__ __forceinline__ void store_t(const Gemm &g, int64_t m, int j, float t, bool fold, float mul) {
    const GemmArgs &a = g.a;
    uint16_t *t16 = g.t16();
    if (!fold) {
        reinterpret_cast<float *>(t16)[m * a.r + j] = t * a.lora_scale;
        return;
    }
    const float u = t * mul;
    const uint16_t hi = f32_to_bf16_bits(u);
    t16[m * 2 * a.r + j] = hi;
    t16[m * 2 * a.r + a.r + j] = f32_to_bf16_bits(u - __uint_as_float((uint32_t)hi << 16));
}

template <int JT>
__global__ __launch_bounds__(kThreads) void prologue_kernel(Gemm g) {
    constexpr int U = JT <= 4 ? 4 : 2;  // 32-column steps in flight per wave
    const GemmArgs &a = g.a;
    __shared__ f32x4_t red[4][JT][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    if (g.p.splits > 1 && blockIdx.x == 0 && blockIdx.y == 0)  // the split tiles' counters
        for (int64_t i = tid; i < g.p.tiles; i += kThreads)
            __hip_atomic_store(g.cnt() + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t row = m0 + lr < a.m ? m0 + lr : a.m - 1;  // rows past m: a repeat, not stored
    const uint16_t *xr = a.x + row * a.ldx;
    const uint16_t *ar[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        const int jr = 16 * j + lr;
        ar[j] = a.lora_a + (int64_t)(jr < a.r ? jr : a.r - 1) * a.k;  // ranks past r: zeroed below
    }
    f32x4_t acc[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // this workgroup's K range (all of K unless the plan splits it)
    const int64_t kbeg = (int64_t)blockIdx.y * g.p.kchunk;
    const int64_t kend = kbeg + g.p.kchunk < a.k ? kbeg + g.p.kchunk : a.k;
    for (int64_t k0 = kbeg + 32 * wave; k0 < kend; k0 += 128 * U) {
        uint4 xv[U], av[U][JT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kk = k0 + 128 * u + 8 * lq;
            const bool in = kk < kend;  // k % 16 == 0, kchunk % 128 == 0: a piece is inside or outside
            const int64_t kc = in ? kk : 0;
            xv[u] = *reinterpret_cast<const uint4 *>(xr + kc);
#pragma unroll
            for (int j = 0; j < JT; ++j) av[u][j] = *reinterpret_cast<const uint4 *>(ar[j] + kc);
            if (!in) {  // past k: zeros on both sides (kc = 0 only keeps the loads in bounds)
                xv[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < JT; ++j) av[u][j] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bf16x8_t xb;
            __builtin_memcpy(&xb, &xv[u], 16);
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                uint4 av_in = 16 * j + lr < a.r ? av[u][j] : make_uint4(0, 0, 0, 0);
                bf16x8_t ab;
                __builtin_memcpy(&ab, &av_in, 16);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, ab, acc[j], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < JT; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    if (wave != 0) return;
    const float mul = a.lora_scale / *a.tensor_scale;
    const bool fold = lora_fold_ok(a.lora_scale, *a.tensor_scale);  // (uniform)
    const bool split = g.p.ksplit > 1;                               // (uniform)
    float *tp = g.tpart() + (int64_t)blockIdx.y * a.m * a.r;        // this K range's partial t
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        const f32x4_t t = ((red[0][j][lane] + red[1][j][lane]) + red[2][j][lane]) + red[3][j][lane];
        const int jr = 16 * j + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + 4 * lq + v;
            if (m >= a.m || jr >= a.r) continue;
            if (split)
                tp[m * a.r + jr] = t[v];
            else
                store_t(g, m, jr, t[v], fold, mul);
        }
    }
}

// K split prologue: t[m, j] = the ranges' partials added in range order
__global__ __launch_bounds__(kThreads) void t_reduce_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.m * a.r) return;
    const float *tp = g.tpart();
    float t = 0.0f;
    for (int64_t s = 0; s < g.p.ksplit; ++s) t += tp[s * a.m * a.r + i];
    store_t(g, i / a.r, (int)(i % a.r), t, lora_fold_ok(a.lora_scale, *a.tensor_scale),
            a.lora_scale / *a.tensor_scale);
}

// ---------------------------------------------------------------------------
// MFMA path (m > 256)
// ---------------------------------------------------------------------------
// Workgroup tile 128 (rows of x) x 256 (weight rows): four waves side by
// side along n, each the full 128 x 64, so no weight fragment is fetched
// twice.  The main K loop is mfma_kloop (mfma_tile.h); what is left of K past
// the last full 128-column block, and the LoRA product as 2r extra K columns
// (t hi/lo x B twice), go through plain_kloop.
constexpr int kXTileBytes = PBM * kTileRowBytes;
#ifndef QERL_GROUP_M
#define QERL_GROUP_M 4
#endif
constexpr int64_t kGroupM = QERL_GROUP_M;  // row blocks per group of the tile order

__shared__ __attribute__((aligned(1024))) uint8_t g_xtile0[kXTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_xtile1[kXTileBytes];
// the workgroup's scale bytes of four blocks (64 kPfWaves rows x 32 bytes),
// two chunks (the main K loop's scales by DMA)
__shared__ __attribute__((aligned(1024))) uint8_t g_sctile0[64 * kPfWaves * 32];
__shared__ __attribute__((aligned(1024))) uint8_t g_sctile1[64 * kPfWaves * 32];

// 8 elements of the extended K range [0, k + 2r) for x row m at column kk:
// x itself, then the BF16 hi/lo halves of t * lora_scale / s_t; zero past
// the end and for rows past m.
__device__ __forceinline__ uint4 x_piece_ext(const Gemm &g, int64_t m, int64_t kk, int64_t klora, bool fold) {
    const GemmArgs &a = g.a;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (m >= a.m) return o;
    if (kk < a.k) return *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + kk);
    const int64_t j0 = kk - a.k;
    if (j0 >= klora || !fold) return o;
    const uint16_t *t16 = g.t16() + m * klora;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (j0 + i < klora) ? t16[j0 + i] : (uint16_t)0;
    __builtin_memcpy(&o, e, 16);
    return o;
}

// The 8 weights of row n at columns [kk, kk + 8) of the extended K range as
// BF16: dequantized NVFP4, then B [n, j] for j = column - k mod r; zero past
// the end and for rows past n.
__device__ __forceinline__ bf16x8_t w_frag_ext(const GemmArgs &a, int64_t n, int64_t kk, int64_t klora) {
    uint4 o = make_uint4(0, 0, 0, 0);
    if (n < a.n) {
        if (kk < a.k) {  // k % 16 == 0: an 8-element piece is inside or outside
            const uint32_t q = *reinterpret_cast<const uint32_t *>(a.packed + n * (a.k >> 1) + (kk >> 1));
            return dequant8_p(q, QERL_E4M3_F32(a.scales[n * (a.k >> 4) + (kk >> 4)], 0));
        }
        const int64_t j0 = kk - a.k;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t j = j0 + i;
            e[i] = j < klora ? a.lora_b[n * a.r + (j < a.r ? j : j - a.r)] : (uint16_t)0;
        }
        __builtin_memcpy(&o, e, 16);
    }
    bf16x8_t v;
    __builtin_memcpy(&v, &o, 16);
    return v;
}

template <bool SPLIT>
__global__ __launch_bounds__(64 * kPfWaves, 8 / kPfWaves) void prefill_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    // XCD-aware tile order: workgroup b runs on XCD b % 8 and each XCD takes
    // a contiguous range of the tile order.  That order walks groups of
    // kGroupM row blocks, n-major inside a group, so the tiles one XCD runs at
    // a time share kGroupM x slabs and a few weight slabs in its L2 rather
    // than one x slab and dozens of weight slabs.
    const int64_t tiles_n = (a.n + PBN - 1) / PBN, tiles_m = (a.m + PBM - 1) / PBM, tiles = tiles_n * tiles_m;
    const int64_t split = SPLIT ? (int64_t)blockIdx.x / tiles : 0;  // K split: blocks [split bps, +bps)
    const int64_t b = (int64_t)blockIdx.x - split * tiles, x8 = b % 8, q8 = tiles / 8, r8 = tiles % 8;
    const int64_t tile = x8 * q8 + (x8 < r8 ? x8 : r8) + b / 8;
    const int64_t grp = tile / (kGroupM * tiles_n), in_grp = tile % (kGroupM * tiles_n);
    const int64_t gm = tiles_m - grp * kGroupM < kGroupM ? tiles_m - grp * kGroupM : kGroupM;  // rows in this group
    const int64_t m0 = (grp * kGroupM + in_grp % gm) * PBM, n0 = (in_grp / gm) * PBN;
    const int64_t klora = 2 * (int64_t)a.r;
    const bool fold = a.r == 0 || lora_fold_ok(a.lora_scale, *a.tensor_scale);  // (uniform)

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const Plan &p = g.p;
    const bool last = !SPLIT || split == p.splits - 1;
    const int64_t blocks = a.ldx <= kTileMaxLdx ? a.k / kTileK : 0;
    const int64_t kb0 = !SPLIT ? 0 : (split * p.bps < blocks ? split * p.bps : blocks);
    const int64_t kb1 = last ? blocks : (kb0 + p.bps < blocks ? kb0 + p.bps : blocks);
    if ((a.k & 255) == 0 && (kb0 & 1) == 0)  // (uniform) 16-byte aligned scale chunks: scales by DMA
        mfma_kloop<8, kPfWaves, 1, false, true>(a.x + m0 * a.ldx, a.m - m0, a.ldx, a.packed + n0 * (a.k >> 1),
                                                a.scales + n0 * (a.k >> 4), a.n - n0, a.k, kb0, kb1, g_xtile0,
                                                g_xtile1, acc, nullptr, 0, g_sctile0, g_sctile1);
    else
        mfma_kloop<8, kPfWaves>(a.x + m0 * a.ldx, a.m - m0, a.ldx, a.packed + n0 * (a.k >> 1),
                                a.scales + n0 * (a.k >> 4), a.n - n0, a.k, kb0, kb1, g_xtile0, g_xtile1, acc);
    // the last split: the rest of K (and all of it for very wide x rows), then
    // the LoRA columns
    const int64_t nw = n0 + wave * 64 + lr;
    if (last)
        plain_kloop<8, kPfWaves>(
            blocks * kTileK, a.k + klora, g_xtile0,
            [&](int row, int64_t kk) { return x_piece_ext(g, m0 + row, kk, klora, fold); },
            [&](int j, int64_t kk) { return w_frag_ext(a, nw + 16 * j, kk, klora); }, acc);

    // y of MFMA tile (i, j): bf16(s_t acc), plus the LoRA term when it is not
    // in the accumulation
    const float st_scale = *a.tensor_scale;
    const float *t32 = reinterpret_cast<const float *>(g.t16());
    auto store_y = [&](int i, int j, const f32x4_t &v4) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + 16 * i + 4 * lq + v;
            const int64_t n = n0 + wave * 64 + 16 * j + lr;
            if (m < a.m && n < a.n) {
                float yv = st_scale * v4[v];
                if (!fold) yv += lora_term(a, t32, m, n);
                a.y[m * a.ldy + n] = f32_to_bf16_bits(yv);
            }
        }
    };
    if (SPLIT) {  // the FP32 tile; the splits meet here (see kSC1) or in reduce_kernel
        // split sp's tile of output tile pt (row-major over the output tiles):
        // f32x4 of MFMA tile (i, j) of wave w at ((32 w + 4 i + j) 64 + lane) 16 bytes
        const int64_t pt = (m0 / PBM) * tiles_n + n0 / PBN;
        auto tile_rsrc = [&](int64_t sp) {
            return __builtin_amdgcn_make_buffer_rsrc(g.part() + (sp * p.tiles + pt) * (kPartTileBytes / 4), 0,
                                                     (int)kPartTileBytes, 0x00020000);
        };
        const int lo = (wave * 32 * 64 + lane) * 16;
        {
            const __amdgpu_buffer_rsrc_t rm = tile_rsrc(split);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    i32x4_t v;
                    __builtin_memcpy(&v, &acc[i][j], 16);
                    if (p.meet)  // (uniform)
                        __builtin_amdgcn_raw_buffer_store_b128(v, rm, lo + (4 * i + j) * 1024, 0, kSC1);
                    else
                        __builtin_amdgcn_raw_buffer_store_b128(v, rm, lo + (4 * i + j) * 1024, 0, 0);
                }
        }
        if (!p.meet) return;
        // the arrival's outcome goes through the scale chunk's LDS, idle once
        // every wave has passed the barrier below
        volatile uint32_t *s_fin = reinterpret_cast<volatile uint32_t *>(g_sctile1);
        wait_vmcnt<0>();  // this wave's stores have completed
        __syncthreads();
        if (tid == 0) {
            const uint32_t fin = __hip_atomic_fetch_add(g.cnt() + pt, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT) + 1 == (uint32_t)p.splits;
            if (fin) __hip_atomic_store(g.cnt() + pt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_fin = fin;
        }
        __syncthreads();
        if (!*s_fin) return;  // (uniform)
        // the last split: every split's tile (its own too) summed in split
        // order, eight MFMA tiles and four splits of loads in flight at a time
#pragma unroll
        for (int t0 = 0; t0 < 32; t0 += 8) {
            f32x4_t sum[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) sum[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t s0 = 0; s0 < p.splits; s0 += 4) {
                i32x4_t v[4][8];
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (s0 + b < p.splits) {  // (uniform)
                        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(s0 + b);
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            v[b][t] = __builtin_amdgcn_raw_buffer_load_b128(rs, lo + (t0 + t) * 1024, 0, kSC1);
                    }
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (s0 + b < p.splits)
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            f32x4_t f;
                            __builtin_memcpy(&f, &v[b][t], 16);
                            sum[t] = sum[t] + f;
                        }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) store_y((t0 + t) >> 2, (t0 + t) & 3, sum[t]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) store_y(i, j, acc[i][j]);
}

template __global__ void prefill_kernel<false>(Gemm);
template __global__ void prefill_kernel<true>(Gemm);

// Split K without meeting in the launch: thread i sums f32x4 slot i % 8192 of
// output tile i / 8192 over the splits in split order (the slot holds rows
// 4 lq .. 4 lq + 3 of MFMA tile (i, j) of wave w, column lane % 16) and
// writes those four outputs as prefill_kernel's epilogue does.
__global__ __launch_bounds__(kThreads) void reduce_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    const Plan &p = g.p;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= p.tiles * 8192) return;
    const int64_t pt = idx >> 13;
    const int slot = (int)(idx & 8191), w = slot >> 11, ij = (slot >> 6) & 31, lane = slot & 63;
    const int i = ij >> 2, j = ij & 3, lr = lane & 15, lq = lane >> 4;
    const int64_t tiles_n = (a.n + PBN - 1) / PBN;
    const int64_t m0 = (pt / tiles_n) * PBM, n0 = (pt % tiles_n) * PBN;
    const int64_t n = n0 + w * 64 + 16 * j + lr;
    const f32x4_t *part = reinterpret_cast<const f32x4_t *>(g.part()) + pt * (kPartTileBytes / 16) + slot;
    f32x4_t v[kMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < p.splits) v[sp] = part[sp * p.tiles * (kPartTileBytes / 16)];
    f32x4_t sum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < p.splits) sum = sum + v[sp];
    if (n >= a.n) return;
    const float st = *a.tensor_scale;
    const bool fold = a.r == 0 || lora_fold_ok(a.lora_scale, st);
    const float *t32 = reinterpret_cast<const float *>(g.t16());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + 16 * i + 4 * lq + e;
        if (m < a.m) {
            float yv = st * sum[e];
            if (!fold) yv += lora_term(a, t32, m, n);
            a.y[m * a.ldy + n] = f32_to_bf16_bits(yv);
        }
    }
}

// the split tiles' counters, for a launch without LoRA (no prologue to clear them)
__global__ __launch_bounds__(kThreads) void cnt_zero_kernel(Gemm g) {
    for (int64_t i = threadIdx.x; i < g.p.tiles; i += kThreads)
        __hip_atomic_store(g.cnt() + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    if (m <= kDecodeMaxM) return decode_workspace_bytes(m, n, k, r);
    return (size_t)make_plan(m, n, k, r).bytes;
}

size_t gemm_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg) {
    if (m > kDecodeMaxM) {  // one segment after another, each with the whole workspace
        size_t b = 0;
        for (int j = 0; j < nseg; ++j) {
            const size_t bj = gemm_workspace_bytes(m, n[j], k, r[j]);
            b = bj > b ? bj : b;
        }
        return b;
    }
    return decode_multi_workspace_bytes(m, k, n, r, nseg);
}

hipError_t launch_w4a16_lora_gemm_multi(const GemmArgs *segs, int nseg, hipStream_t stream) {
    if (segs[0].m <= kDecodeMaxM) return launch_decode_multi(segs, nseg, stream);
    for (int i = 0; i < nseg; ++i) {  // large m: the launches are large already
        const hipError_t e = launch_w4a16_lora_gemm(segs[i], stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// RMSNorm + GEMMs: fused into the decode launch (the producers also sum the
// squares of x, the units stage bf16(x * norm_w), the epilogue applies 1 / rms)
// when m <= kNormFuseMaxM and k % 32 == 0; otherwise the norm is a launch of
// its own into the workspace, after the GEMM's part of it.
static bool norm_fused(int64_t m, int64_t k) { return m <= kNormFuseMaxM && k % 32 == 0; }

size_t norm_gemm_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg) {
    if (norm_fused(m, k)) return decode_multi_workspace_bytes(m, k, n, r, nseg, true);
    return (size_t)align256((int64_t)gemm_multi_workspace_bytes(m, k, n, r, nseg)) + (size_t)align256(m * k * 2);
}

hipError_t launch_norm_gemm_multi(const GemmArgs *segs, int nseg, hipStream_t stream) {
    const GemmArgs &a = segs[0];
    if (norm_fused(a.m, a.k)) return launch_decode_multi(segs, nseg, stream);
    int64_t n[QERL_MAX_SEGMENTS];
    int r[QERL_MAX_SEGMENTS];
    for (int i = 0; i < nseg; ++i) {
        n[i] = segs[i].n;
        r[i] = segs[i].r;
    }
    uint16_t *xn = reinterpret_cast<uint16_t *>(static_cast<char *>(a.workspace) +
                                                align256((int64_t)gemm_multi_workspace_bytes(a.m, a.k, n, r, nseg)));
    AqnArgs na{};  // sigma 0: the plain RMSNorm with scale vector norm_w
    na.x = a.x;
    na.m = a.m;
    na.h = a.k;
    na.ldx = a.ldx;
    na.weight = a.norm_w;
    na.eps = a.norm_eps;
    na.y_bf16 = xn;
    na.ldy = a.k;
    hipError_t e = launch_aqn_rmsnorm(na, stream);
    if (e != hipSuccess) return e;
    GemmArgs g[QERL_MAX_SEGMENTS];
    for (int i = 0; i < nseg; ++i) {
        g[i] = segs[i];
        g[i].x = xn;
        g[i].ldx = a.k;
        g[i].norm_w = nullptr;
    }
    return launch_w4a16_lora_gemm_multi(g, nseg, stream);
}

// The workspace use of one projection's launch against its size query (the
// decode plan's own check for m <= 256): the prologue's t region [m][r] four
// bytes each (BF16 hi/lo or FP32), the split counters and partial tiles, and
// the grid limits.
int gemm_plan_check(int64_t m, int64_t n, int64_t k, int r, int64_t size, char *msg, size_t len) {
    if (m <= kDecodeMaxM) return decode_plan_check(m, k, &n, &r, 1, false, msg, len);
    const Plan p = make_plan(m, n, k, r);
    auto fail = [&](const char *what, int64_t a, int64_t b) {
        snprintf(msg, len, "prefill m=%lld n=%lld k=%lld r=%d: %s (%lld > %lld)", (long long)m, (long long)n,
                 (long long)k, r, what, (long long)a, (long long)b);
        return 1;
    };
    if (p.t_off + m * (int64_t)r * 4 > p.tpart_off) return fail("t region", p.t_off + m * (int64_t)r * 4, p.tpart_off);
    const int64_t tpart_end = p.tpart_off + (p.ksplit > 1 ? p.ksplit * m * (int64_t)r * 4 : 0);
    if (tpart_end > p.part_off) return fail("partial t region", tpart_end, p.part_off);
    if (p.ksplit > 1 && ((p.kchunk % 128) != 0 || (p.ksplit - 1) * p.kchunk >= k))
        return fail("prologue K ranges", (p.ksplit - 1) * p.kchunk, k - 1);
    if (p.ksplit > 0xFFFF) return fail("prologue grid", p.ksplit, 0xFFFF);
    const int64_t cnt_end = p.cnt_off + (p.splits > 1 ? p.tiles * 4 : 0);
    if (cnt_end > p.part_off) return fail("split counters", cnt_end, p.part_off);
    const int64_t part_end = p.part_off + (p.splits > 1 ? p.splits * p.tiles * kPartTileBytes : 0);
    if (part_end > size) return fail("partial tiles", part_end, size);
    if (p.splits > 1 && p.splits * p.tiles * kPartTileBytes > 0x7FFFFFFF)
        return fail("partial tiles (32-bit buffer offsets)", p.splits * p.tiles * kPartTileBytes, 0x7FFFFFFF);
    if (p.splits > kMaxSplits) return fail("splits", p.splits, kMaxSplits);
    if (p.splits > 1 && (p.splits - 1) * p.bps >= k / 128) return fail("empty split", (p.splits - 1) * p.bps, k / 128 - 1);
    if (p.tiles * p.splits > 0x7FFFFFFF) return fail("grid", p.tiles * p.splits, 0x7FFFFFFF);
    return 0;
}

int gemm_multi_plan_check(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm, char *msg,
                          size_t len) {
    if (norm ? norm_fused(m, k) : m <= kDecodeMaxM) return decode_plan_check(m, k, n, r, nseg, norm, msg, len);
    const int64_t size = (int64_t)gemm_multi_workspace_bytes(m, k, n, r, nseg);
    for (int j = 0; j < nseg; ++j)  // one launch after another, each with the whole workspace
        if (gemm_plan_check(m, n[j], k, r[j], size, msg, len)) return 1;
    if (norm) {  // the normed x after the GEMMs' part
        const int64_t xn_end = align256(size) + m * k * 2, nsize = (int64_t)norm_gemm_multi_workspace_bytes(m, k, n, r, nseg);
        if (xn_end > nsize) {
            snprintf(msg, len, "norm m=%lld k=%lld: normed x past the size query (%lld > %lld)", (long long)m,
                     (long long)k, (long long)xn_end, (long long)nsize);
            return 1;
        }
    }
    return 0;
}

hipError_t launch_w4a16_lora_gemm(const GemmArgs &a, hipStream_t stream) {
    if (a.m <= kDecodeMaxM) return launch_decode(a, stream);
    const Gemm g{a, make_plan(a.m, a.n, a.k, a.r)};
    if (a.r > 0) {
        const dim3 pgrid((unsigned)((a.m + 15) / 16), (unsigned)g.p.ksplit);
        const int jt = (a.r + 15) / 16;
        if (jt <= 1)
            hipLaunchKernelGGL(prologue_kernel<1>, pgrid, dim3(kThreads), 0, stream, g);
        else if (jt <= 2)
            hipLaunchKernelGGL(prologue_kernel<2>, pgrid, dim3(kThreads), 0, stream, g);
        else if (jt <= 4)
            hipLaunchKernelGGL(prologue_kernel<4>, pgrid, dim3(kThreads), 0, stream, g);
        else
            hipLaunchKernelGGL(prologue_kernel<8>, pgrid, dim3(kThreads), 0, stream, g);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (g.p.ksplit > 1) {
            hipLaunchKernelGGL(t_reduce_kernel, dim3((unsigned)((a.m * a.r + kThreads - 1) / kThreads)), dim3(kThreads),
                               0, stream, g);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    const int64_t grid = g.p.tiles * g.p.splits;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (g.p.splits == 1) {
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(64 * kPfWaves), 0, stream, g);
        return hipGetLastError();
    }
    if (g.p.meet && a.r == 0) {  // the prologue clears the counters; without LoRA this does
        hipLaunchKernelGGL(cnt_zero_kernel, dim3(1), dim3(kThreads), 0, stream, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(64 * kPfWaves), 0, stream, g);
    if (g.p.meet) return hipGetLastError();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((g.p.tiles * 8192 + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, stream, g);
    return hipGetLastError();
}

}  // namespace qerl
