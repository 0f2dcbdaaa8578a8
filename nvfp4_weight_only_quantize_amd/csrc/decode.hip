// decode.hip -- W4A16 (NVFP4 weight x BF16 activation) + LoRA for decode
// batches, 1 <= m <= 256, on gfx950.
//
//   y[m, n] = s_t * sum_k x[m,k] e2m1(q[n,k]) e4m3(sb[n,k/16])
//           + lora_scale * sum_j t[m,j] B[n,j],        t = x A^T
//
// (the NVFP4 x BF16 rollout kernel of the "NVlabs/QeRL" README,
// "Acknowledgement", with the LoRA sum of the bitsofall page, "LoRA
// (Low-Rank Adaptation)" and "Implementation and Practical Details").
//
// Decode is bound by the bytes of the packed weights (0.5625 B per weight),
// which are read exactly once.  Weights are decoded to exact BF16 (e2m1 *
// e4m3 has <= 6 significant bits) and multiplied on the BF16 MFMA in FP32.
//
// Two launches per call, with no counter, flag or wait between workgroups:
//  * the main kernel: "producer" workgroups at the head of the grid compute
//    partial sums of t = x A^T over ranges of K (and, with the fused RMSNorm,
//    of x^2), and "units" stream a block of weight rows over a slice of K;
//    every workgroup stores its FP32 partial tile and exits.
//  * finish_kernel sums the producers' partial tiles (into t, K-range order)
//    and the units' partial tiles (slice order) -- deterministic -- and writes
//    y = bf16(inv_rms * (s_t * acc + lora_scale * t B^T)).
// A call with a single slice, no LoRA and no norm writes y from the units.
//
// m <= 16, stream_kernel.  Units are 128 weight rows x one K slice; each of
// the 8 waves owns 16 rows.  The unit's x slice is staged into LDS (bf16(x *
// norm_w) with the norm); the weights stream in the span layout (below), one
// group of loads in flight per wave, and latency is covered by several
// resident units per CU (registers are capped for that).
//
// 16 < m <= 256, mfma_unit_kernel.  Units are (256 weight rows) x (slice of K)
// running the K loops of mfma_tile.h with up to 128 rows of x as the x tile
// (m > 128: one unit per 128-row m-block of x, the m-blocks one after another
// in the grid).
//
// Several projections of one x (q/k/v, gate/up) share a launch: the segment
// is a grid dimension; a one-segment launch is its own instantiation with a
// one-plan argument.
#include <stdio.h>

#include "device_common.h"
#include "mfma_tile.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreadsD = kWaves * 64;
#ifndef QERL_STREAM_UNIT_WAVES
#define QERL_STREAM_UNIT_WAVES 8
#endif
// waves of a stream_kernel unit (16 weight rows each): eight share one staged
// x slice, half the x bytes per weight byte of four (32B layer at m = 16: 137
// -> 128 us per decode pass); sixteen were slower
constexpr int kSW = QERL_STREAM_UNIT_WAVES;
constexpr int kThreadsS = 64 * kSW;
// waves of a 16 < m unit (64 weight rows each).  Eight waves sharing one x
// tile, or weights fetched two blocks ahead, were measured slower: the unit is
// bound by its CU's vector memory path, not by latency.
constexpr int kUnitWaves = 4;
constexpr int64_t kChunkK = 128;          // K elements per chunk
constexpr int kXPad = 8;                  // BF16 padding per staged x row
constexpr int64_t kGroupK = 4 * kChunkK;  // m <= 16: K elements of one span group (four chunks)
#ifndef QERL_XSLICE_KB
#define QERL_XSLICE_KB 36
#endif
#ifndef QERL_UNITS_PER_CU
#define QERL_UNITS_PER_CU 3
#endif
#ifndef QERL_STREAM_WAVES_PER_SIMD
#define QERL_STREAM_WAVES_PER_SIMD 6
#endif
constexpr int64_t kXSliceBudget = QERL_XSLICE_KB * 1024;  // m <= 16: LDS for a unit's x slice, so that several units share a CU
constexpr int64_t kUnitsPerCu = QERL_UNITS_PER_CU;        // m <= 16: units per compute unit the K split aims for
constexpr int64_t kLdsLimit = 140 * 1024;  // of the 160 KiB a gfx950 workgroup may hold
constexpr int64_t kProdChunks = 4;        // least K chunks per LoRA producer
constexpr int64_t kMaxProdRanges = 8;     // K ranges of the producers, at most (finish_kernel sums them in one batch)
constexpr int kProdTiles = 1;             // rank tiles a producer accumulates
constexpr int kBatch = 8;                // loads in flight per thread in reductions and staging
constexpr int kMaxRank = 128;            // QERL_MAX_LORA_RANK
constexpr int64_t kUnitScBytes = 24 * 1024;  // 16 < m: LDS for a unit's scale tile
#ifndef QERL_MFMA_UNIT_CHUNKS
#define QERL_MFMA_UNIT_CHUNKS 10
#endif
#ifndef QERL_MFMA_UNITS_PER_CU
#define QERL_MFMA_UNITS_PER_CU 1
#endif
constexpr int64_t kUnitChunks = QERL_MFMA_UNIT_CHUNKS;        // 16 < m: K chunks per unit the split aims for, at most
constexpr int64_t kMfmaUnitsPerCu = QERL_MFMA_UNITS_PER_CU;  // 16 < m: units per CU the K split aims for
constexpr int64_t kMaxRowBlocks = (int64_t)1 << 24;  // row blocks of one call (grid x stays in range)

struct DecodePlan {
    int mt, nw, px;
    int mb, mtp;                   // m-blocks of 16 mt rows (a unit takes one), m-tiles of the producers (mb mt)
    int64_t rows_per_unit, row_blocks;
    int64_t chunks, full_chunks;   // chunks of K (the last may be partial), full chunks
    int64_t cps, slices, units;    // chunks per slice (a multiple of 4/nw)
    int64_t producers, jt;         // LoRA producers, 16-wide rank tiles
    int64_t prod_kr, prod_groups;  // producers: K ranges x (m-tile, rank-tile group) groups
    int64_t prod_chunks;           // K chunks of one producer range
    int64_t xpitch, lds_bytes;     // m <= 16: BF16 elements per LDS x row; dynamic LDS bytes
    int64_t unit_sc_pitch;         // 16 < m: LDS pitch of the unit's scale tile
    bool unit_sc;                  // 16 < m: scales staged in LDS
    // workspace offsets from the segment's data: the units' partial tiles,
    // the producers' partial tiles of t, their sums of squares
    int64_t part_off, tpart_off, ss_off, bytes;
    // RMSNorm prologue (m <= 16): the producers also sum x^2 per K range,
    // [prod_kr][16] at ss_off
    bool norm;
    // the units write y themselves (one slice, no LoRA, no norm)
    bool direct_out;
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

// compute units of the current device (queried once)
int64_t cu_count() {
    static const int64_t cus = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        return (int64_t)v;
    }();
    return cus;
}

// slice_rows: the row blocks the CUs are shared by (a multi-segment launch
// passes the total over its segments, so every segment gets the same slices)
// norm: an RMSNorm prologue (m <= 16 only): producers run even without LoRA
// and also sum the squares of x.
DecodePlan make_decode_plan(int64_t m, int64_t n, int64_t k, int r, int64_t slice_rows = 0, bool norm = false) {
    DecodePlan p{};
    p.mt = m <= 16 ? 1 : (m <= 32 ? 2 : (m <= 64 ? 4 : 8));
    p.mb = (int)((m + 16 * p.mt - 1) / (16 * p.mt));  // more than one for m > 128
    p.mtp = p.mb * p.mt;
    p.nw = p.mt == 1 ? 1 : kUnitWaves * 4 / kWaves;  // 16 < m: MFMA units of 64 kUnitWaves weight rows
    p.rows_per_unit = p.mt == 1 ? 16 * kSW : 16 * kWaves * (int64_t)p.nw;
    p.row_blocks = (n + p.rows_per_unit - 1) / p.rows_per_unit;
    if (p.row_blocks > kMaxRowBlocks) p.row_blocks = 0;  // one counter per row block: rejected at launch
    p.chunks = (k + kChunkK - 1) / kChunkK;
    p.full_chunks = k / kChunkK;
    p.px = 1;
    p.jt = (r + 15) / 16;
    p.prod_chunks = (p.chunks + kMaxProdRanges - 1) / kMaxProdRanges;
    if (p.prod_chunks < kProdChunks) p.prod_chunks = kProdChunks;
    p.prod_kr = (p.chunks + p.prod_chunks - 1) / p.prod_chunks;
    p.prod_groups = p.mtp * ((p.jt + kProdTiles - 1) / kProdTiles);
    p.norm = norm && p.mt == 1;
    if (p.norm && p.prod_groups < 1) p.prod_groups = 1;  // sums of squares only
    p.producers = (r > 0 || p.norm) ? p.prod_kr * p.prod_groups : 0;
    // slices: as many units as compute units without going over (a CU that
    // runs two units while others run one sets the time), and the FP32
    // partials below the weight bytes
    if (slice_rows < p.row_blocks) slice_rows = p.row_blocks;
    int64_t s = slice_rows > 0 ? cu_count() / slice_rows : 1;
    int64_t s_cap = (k * 9) / (64 * m);
    if (s_cap < 1) s_cap = 1;
    if (s > s_cap) s = s_cap;
    if (s < 1) s = 1;
    const int64_t tile = p.rows_per_unit * 16 * p.mt * 4;
    if (p.mt > 1) {  // mfma_unit_kernel: static LDS, the whole x as its x tile
        // fewer row blocks than CUs split K as above; more still split K so
        // that a unit takes at most kUnitChunks chunks (several units per CU
        // keep more loads in flight than one long unit): 32B layer at M = 64
        // 201 -> 188 us against the floor of chunks / 8 (4 slices of 10 chunks
        // for K = 5120 rather than 5 of 8, 22 rather than 27 for K = 27648),
        // the 7B layer unchanged
        const int64_t s_work = (p.chunks + kUnitChunks - 1) / kUnitChunks;
        if (s < s_work) s = s_work < s_cap ? s_work : s_cap;
        const int64_t s_occ = (cu_count() * kMfmaUnitsPerCu + slice_rows * p.mb - 1) / (slice_rows * p.mb);
        const int64_t s_most = p.chunks / 2 < s_cap ? p.chunks / 2 : s_cap;  // at least two chunks per unit
        if (s < s_occ) s = s_occ < s_most ? s_occ : s_most;
        if (s < 1) s = 1;
        p.cps = (p.chunks + s - 1) / s;
        p.slices = (p.chunks + p.cps - 1) / p.cps;
        p.units = p.row_blocks * p.slices * p.mb;
        int64_t scp = (p.cps * 8 + 15) / 16;  // rows an odd multiple of 16 bytes apart
        if (scp % 2 == 0) ++scp;
        p.unit_sc_pitch = scp * 16;
        p.unit_sc = p.rows_per_unit * p.unit_sc_pitch <= kUnitScBytes;
        p.part_off = 0;
        p.tpart_off = align256(p.part_off + p.units * tile);
        p.ss_off = align256(p.tpart_off + p.prod_kr * (int64_t)p.mtp * p.jt * 64 * 16);
        p.bytes = p.ss_off;
        return p;
    }
    // m <= 16: stream_kernel.  K is cut into slices of whole 512-element
    // groups (the span layout of the main loop) so that there are about
    // kUnitsPerCu units per compute unit: a unit's loads are in flight only
    // while it waits for them, so memory-level parallelism comes from several
    // resident units per CU.  The x slice (the unit's only LDS besides the
    // epilogue and producer scratch) is bounded so that they fit together.
    const int64_t groups = (p.chunks + 3) / 4;  // the last one may be short
    int64_t sl = (cu_count() * kUnitsPerCu + slice_rows - 1) / slice_rows;
    if (sl > s_cap) sl = s_cap;
    if (sl > groups) sl = groups;
    if (sl < 1) sl = 1;
    int64_t gps = (groups + sl - 1) / sl;
    const int64_t g_max = (kXSliceBudget / (2 * m) - kXPad) / kGroupK;
    if (gps > g_max) gps = g_max;
    if (gps < 1) gps = 1;
    const int64_t cps = gps * 4;
    p.cps = cps;
    p.slices = (p.chunks + cps - 1) / cps;
    p.units = p.row_blocks * p.slices;
    p.direct_out = r == 0 && !p.norm && p.slices == 1;
    p.xpitch = cps * kChunkK + kXPad;
    int64_t lds = m * p.xpitch * 2;
    const int64_t prod = (int64_t)kWaves * kProdTiles * 64 * 16 + kWaves * 16 * 4;  // producer wave reductions
    if (lds < prod) lds = prod;
    p.lds_bytes = lds;
    // workspace: the units' partial tiles (every unit has one: a launch over
    // several segments writes y from the units only if every segment can),
    // the producers' partial tiles of t, their sums of squares
    p.part_off = 0;
    p.tpart_off = align256(p.part_off + p.units * tile);
    p.ss_off = align256(p.tpart_off + p.prod_kr * (int64_t)p.mtp * p.jt * 64 * 16);
    p.bytes = align256(p.ss_off + (p.norm ? p.prod_kr * 16 * 4 : 0));
    return p;
}

struct Decode {
    GemmArgs a;  // a.workspace: this segment's data region
    DecodePlan p;
    __device__ float *part() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.part_off); }
    __device__ float *tpart() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.tpart_off); }
    __device__ float *ssp() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.ss_off); }
};

// One launch over up to kMaxSegments GEMMs that share x (m, k, ldx): the
// segment is a grid dimension (y for the main kernels, z for finish_kernel),
// so a workgroup reads its segment's fields without first reading a table;
// the grid is as wide as the widest segment and the surplus workgroups of
// the others exit at once.  Each segment has its own workspace region.
// A one-segment launch takes a one-segment set, so its kernel arguments stay
// as small as one plan.
constexpr int kMaxSegments = QERL_MAX_SEGMENTS;
template <int NS>
struct DecodeSetN {
    Decode seg[NS];
    int nseg;
};
using DecodeSet = DecodeSetN<kMaxSegments>;

__device__ __forceinline__ bf16x8_t as_bf16x8_d(const uint4 &u) {
    bf16x8_t v;
    __builtin_memcpy(&v, &u, 16);
    return v;
}

// exact BF16 of e2m1 * e4m3 for the 8 elements of one packed 32-bit word
__device__ __forceinline__ bf16x8_t dequant8_d(uint32_t q, float s) {
    const f32x2_t f0 = QERL_FP4_PAIR_F32(q, 0), f1 = QERL_FP4_PAIR_F32(q, 1);
    const f32x2_t f2 = QERL_FP4_PAIR_F32(q, 2), f3 = QERL_FP4_PAIR_F32(q, 3);
    return as_bf16x8_d(make_uint4(pack_bf16x2(f0.x * s, f0.y * s), pack_bf16x2(f1.x * s, f1.y * s),
                                  pack_bf16x2(f2.x * s, f2.y * s), pack_bf16x2(f3.x * s, f3.y * s)));
}

// ---------------------------------------------------------------------------
// LoRA producers: t = x A^T
// ---------------------------------------------------------------------------
// Producer p covers one range of prod_chunks chunks of K for one 16-row
// m-tile and kProdTiles 16-rank tiles (the producers of a launch enumerate
// K ranges x m-tiles x rank-tile groups); its 4 waves take interleaved
// 32-element steps.  A lane supplies x row 16*mt + (lane % 16) and A row
// 16*jt + (lane % 16), 8 elements at 8*(lane / 16) of the step, so MFMA tile
// (mt, jt) holds t[16 mt + 4 (lane/16) + v][16 jt + lane % 16] in element v.
// The range's tiles go to the workspace; finish_kernel sums the ranges.
// NORM (m <= 16): x enters as bf16(x * norm_w) and the first group of each K
// range also stores the sums of the squares of x over the range.
template <int MT, bool NORM = false>
__device__ void lora_producer(const Decode &d, int64_t p, uint8_t *lds) {
    static_assert(!NORM || MT == 1, "the norm prologue is for m <= 16");
    const GemmArgs &a = d.a;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int JT = (int)d.p.jt, JG = (JT + kProdTiles - 1) / kProdTiles;
    const int JGd = JG > 0 ? JG : 1;  // (r == 0 with the norm: one group, no rank tiles)
    // producer p: K range kr, m-tile mt, rank tiles jg .. jg + kProdTiles - 1
    // (one pass each, so that no producer runs all m-tiles and ranks in turn)
    const int64_t kr = p / d.p.prod_groups;
    const int grp = (int)(p - kr * d.p.prod_groups);
    const int64_t kb = kr * d.p.prod_chunks * kChunkK;
    const int64_t ke = kb + d.p.prod_chunks * kChunkK < a.k ? kb + d.p.prod_chunks * kChunkK : a.k;
    const int64_t tile_floats = (int64_t)(MT == 8 ? d.p.mtp : MT) * JT * 64 * 4;  // all m-tiles of x (m-blocks: MT == 8)
    f32x4_t *own = reinterpret_cast<f32x4_t *>(d.tpart() + kr * tile_floats);  // this K range's tiles
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [wave][2 tiles][64 lanes]
    float *red_ss = reinterpret_cast<float *>(lds + kWaves * kProdTiles * 64 * 16);  // [wave][16]
    // one m-tile and two rank tiles, so the producer path never needs more
    // registers than the streaming path; each wave's steps (32 elements,
    // every 4th of the range) in groups of PS with all loads of a group
    // issued before its products
    constexpr int PS = 2;
    {
        const int mt = grp / JGd, jg = (grp - mt * JGd) * kProdTiles;
        const bool sum_sq = NORM && grp == 0;  // (uniform)
        const int64_t mrow = 16 * mt + lr < a.m ? 16 * mt + lr : a.m - 1;
        const uint16_t *xrow = a.x + mrow * a.ldx;
        float ss = 0.0f;
        {
            f32x4_t acc[kProdTiles];
#pragma unroll
            for (int j = 0; j < kProdTiles; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            // (in a wider workgroup only the first kWaves waves work; the rest
            // keep to the barriers)
            for (int64_t k0 = wave < kWaves ? kb + 32 * wave : ke; k0 < ke; k0 += 4 * 32 * PS) {
                uint4 xv[PS], av[PS][kProdTiles];
                float4 nv[PS][2];
#pragma unroll
                for (int u = 0; u < PS; ++u) {
                    const int64_t kk = k0 + 128 * u + 8 * lq;
                    const int64_t kc = kk < ke ? kk : ke - 8;  // k % 16 == 0: a piece never straddles the end
                    xv[u] = *reinterpret_cast<const uint4 *>(xrow + kc);
                    if (NORM) {
                        nv[u][0] = *reinterpret_cast<const float4 *>(a.norm_w + kc);
                        nv[u][1] = *reinterpret_cast<const float4 *>(a.norm_w + kc + 4);
                    }
#pragma unroll
                    for (int jj = 0; jj < kProdTiles; ++jj) {
                        av[u][jj] = make_uint4(0, 0, 0, 0);
                        if (jg + jj < JT) {  // (uniform)
                            const int jr = 16 * (jg + jj) + lr;
                            const int64_t j = jr < a.r ? jr : a.r - 1;
                            av[u][jj] = *reinterpret_cast<const uint4 *>(a.lora_a + j * a.k + kc);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < PS; ++u) {
                    const bool kin = k0 + 128 * u + 8 * lq < ke;
                    uint4 xu = kin ? xv[u] : make_uint4(0, 0, 0, 0);
                    if (NORM) {
                        const float xf[8] = {bf16lo_to_f32(xu.x), bf16hi_to_f32(xu.x), bf16lo_to_f32(xu.y),
                                             bf16hi_to_f32(xu.y), bf16lo_to_f32(xu.z), bf16hi_to_f32(xu.z),
                                             bf16lo_to_f32(xu.w), bf16hi_to_f32(xu.w)};
                        if (sum_sq)
#pragma unroll
                            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(xf[e], xf[e], ss);
                        const float4 n0 = nv[u][0], n1 = nv[u][1];
                        xu = make_uint4(pack_bf16x2(xf[0] * n0.x, xf[1] * n0.y), pack_bf16x2(xf[2] * n0.z, xf[3] * n0.w),
                                        pack_bf16x2(xf[4] * n1.x, xf[5] * n1.y), pack_bf16x2(xf[6] * n1.z, xf[7] * n1.w));
                    }
                    const bf16x8_t xa = as_bf16x8_d(xu);
#pragma unroll
                    for (int jj = 0; jj < kProdTiles; ++jj) {
                        const bool jin = kin && 16 * (jg + jj) + lr < a.r;
                        acc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            xa, as_bf16x8_d(jin ? av[u][jj] : make_uint4(0, 0, 0, 0)), acc[jj], 0, 0, 0);
                    }
                }
            }
            // the four waves' tiles, summed in wave order by wave 0 and stored;
            // finish_kernel reads them after the kernel boundary
            if (wave < kWaves)
#pragma unroll
                for (int jj = 0; jj < kProdTiles; ++jj) red[(wave * kProdTiles + jj) * 64 + lane] = acc[jj];
            if (NORM && sum_sq) {  // a row's squares: its 4 lanes in each wave, then the waves
                ss += __shfl_xor(ss, 16, 64);
                ss += __shfl_xor(ss, 32, 64);
                if (wave < kWaves && lq == 0) red_ss[wave * 16 + lr] = ss;
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int jj = 0; jj < kProdTiles; ++jj) {
                    if (jg + jj >= JT) continue;
                    f32x4_t t = red[jj * 64 + lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) t = t + red[(w * kProdTiles + jj) * 64 + lane];
                    own[(mt * JT + jg + jj) * 64 + lane] = t;
                }
                if (NORM && sum_sq && lane < 16) {
                    float tot = red_ss[lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) tot += red_ss[w * 16 + lane];
                    d.ssp()[kr * 16 + lane] = tot;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The streaming kernel
// ---------------------------------------------------------------------------
// One full chunk of the weights for lane (lr, lq) of row group g: row n,
// elements 128c + 32lq .. +32 (16 packed bytes).  Rows past n are clamped
// (their outputs are discarded).  K32: k % 32 == 0, packed rows 16-byte aligned.
template <int NW, bool K32>
__device__ __forceinline__ void load_chunk(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq, uint4 (&w)[NW]) {
    const int64_t e0 = c * kChunkK + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        int64_t n = n0 + 16 * g + lr;
        n = n < a.n ? n : a.n - 1;
        const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
        if (K32) {
            w[g] = *reinterpret_cast<const uint4 *>(prow);
        } else {
            const uint2 lo = reinterpret_cast<const uint2 *>(prow)[0];
            const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
            w[g] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }
}

// The partial last chunk (k % 128 != 0): elements past k read as zero.
template <int NW>
__device__ __forceinline__ void load_chunk_tail(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq,
                                                uint4 (&w)[NW]) {
    const int64_t e0 = c * kChunkK + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        int64_t n = n0 + 16 * g + lr;
        n = n < a.n ? n : a.n - 1;
        const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
        w[g] = make_uint4(0, 0, 0, 0);
        if (e0 + 16 <= a.k) {
            const uint2 lo = *reinterpret_cast<const uint2 *>(prow);
            w[g].x = lo.x;
            w[g].y = lo.y;
            if (e0 + 32 <= a.k) {
                const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
                w[g].z = hi.x;
                w[g].w = hi.y;
            }
        }
    }
}

// Copy a rows x per_row grid of items from global to LDS, kBatch per thread
// in flight (a plain loop would wait for every load before issuing the next).
// Item i = thread + kThreadsD * step is (i / per_row, i % per_row); the pair
// is advanced by the block's stride instead of dividing per item, in 32 bits.
template <typename T, typename Src, typename Dst>
__device__ __forceinline__ void batched_copy_2d(int rows, int per_row, Src src, Dst dst) {
    const int total = rows * per_row;
    const int dr = kThreadsD / per_row, dc = kThreadsD - dr * per_row;
    int r = (int)threadIdx.x / per_row, c = (int)threadIdx.x - r * per_row;
    for (int base = threadIdx.x; base < total; base += kBatch * kThreadsD) {
        T v[kBatch];
        int rr[kBatch], cc[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            rr[u] = r;
            cc[u] = c;
            if (base + u * kThreadsD < total) v[u] = src(r, c);
            r += dr;
            c += dc;
            if (c >= per_row) {
                c -= per_row;
                ++r;
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (base + u * kThreadsD < total) dst(rr[u], cc[u], v[u]);
    }
}

// The unit's x slice, rows [0, m) x columns [k0, k0 + width), into LDS rows
// of `pitch` elements; columns at or past k are zero.  NORM: each element
// enters as bf16(x * norm_w[column]) (the row's 1 / rms is applied in the
// epilogue).
template <bool NORM, int NT = kThreadsD>
__device__ void stage_x_slice(const GemmArgs &a, uint16_t *xs, int64_t pitch, int64_t k0, int64_t width) {
    // 8-element pieces i = row * per_row + piece, kStage per thread in flight
    // (every load of a round issued before its stores)
    constexpr int kStage = 4;
    const int per_row = (int)(width / 8), total = (int)a.m * per_row;
    for (int base = threadIdx.x; base < total; base += kStage * NT) {
        uint4 v[kStage];
        float4 w0[kStage], w1[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = base + u * NT;
            const int row = i / per_row, pc = i - row * per_row;
            const int64_t col = k0 + 8 * pc;
            const bool in = i < total && col < a.k;  // k % 16 == 0: a piece is inside or outside
            v[u] = in ? *reinterpret_cast<const uint4 *>(a.x + row * a.ldx + col) : make_uint4(0, 0, 0, 0);
            if (NORM) {
                w0[u] = in ? *reinterpret_cast<const float4 *>(a.norm_w + col) : make_float4(0.f, 0.f, 0.f, 0.f);
                w1[u] = in ? *reinterpret_cast<const float4 *>(a.norm_w + col + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = base + u * NT;
            if (i >= total) break;
            const int row = i / per_row, pc = i - row * per_row;
            uint4 o = v[u];
            if (NORM)
                o = make_uint4(pack_bf16x2(bf16lo_to_f32(o.x) * w0[u].x, bf16hi_to_f32(o.x) * w0[u].y),
                               pack_bf16x2(bf16lo_to_f32(o.y) * w0[u].z, bf16hi_to_f32(o.y) * w0[u].w),
                               pack_bf16x2(bf16lo_to_f32(o.z) * w1[u].x, bf16hi_to_f32(o.z) * w1[u].y),
                               pack_bf16x2(bf16lo_to_f32(o.w) * w1[u].z, bf16hi_to_f32(o.w) * w1[u].w));
            *reinterpret_cast<uint4 *>(xs + row * pitch + 8 * pc) = o;
        }
    }
}

// Stage the unit's scale bytes: rows [n0, n0 + R) x bytes [b0, b0 + nb) of
// the [n, k/16] scale matrix into LDS rows of `pitch` bytes.
__device__ void stage_scales(const GemmArgs &a, uint8_t *sc, int64_t pitch, int64_t n0, int64_t R, int64_t b0,
                             int64_t nb) {
    const int64_t row_bytes = a.k >> 4;
    auto row_of = [&](int rr) { return n0 + rr < a.n ? n0 + rr : a.n - 1; };
    if (row_bytes % 16 == 0 && b0 % 16 == 0) {
        // 16-byte pieces; the last may run past nb but not past the row
        batched_copy_2d<uint4>(
            (int)R, (int)((nb + 15) / 16),
            [&](int rr, int pc) {
                return *reinterpret_cast<const uint4 *>(a.scales + row_of(rr) * row_bytes + b0 + 16 * pc);
            },
            [&](int rr, int pc, const uint4 &v) { *reinterpret_cast<uint4 *>(sc + rr * pitch + 16 * pc) = v; });
    } else if (row_bytes % 4 == 0) {  // b0 is a multiple of 8
        batched_copy_2d<uint32_t>(
            (int)R, (int)((nb + 3) / 4),
            [&](int rr, int pc) {
                return *reinterpret_cast<const uint32_t *>(a.scales + row_of(rr) * row_bytes + b0 + 4 * pc);
            },
            [&](int rr, int pc, const uint32_t &v) { *reinterpret_cast<uint32_t *>(sc + rr * pitch + 4 * pc) = v; });
    } else {
        batched_copy_2d<uint8_t>(
            (int)R, (int)nb, [&](int rr, int pc) { return a.scales[row_of(rr) * row_bytes + b0 + pc]; },
            [&](int rr, int pc, const uint8_t &v) { sc[rr * pitch + pc] = v; });
    }
}

// ---- m <= 16 main loop: the span layout ----
// A 512-element group of K is permuted identically on both MFMA operands:
// lane quarter q takes elements 128 q .. 128 q + 127 of the group, i.e. 64
// contiguous packed bytes (four 16-byte loads) and the 8 scale bytes of its 8
// blocks (one 8-byte load), spread over the group's 16 MFMA steps (8 elements
// each).  Against one 16-byte code load and one 2-byte scale load per
// 128-element chunk, that is 5 loads instead of 8 per 512 elements, and scale
// loads 8 bytes wide: measured on gfx950 this layout streams a 38 MB weight at
// 3.8-4.0 TB/s where the chunk layout reaches 2.2 TB/s.
struct SpanGroup {
    uint4 q0, q1, q2, q3;  // packed codes: 32 elements each
    uint2 sc;              // E4M3 scales of the 8 blocks
};

__device__ __forceinline__ SpanGroup load_span_group(const uint8_t *prow, const uint8_t *srow, int64_t g, int lq) {
    const uint4 *q = reinterpret_cast<const uint4 *>(prow + g * (kGroupK / 2) + 64 * lq);
    SpanGroup v;
    v.q0 = q[0];
    v.q1 = q[1];
    v.q2 = q[2];
    v.q3 = q[3];
    v.sc = *reinterpret_cast<const uint2 *>(srow + g * (kGroupK / 16) + 8 * lq);
    return v;
}

// 16-byte piece of codes `q` (blocks b0, b1 of scale word `sw`, bytes B0 and
// B0 + 1) against the x elements at xp .. xp + 31
template <int B0>
__device__ __forceinline__ void mma_piece(const uint4 &q, uint32_t sw, const uint16_t *xp, f32x4_t &acc) {
    const float s0 = QERL_E4M3_F32(sw, B0), s1 = QERL_E4M3_F32(sw, B0 + 1);
    const bf16x8_t x0 = *reinterpret_cast<const bf16x8_t *>(xp), x1 = *reinterpret_cast<const bf16x8_t *>(xp + 8);
    const bf16x8_t x2 = *reinterpret_cast<const bf16x8_t *>(xp + 16), x3 = *reinterpret_cast<const bf16x8_t *>(xp + 24);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, dequant8_d(q.x, s0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, dequant8_d(q.y, s0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x2, dequant8_d(q.z, s1), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x3, dequant8_d(q.w, s1), acc, 0, 0, 0);
}

// One group: xg is this lane's x row at element 128 lq of the group
// (the scheduling barriers keep the compiler from hoisting all 16 x
// fragments of a group, which would cost 64 registers and with them resident
// waves)
__device__ __forceinline__ void mma_span_group(const SpanGroup &v, const uint16_t *xg, f32x4_t &acc) {
    mma_piece<0>(v.q0, v.sc.x, xg, acc);
    __builtin_amdgcn_sched_barrier(0);
    mma_piece<2>(v.q1, v.sc.x, xg + 32, acc);
    __builtin_amdgcn_sched_barrier(0);
    mma_piece<0>(v.q2, v.sc.y, xg + 64, acc);
    __builtin_amdgcn_sched_barrier(0);
    mma_piece<2>(v.q3, v.sc.y, xg + 96, acc);
}

// The scale bytes b, b + 1 of a row holding nb of them (bytes past nb read
// as zero).  ALIGNED: nb even and b even, so one 16-bit load.
template <bool ALIGNED>
__device__ __forceinline__ uint32_t load_scale_pair(const uint8_t *srow, int64_t b, int64_t nb) {
    if (ALIGNED) return *reinterpret_cast<const uint16_t *>(srow + b);
    const uint32_t lo = b < nb ? srow[b] : 0u, hi = b + 1 < nb ? srow[b + 1] : 0u;
    return lo | hi << 8;
}

// One 128-element chunk in the chunk layout (lane quarter q: elements 32 q ..
// 32 q + 31; scale pair s2): xp is this lane's x row at element 32 q of it
__device__ __forceinline__ void mma_chunk_sc(const uint4 &w, uint32_t s2, const uint16_t *xp, f32x4_t &acc) {
    mma_piece<0>(w, s2, xp, acc);
}

// K32: k % 32 == 0; DIRECT: the units write y (every segment has one slice,
// no LoRA, no norm), else each stores its FP32 partial tile for
// finish_kernel; LORA: some segment has r > 0; NORM: the RMSNorm in front.
template <int NS, bool K32, bool DIRECT, bool LORA, bool NORM>
// Registers are capped so that QERL_STREAM_WAVES_PER_SIMD waves fit each SIMD
// (the main loop needs about 60; the producer and epilogue paths would take
// more and are allowed to spill a little).
__global__ __launch_bounds__(kThreadsS) __attribute__((amdgpu_waves_per_eu(QERL_STREAM_WAVES_PER_SIMD, 8)))
void stream_kernel(DecodeSetN<NS> ds) {
    constexpr int MT = 1, NW = 1;  // one 16-row m-tile, one 16-row weight group per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.y];
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    const int64_t bx = blockIdx.x;
    if (NS > 1 && bx >= p.producers + p.units) return;  // past a narrower segment
    if ((LORA || NORM) && bx < p.producers) {  // (a segment without LoRA or norm has none)
        lora_producer<MT, NORM>(d, bx, lds);
        return;
    }
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
    const int64_t u = bx - p.producers;
    const int64_t slice = u / p.row_blocks, rblk = u - slice * p.row_blocks;
    const int64_t c_begin = slice * p.cps;  // a multiple of 4 chunks
    const int64_t c_end = c_begin + p.cps < p.chunks ? c_begin + p.cps : p.chunks;
    const int64_t c_full_end = c_end < p.full_chunks ? c_end : p.full_chunks;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t R = p.rows_per_unit;
    const int64_t n_unit = rblk * R;
    const int64_t n0 = n_unit + (int64_t)wave * 16 * NW;
    const int m_last = (int)a.m - 1;

    f32x4_t acc[MT][NW];
    acc[0][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's weight row (rows past n repeat row n - 1; their outputs are
    // discarded) and x row (rows past m repeat row m - 1)
    const int64_t nrow = n0 + lr < a.n ? n0 + lr : a.n - 1;
    const uint8_t *prow = a.packed + nrow * (a.k >> 1);
    const uint8_t *srow = a.scales + nrow * (a.k >> 4);
    const uint16_t *xrow = xs + (lr < m_last ? lr : m_last) * p.xpitch;
    // whole 512-element groups of the slice in the span layout (k % 128 == 0
    // keeps their 16-byte code and 8-byte scale loads aligned); the other
    // chunks, if any, in the chunk layout
    const int64_t ng = (a.k & 127) == 0 ? (c_full_end - c_begin) / 4 : 0;
    // ---- the first group's loads travel while the x slice is staged ----
    SpanGroup cur;
    if (ng > 0) cur = load_span_group(prow, srow, c_begin / 4, lq);
    stage_x_slice<NORM, kThreadsS>(a, xs, p.xpitch, c_begin * kChunkK, (c_end - c_begin) * kChunkK);
    __syncthreads();
    // One group in flight per wave: latency is covered by the other resident
    // units and waves (registers kept low for that), not by a deeper ring.
    for (int64_t gl = 0; gl < ng; ++gl) {
        if (gl > 0) cur = load_span_group(prow, srow, c_begin / 4 + gl, lq);
        mma_span_group(cur, xrow + gl * kGroupK + 128 * lq, acc[0][0]);
    }
    // the remaining full chunks (k % 512 != 0 or k % 128 != 0), chunk layout
    for (int64_t c = c_begin + 4 * ng; c < c_full_end; ++c) {
        uint4 w[NW];
        load_chunk<NW, K32>(a, n0, c, lr, lq, w);
        const uint32_t s2 = load_scale_pair<K32>(srow, c * 8 + 2 * lq, a.k >> 4);
        mma_chunk_sc(w[0], s2, xrow + (c - c_begin) * kChunkK + 32 * lq, acc[0][0]);
    }
    if (c_end > c_full_end) {  // the partial last chunk of K (k % 128 != 0): zeros past k
        uint4 wt[NW];
        load_chunk_tail<NW>(a, n0, p.full_chunks, lr, lq, wt);
        const uint32_t s2 = load_scale_pair<false>(srow, p.full_chunks * 8 + 2 * lq, a.k >> 4);
        mma_chunk_sc(wt[0], s2, xrow + (p.full_chunks - c_begin) * kChunkK + 32 * lq, acc[0][0]);
    }
    // Lane (lr, lq) holds rows 4 lq .. 4 lq + 3 of column n0 + lr.
    if (DIRECT) {
        const float st = *a.tensor_scale;
        const int64_t n = n0 + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = 4 * lq + v;
            if (m < a.m && n < a.n) a.y[m * a.ldy + n] = f32_to_bf16_bits(st * acc[0][0][v]);
        }
    } else if (4 * lq < a.m) {  // this unit's FP32 tile, slot wave * 64 + lane
        reinterpret_cast<f32x4_t *>(d.part() + u * (R * 16))[wave * 64 + lane] = acc[0][0];
    }
}

// ---------------------------------------------------------------------------
// finish_kernel: y from the partial tiles of the main kernel
// ---------------------------------------------------------------------------
// Workgroup: 64 columns x one 16-row m-tile of one segment, 256 threads, one
// round trip of loads (every load a thread needs is issued before any is
// used), then two LDS stages; every sum runs in the same order on every call.
//  * t of the m-tile's rows: the producers' tiles summed over the K ranges
//    (at most kMaxProdRanges).  Each (rank tile, lane) item has P threads
//    that sum contiguous runs of K ranges, added in order through LDS.
//  * NORM: the rows' 1 / rms from the producers' sums of squares (K-range
//    order), as the standalone norm forms it.
//  * Output (n, quad) -- rows 4 quad .. 4 quad + 3 of column n, which one
//    lane of one unit tile holds as a float4 -- takes 4 / Q threads (Q quads
//    in the tile): thread part p sums its run of slices in order and its run
//    of ranks of the LoRA dot; the parts are added in order.
//  y = bf16(inv (s_t acc + lora_scale t B[n]^T)).
template <int NS, int MT, int NW, bool NORM>
__global__ __launch_bounds__(256) void finish_kernel(DecodeSetN<NS> ds) {
    constexpr int kFinS = 8, kFinB = 4, kFinT = 8;  // loads of each kind issued at once
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.z];
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    const int64_t bx = blockIdx.x;
    if (NS > 1 && bx * 64 >= a.n) return;  // past a narrower segment
    __shared__ float ts[16][kMaxRank];
    __shared__ f32x4_t tred[512];
    __shared__ f32x4_t ored[2][256];
    __shared__ float s_inv[16];
    const int tid = threadIdx.x, col = tid & 63, h = tid >> 6;
    const int mt = (int)blockIdx.y;
    const int64_t rows = a.m - 16 * (int64_t)mt < 16 ? a.m - 16 * (int64_t)mt : 16;
    const int Q = (int)((rows + 3) / 4), P = Q == 1 ? 4 : (Q == 2 ? 2 : 1);
    const int quad_l = h % Q, part = h / Q;  // part < P, except the idle h = 3 when Q = 3
    const int64_t n = bx * 64 + col, quad = (int64_t)mt * 4 + quad_l;
    const bool out = n < a.n && part < P;
    // this output's place in the units' tiles
    const int64_t R = p.rows_per_unit;
    const int64_t nc = n < a.n ? n : a.n - 1;
    const int64_t rblk = nc / R, rem = nc - rblk * R;
    const int64_t wave = rem / (16 * NW), g = (rem / 16) % NW, lr = rem % 16;
    const int64_t lq = quad % 4;
    // m-tile mt is m-tile mt % MT of m-block mt / MT, whose units follow those
    // of the m-blocks before it (only units of eight m-tiles have several)
    const int mtl = MT == 8 ? mt % MT : mt;
    const int64_t mblk = MT == 8 ? mt / MT : 0;
    const int64_t slot = ((wave * MT + mtl) * NW + g) * 64 + lq * 16 + lr;
    const int64_t tile_floats = R * 16 * MT;
    const float *part_base = d.part() + (mblk * p.slices * p.row_blocks + rblk) * tile_floats + slot * 4;
    const int64_t sstride = p.row_blocks * tile_floats;  // floats between slices
    const int pp = part < P ? part : 0;
    const int64_t s0 = p.slices * pp / P, s1 = p.slices * (pp + 1) / P;
    // ---- issue: this part's slice tiles, its ranks of B[n], its share of t ----
    f32x4_t pv[kFinS];
#pragma unroll
    for (int u = 0; u < kFinS; ++u) {
        const int64_t sl = s0 + u < s1 ? s0 + u : (s1 > s0 ? s1 - 1 : s0);
        pv[u] = *reinterpret_cast<const f32x4_t *>(part_base + sl * sstride);
    }
    const bool r8 = (a.r & 7) == 0;
    const int units8 = a.r / 8;  // 8-rank pieces of B (r % 8 == 0)
    const int b0 = r8 ? units8 * pp / P : 0, b1 = r8 ? units8 * (pp + 1) / P : 0;
    const uint16_t *br = a.lora_b + nc * a.r;
    uint4 bq[kFinB];
#pragma unroll
    for (int u = 0; u < kFinB; ++u)
        bq[u] = b0 + u < b1 ? *reinterpret_cast<const uint4 *>(br + 8 * (b0 + u)) : make_uint4(0, 0, 0, 0);
    const int JT = (int)p.jt, items = JT * 64, PT = items >= 256 ? 1 : 256 / items;
    const f32x4_t *tp = reinterpret_cast<const f32x4_t *>(d.tpart()) + ((int64_t)mt * JT) * 64;
    const int64_t kstride = (int64_t)(MT == 8 ? p.mtp : MT) * JT * 64;  // f32x4 between K ranges
    // (r <= 64: one (item, run) per thread; larger ranks take a second one)
    auto t_run = [&](int w, int64_t &kr0, int64_t &kr1) {
        const int q = w / items;
        kr0 = p.prod_kr * q / PT;
        kr1 = p.prod_kr * (q + 1) / PT;
    };
    f32x4_t tv[kFinT];
    const bool t_mine = a.r > 0 && tid < items * PT;
    int64_t kr0 = 0, kr1 = 0;
    if (t_mine) {
        t_run(tid, kr0, kr1);
        const f32x4_t *src = tp + tid % items;
#pragma unroll
        for (int u = 0; u < kFinT; ++u) tv[u] = src[(kr0 + u < kr1 ? kr0 + u : (kr1 > kr0 ? kr1 - 1 : kr0)) * kstride];
    }
    float ssv[kMaxProdRanges];
    if (NORM && tid < 16)
#pragma unroll
        for (int q = 0; q < kMaxProdRanges; ++q) ssv[q] = q < p.prod_kr ? d.ssp()[q * 16 + tid] : 0.0f;
    // ---- t and 1 / rms ----
    if (t_mine) {
        f32x4_t sum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < kFinT; ++u)
            if (kr0 + u < kr1) sum = sum + tv[u];
        for (int64_t k0 = kr0 + kFinT; k0 < kr1; ++k0)  // (more ranges than kFinT: never with the plan's bound)
            sum = sum + tp[tid % items + k0 * kstride];
        tred[tid] = sum;  // = tred[q * items + item]
    }
    for (int w = tid + 256; a.r > 0 && w < items * PT; w += 256) {  // r > 64
        int64_t k0, k1;
        t_run(w, k0, k1);
        f32x4_t sum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t k = k0; k < k1; ++k) sum = sum + tp[w % items + k * kstride];
        tred[w] = sum;
    }
    if (NORM && tid < 16) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < kMaxProdRanges; ++q) tot += ssv[q];  // zeros past prod_kr
        s_inv[tid] = 1.0f / sqrtf(tot * (1.0f / (float)a.k) + a.norm_eps);
    }
    __syncthreads();
    if (a.r > 0) {
        for (int item = tid; item < items; item += 256) {
            f32x4_t t = tred[item];
            for (int q = 1; q < PT; ++q) t = t + tred[q * items + item];
            // tile jt, lane l: t[4 (l / 16) + v][16 jt + l % 16]
            const int jt = item / 64, l = item % 64, j = 16 * jt + (l & 15);
            if (j < a.r)
#pragma unroll
                for (int v = 0; v < 4; ++v) ts[4 * (l >> 4) + v][j] = t[v];
        }
        __syncthreads();
    }
    // ---- this part's slices and ranks ----
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kFinS; ++u)
        if (s0 + u < s1) acc = acc + pv[u];
    constexpr int kFinS2 = 4;  // more slices: this many loads at a time, same order
    for (int64_t sb = s0 + kFinS; sb < s1; sb += kFinS2) {
        f32x4_t pw[kFinS2];
#pragma unroll
        for (int u = 0; u < kFinS2; ++u)
            pw[u] = *reinterpret_cast<const f32x4_t *>(part_base + (sb + u < s1 ? sb + u : s1 - 1) * sstride);
#pragma unroll
        for (int u = 0; u < kFinS2; ++u)
            if (sb + u < s1) acc = acc + pw[u];
    }
    f32x4_t lora = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int q0 = quad_l * 4;  // this output's first row in ts
    auto dot8 = [&](const uint4 &b8, int j) {
        const uint32_t bw[4] = {b8.x, b8.y, b8.z, b8.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                lora[v] = __builtin_fmaf(ts[q0 + v][j + 2 * e], bf16lo_to_f32(bw[e]), lora[v]);
                lora[v] = __builtin_fmaf(ts[q0 + v][j + 2 * e + 1], bf16hi_to_f32(bw[e]), lora[v]);
            }
    };
    if (r8) {
#pragma unroll
        for (int u = 0; u < kFinB; ++u)
            if (b0 + u < b1) dot8(bq[u], 8 * (b0 + u));
        for (int u = b0 + kFinB; u < b1; ++u) dot8(*reinterpret_cast<const uint4 *>(br + 8 * u), 8 * u);
    } else if (pp == 0) {  // r % 8 != 0: the first part takes every rank
        for (int j = 0; j < a.r; ++j) {
            const float b = bf16lo_to_f32(br[j]);
#pragma unroll
            for (int v = 0; v < 4; ++v) lora[v] = __builtin_fmaf(ts[q0 + v][j], b, lora[v]);
        }
    }
    ored[0][tid] = acc;
    ored[1][tid] = lora;
    __syncthreads();
    if (!out || part != 0) return;
    for (int q = 1; q < P; ++q) {  // the parts in order
        acc = acc + ored[0][(q * Q + quad_l) * 64 + col];
        lora = lora + ored[1][(q * Q + quad_l) * 64 + col];
    }
    const float st = *a.tensor_scale, lam = a.lora_scale;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t m = 4 * quad + v;
        const float y = st * acc[v] + lam * lora[v];
        if (m < a.m) a.y[m * a.ldy + n] = f32_to_bf16_bits(NORM ? s_inv[q0 + v] * y : y);
    }
}

// ---------------------------------------------------------------------------
// 16 < m: MFMA units
// ---------------------------------------------------------------------------
// Unit u = (slice of K, block of 64 kUnitWaves weight rows) runs the K loops
// of mfma_tile.h over its chunks with all 16 MT rows of x as the x tile, so
// the eight waves share one x tile (x bytes per weight byte halve against
// four waves).  It stores its FP32 tile where finish_kernel<MT, NW> reads it,
// NW = 4 kUnitWaves / kWaves n-tiles per wave of a four-wave layout: wave w's
// n-tile j (unit rows 64w + 16j ..) is n-tile (4w + j) % NW of layout wave
// w / (kUnitWaves / kWaves), so m-tile i goes to f32x4 slot
// ((layout wave MT + i) NW + (4w + j) % NW) 64 + lane.  Producers of t lead the grid, as in stream_kernel; only
// the first four waves of a producer work.
__shared__ __attribute__((aligned(1024))) uint8_t g_dxtile0[64 * kTileRowBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_dxtile1[64 * kTileRowBytes];
// the x tiles of eight m-tiles (m > 64: one 128-row m-block), a kernel of their own
__shared__ __attribute__((aligned(1024))) uint8_t g_dxtile8_0[128 * kTileRowBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_dxtile8_1[128 * kTileRowBytes];
// the unit's scale bytes (256 rows x its slice), when they fit: 2-byte
// global loads of 16 rows each cost more of the CU's memory path than the
// weights they scale
__shared__ __attribute__((aligned(16))) uint8_t g_dsc[kUnitScBytes];

// one workgroup of mfma_unit_kernel: a LoRA producer or a unit
// SCL: the unit's scales staged in LDS (p.unit_sc)
template <int MT, bool SCL>
__device__ __forceinline__ void mfma_unit(const Decode &d, int64_t bx) {
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    if (bx < p.producers) {
        lora_producer<MT>(d, bx, MT == 8 ? g_dxtile8_0 : g_dxtile0);
        return;
    }
    constexpr int NW = 4 * kUnitWaves / kWaves;  // n-tiles per wave of the four-wave tile layout
    constexpr int kPer = kUnitWaves / kWaves;     // unit waves per layout wave
    int64_t u = bx - p.producers;
    // unit u: m-block mbi (16 MT rows of x), then slice, then row block.  With
    // several m-blocks the grid runs the units of one (slice, row block) eight
    // workgroups apart, so that they share an XCD (workgroups go to the XCDs
    // in turn) and its L2 copy of the weights: u is recovered from the
    // position v as below (the last group of fewer than eight in order)
    if (MT == 8 && p.mb > 1) {
        const int64_t W = p.slices * p.row_blocks, full = W / 8 * 8, v = u;
        int64_t w, mb_i;
        if (v < full * p.mb) {
            const int64_t q = v / 8;
            mb_i = q % p.mb;
            w = q / p.mb * 8 + v % 8;
        } else {
            const int64_t t = v - full * p.mb;
            w = full + t / p.mb;
            mb_i = t % p.mb;
        }
        u = mb_i * W + w;
    }
    const int64_t mbi = MT == 8 ? u / (p.slices * p.row_blocks) : 0, us = u - mbi * p.slices * p.row_blocks;
    const int64_t slice = us / p.row_blocks, rblk = us - slice * p.row_blocks;
    const uint16_t *xb = a.x + mbi * 16 * MT * a.ldx;  // this m-block's rows of x
    const int64_t mrows = a.m - mbi * 16 * MT < 16 * MT ? a.m - mbi * 16 * MT : 16 * MT;
    const int64_t c_begin = slice * p.cps;
    const int64_t c_end = c_begin + p.cps < p.chunks ? c_begin + p.cps : p.chunks;
    const int64_t c_full_end = c_end < p.full_chunks ? c_end : p.full_chunks;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t n0 = rblk * p.rows_per_unit, kb = a.k >> 1, ks = a.k >> 4;

    f32x4_t acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t fast_end = a.ldx <= kTileMaxLdx ? c_full_end : c_begin;
    static_assert(64 * kUnitWaves == kThreadsD, "the staging helpers assume kThreadsD threads");
    if (SCL && fast_end > c_begin) {  // (uniform) the slice's full blocks; visible after the barrier
        stage_scales(a, g_dsc, p.unit_sc_pitch, n0, p.rows_per_unit, c_begin * 8, (fast_end - c_begin) * 8);
        __syncthreads();
    }
    mfma_kloop<MT, kUnitWaves, 1, SCL>(xb, mrows, a.ldx, a.packed + n0 * kb, a.scales + n0 * ks, a.n - n0, a.k,
                                       c_begin, fast_end, MT == 8 ? g_dxtile8_0 : g_dxtile0,
                                       MT == 8 ? g_dxtile8_1 : g_dxtile1, acc, g_dsc, (int)p.unit_sc_pitch);
    // the rest of the slice (the partial last chunk of K, or all of it for
    // very wide x rows)
    const int64_t nw = n0 + wave * 64 + lr;
    plain_kloop<MT, kUnitWaves>(
        fast_end * kChunkK, c_end * kChunkK < a.k ? c_end * kChunkK : a.k, MT == 8 ? g_dxtile8_0 : g_dxtile0,
        [&](int row, int64_t kk) {
            uint4 o = make_uint4(0, 0, 0, 0);
            if (row < mrows && kk < a.k) o = *reinterpret_cast<const uint4 *>(xb + row * a.ldx + kk);
            return o;
        },
        [&](int j, int64_t kk) {
            const int64_t n = nw + 16 * j;
            if (n < a.n && kk < a.k)  // k % 16 == 0: an 8-element piece is inside or outside
                return dequant8_p(*reinterpret_cast<const uint32_t *>(a.packed + n * kb + (kk >> 1)),
                                  QERL_E4M3_F32(a.scales[n * ks + (kk >> 4)], 0));
            return as_bf16x8_d(make_uint4(0, 0, 0, 0));
        },
        acc);

    f32x4_t *tile = reinterpret_cast<f32x4_t *>(d.part() + u * (p.rows_per_unit * 16 * MT)) + lane;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (16 * i + 4 * lq < mrows) tile[(((wave / kPer) * MT + i) * NW + (4 * wave + j) % NW) * 64] = acc[i][j];
}

template <int NS, int MT, bool SCL>
__global__ __launch_bounds__(64 * kUnitWaves) void mfma_unit_kernel(DecodeSetN<NS> ds) {
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.y];
    if (NS > 1 && (int64_t)blockIdx.x >= d.p.producers + d.p.units) return;  // past a narrower segment
    mfma_unit<MT, SCL>(d, blockIdx.x);
}

// the finish launch: (column blocks of the widest segment) x m-tiles x segments
template <int NS, int MT, int NW, bool NORM>
hipError_t launch_finish(const DecodeSetN<NS> &ds, hipStream_t stream) {
    int64_t fblocks = 0;
    for (int i = 0; i < ds.nseg; ++i) {
        const int64_t f = (ds.seg[i].a.n + 63) / 64;
        fblocks = f > fblocks ? f : fblocks;
    }
    const dim3 fgrid((unsigned)fblocks, (unsigned)((ds.seg[0].a.m + 15) / 16), (unsigned)ds.nseg);
    hipLaunchKernelGGL((finish_kernel<NS, MT, NW, NORM>), fgrid, dim3(256), 0, stream, ds);
    return hipGetLastError();
}

template <int MT, int NS>
hipError_t launch_mfma_units(const DecodeSetN<NS> &ds, hipStream_t stream) {
    const Decode &d = ds.seg[0];  // the unit shape and scale staging are shared by the segments
    int64_t blocks = 0;
    for (int i = 0; i < ds.nseg; ++i) {
        const int64_t b = ds.seg[i].p.producers + ds.seg[i].p.units;
        blocks = b > blocks ? b : blocks;
    }
    const dim3 grid((unsigned)blocks, (unsigned)ds.nseg);
    if (d.p.unit_sc)
        hipLaunchKernelGGL((mfma_unit_kernel<NS, MT, true>), grid, dim3(64 * kUnitWaves), 0, stream, ds);
    else
        hipLaunchKernelGGL((mfma_unit_kernel<NS, MT, false>), grid, dim3(64 * kUnitWaves), 0, stream, ds);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_finish<NS, MT, 4 * kUnitWaves / kWaves, false>(ds, stream);
}

template <bool K32, bool DIRECT, bool LORA, bool NORM, int NS>
hipError_t launch_stream(const DecodeSetN<NS> &ds, int64_t lds_bytes, hipStream_t stream) {
    auto kern = stream_kernel<NS, K32, DIRECT, LORA, NORM>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    if (attr != hipSuccess) return attr;
    int64_t blocks = 0;
    for (int i = 0; i < ds.nseg; ++i) {
        const int64_t b = ds.seg[i].p.producers + ds.seg[i].p.units;
        blocks = b > blocks ? b : blocks;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks, (unsigned)ds.nseg), dim3(kThreadsS), (size_t)lds_bytes, stream, ds);
    const hipError_t e = hipGetLastError();
    if (DIRECT || e != hipSuccess) return e;
    return launch_finish<NS, 1, 1, NORM>(ds, stream);
}

template <bool K32, int NS>
hipError_t launch_stream(const DecodeSetN<NS> &ds, int64_t lds_bytes, bool lora, bool direct, hipStream_t stream) {
    if (ds.seg[0].p.norm) {  // the norm prologue: k % 32 == 0 only (checked by the caller)
        if constexpr (K32) {
            return lora ? launch_stream<K32, false, true, true>(ds, lds_bytes, stream)
                        : launch_stream<K32, false, false, true>(ds, lds_bytes, stream);
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (direct) return launch_stream<K32, true, false, false>(ds, lds_bytes, stream);
    return lora ? launch_stream<K32, false, true, false>(ds, lds_bytes, stream)
                : launch_stream<K32, false, false, false>(ds, lds_bytes, stream);
}

// the plans of a launch over segs[0 .. nseg) (shared x), slices shared
DecodeSet make_decode_set(const GemmArgs *segs, int nseg) {
    DecodeSet ds{};
    ds.nseg = nseg;
    const bool norm = segs[0].norm_w != nullptr;
    int64_t rows = 0;
    for (int i = 0; i < nseg; ++i)
        rows += make_decode_plan(segs[i].m, segs[i].n, segs[i].k, segs[i].r, 0, norm).row_blocks;
    char *base = static_cast<char *>(segs[0].workspace);  // one workspace for the launch
    int64_t data = 0;
    for (int i = 0; i < nseg; ++i) {
        ds.seg[i].a = segs[i];
        ds.seg[i].p = make_decode_plan(segs[i].m, segs[i].n, segs[i].k, segs[i].r, rows, norm);
        ds.seg[i].a.workspace = base + data;
        data += align256(ds.seg[i].p.bytes);
    }
    return ds;
}

template <int NS>
hipError_t launch_checked(const DecodeSetN<NS> &ds, int64_t lds, bool lora, bool direct, hipStream_t stream) {
    const Decode &d0 = ds.seg[0];
    if (d0.p.mt == 2) return launch_mfma_units<2>(ds, stream);
    if (d0.p.mt == 4) return launch_mfma_units<4>(ds, stream);
    if (d0.p.mt == 8) return launch_mfma_units<8>(ds, stream);
    return (d0.a.k & 31) == 0 ? launch_stream<true>(ds, lds, lora, direct, stream)
                              : launch_stream<false>(ds, lds, lora, direct, stream);
}

hipError_t launch_decode_set(const DecodeSet &ds, hipStream_t stream) {
    int64_t lds = 0;
    bool lora = false, direct = true;
    for (int i = 0; i < ds.nseg; ++i) {
        const Decode &d = ds.seg[i];
        if (d.p.row_blocks < 1 || d.p.lds_bytes > kLdsLimit ||
            d.p.rows_per_unit * 16 * d.p.mt * d.p.units * 4 > 0x7FFFFFFF)
            return hipErrorInvalidConfiguration;
        if (d.p.slices != ds.seg[0].p.slices || d.p.unit_sc != ds.seg[0].p.unit_sc || d.p.norm != ds.seg[0].p.norm ||
            (d.a.norm_w != nullptr) != d.p.norm)
            return hipErrorInvalidConfiguration;
        lds = d.p.lds_bytes > lds ? d.p.lds_bytes : lds;
        lora = lora || d.a.r > 0;
        direct = direct && d.p.direct_out;
    }
    for (int i = 0; i < ds.nseg; ++i)
        if (ds.seg[i].p.producers + ds.seg[i].p.units > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (ds.nseg == 1) return launch_checked(DecodeSetN<1>{{ds.seg[0]}, 1}, lds, lora, direct, stream);
    return launch_checked(ds, lds, lora, direct, stream);
}

}  // namespace

size_t decode_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    return (size_t)align256(make_decode_plan(m, n, k, r).bytes);
}

hipError_t launch_decode(const GemmArgs &a, hipStream_t stream) {
    return launch_decode_set(make_decode_set(&a, 1), stream);
}

size_t decode_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm) {
    int64_t rows = 0;
    for (int j = 0; j < nseg; ++j) rows += make_decode_plan(m, n[j], k, r[j], 0, norm).row_blocks;
    int64_t bytes = 0;
    for (int j = 0; j < nseg; ++j) bytes += align256(make_decode_plan(m, n[j], k, r[j], rows, norm).bytes);
    return (size_t)bytes;
}

hipError_t launch_decode_multi(const GemmArgs *segs, int nseg, hipStream_t stream) {
    if (nseg < 1 || nseg > kMaxSegments) return hipErrorInvalidValue;
    return launch_decode_set(make_decode_set(segs, nseg), stream);
}

// The furthest workspace byte each kernel of a decode launch addresses,
// recomputed from the plan fields its indexing uses, against the size query
// the caller sized the workspace by; and the grid and LDS limits the
// launcher relies on.
int decode_plan_check(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm, char *msg,
                      size_t len) {
    auto fail = [&](const char *what, int64_t seg, int64_t a, int64_t b) {
        snprintf(msg, len, "decode m=%lld k=%lld segment %lld: %s (%lld > %lld)", (long long)m, (long long)k,
                 (long long)seg, what, (long long)a, (long long)b);
        return 1;
    };
    if (nseg < 1 || nseg > kMaxSegments) return fail("segment count", 0, nseg, kMaxSegments);
    const int64_t size = nseg == 1 && !norm ? (int64_t)decode_workspace_bytes(m, n[0], k, r[0])
                                            : (int64_t)decode_multi_workspace_bytes(m, k, n, r, nseg, norm);
    int64_t rows = 0;
    for (int j = 0; j < nseg; ++j) rows += make_decode_plan(m, n[j], k, r[j], 0, norm).row_blocks;
    int64_t off = 0, slices0 = -1;
    for (int j = 0; j < nseg; ++j) {
        const DecodePlan p = make_decode_plan(m, n[j], k, r[j], rows, norm);
        if (p.row_blocks < 1) return fail("no row blocks", j, 1, p.row_blocks);
        if (slices0 < 0) slices0 = p.slices;
        if (p.slices != slices0) return fail("slices differ between segments", j, p.slices, slices0);
        if (p.row_blocks * p.rows_per_unit < n[j]) return fail("rows not covered", j, n[j], p.row_blocks * p.rows_per_unit);
        if (p.slices * p.cps < p.chunks) return fail("K not covered", j, p.chunks, p.slices * p.cps);
        const int64_t tile = p.rows_per_unit * 16 * p.mt * 4;  // bytes of one unit's FP32 tile
        // f32x4 slots a unit writes: stream_kernel wave * 64 + lane; an MFMA
        // unit ((layout wave MT + i) NW + n-tile) 64 + lane
        const int64_t slots = p.mt == 1 ? (int64_t)kSW * 64 : (int64_t)4 * p.mt * p.nw * 64;
        if (slots * 16 > tile) return fail("unit tile slots", j, slots * 16, tile);
        if (p.units != p.row_blocks * p.slices * p.mb) return fail("units", j, p.units, p.row_blocks * p.slices * p.mb);
        if ((int64_t)p.mb * 16 * p.mt < m) return fail("m-blocks", j, m, (int64_t)p.mb * 16 * p.mt);
        const int64_t units_end = p.part_off + p.units * tile;  // written by the units, read by finish_kernel
        if (units_end > p.tpart_off) return fail("unit tiles past their region", j, units_end, p.tpart_off);
        // producers: f32x4 (mt JT + rank tile) 64 + lane of K range kr < prod_kr
        const int64_t prod_end = p.tpart_off + (p.producers ? p.prod_kr * p.mtp * p.jt * 64 * 16 : 0);
        if (prod_end > p.ss_off) return fail("producer tiles past their region", j, prod_end, p.ss_off);
        const int64_t ss_end = p.ss_off + (p.norm && p.producers ? p.prod_kr * 16 * 4 : 0);
        if (ss_end > p.bytes) return fail("sums of squares past the plan", j, ss_end, p.bytes);
        if (p.producers && p.prod_kr > kMaxProdRanges) return fail("producer K ranges", j, p.prod_kr, kMaxProdRanges);
        if (p.producers + p.units > 0x7FFFFFFF) return fail("grid", j, p.producers + p.units, 0x7FFFFFFF);
        if (p.mt == 1 && p.lds_bytes > kLdsLimit) return fail("LDS", j, p.lds_bytes, kLdsLimit);
        off += align256(p.bytes);
        if (off > size) return fail("segment data past the size query", j, off, size);
    }
    return 0;
}

}  // namespace qerl
