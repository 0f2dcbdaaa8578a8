// decode.hip -- W4A16 (NVFP4 weight x BF16 activation) + LoRA for decode
// batches, 1 <= m <= 64, on gfx950.
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
// e4m3 has <= 6 significant bits) and multiplied on the 16x16x32 BF16 MFMA in
// FP32; K is permuted inside each 128-element chunk, identically for both
// operands, so that one 16-byte load gives a lane the packed bytes of four
// MFMA steps.
//
// m <= 16, stream_kernel, one launch per call.  Work units are (64 weight
// rows) x (slice of K); each of the 4 waves of a unit owns 16 rows.
//  * The unit's x slice and E4M3 scales are staged into LDS once with batched
//    wide loads; the weights stream in 128-element chunks (64 packed bytes per
//    row) through a ring of DR chunks per wave, with no barrier.  Every load
//    of the steady state is unconditional, which keeps the compiler's
//    in-order wait counts exact; LDS reads are counted apart from them.
//  * LoRA: "producer" workgroups at the head of the grid compute partial sums
//    of t = x A^T over slices of K (MFMA) and publish them with device-coherent
//    stores; the last producer to finish sums them in producer order and
//    publishes t once, as BF16 hi + lo halves (relative error ~2^-16) in the
//    layout the epilogue multiplies, behind a ready flag.  Short units with
//    few producers ("direct") instead wait for the producers' count and sum
//    their partials themselves, which takes the last-producer stage off the
//    chain.
//  * Every unit but the last of its row block stores its FP32 partial tile
//    (coherent stores) and bumps a counter.  The last to arrive (every unit,
//    when K is not split) loads all partial tiles and t in one batch -- the
//    ready flag was read while its last chunks multiplied, so as a rule no
//    round trip of its own is spent on t (the wait for it is bounded all the
//    same) -- sums the partials in slice order (deterministic), and adds
//    lora_scale * t B^T on the MFMA.
//  * NORM (an RMSNorm of x fused in front): the units stage bf16(x * norm_w),
//    the producers also sum x^2 per K range, and 1 / rms scales t and the
//    output row in the epilogue (a row's 1 / rms factors out of the product).
//  * Several projections of one x (q/k/v, gate/up) share a launch: the
//    segment is a grid dimension; a one-segment launch is its own
//    instantiation with a one-plan argument.
//
// 16 < m <= 64, mfma_unit_kernel + finish_kernel, two launches.  Units are
// (256 weight rows) x (slice of K) running the K loops of mfma_tile.h with all
// of x as the x tile; every unit stores its FP32 tile and finish_kernel sums
// them (in slice order) in parallel over the outputs; the last producer sums
// t, which finish_kernel reads after the kernel boundary.
//
// Counters live in the first kGemmCtrBytes of the workspace: they must be zero
// before the first call, and every call leaves them zero.
#include "device_common.h"
#include "mfma_tile.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreadsD = kWaves * 64;
// waves of a 16 < m unit (64 weight rows each).  Eight waves sharing one x
// tile, or weights fetched two blocks ahead, were measured slower: the unit is
// bound by its CU's vector memory path, not by latency.
constexpr int kUnitWaves = 4;
constexpr int64_t kChunkK = 128;          // K elements per chunk
constexpr int kXPad = 8;                  // BF16 padding per staged x row
constexpr int64_t kScBudget = 24 * 1024;  // LDS for the unit's scales
constexpr int64_t kXBudget = 96 * 1024;   // LDS for a unit's x slice (m <= 16)
constexpr int64_t kLdsLimit = 140 * 1024;  // of the 160 KiB a gfx950 workgroup may hold
constexpr int64_t kProdChunks = 4;        // K chunks per LoRA producer
constexpr int kProdTiles = 2;            // rank tiles a producer accumulates at once
constexpr int kBatch = 8;                // loads in flight per thread in reductions and staging
constexpr int kMaxRank = 128;            // QERL_MAX_LORA_RANK
constexpr uint32_t kSpinLimit = 1u << 20;  // polls of the bounded wait for t (2^20 x s_sleep 2)
constexpr int64_t kUnitScBytes = 24 * 1024;  // 16 < m: LDS for a unit's scale tile
constexpr int64_t kUnitMinChunks = 8;        // 16 < m: K chunks per unit the split may go down to
constexpr int64_t kDirectMaxKr = 8;          // m <= 16: most producer K ranges the epilogue sums itself
constexpr int64_t kDirectMaxCps = 12;        // ... in units of at most this many chunks
#ifndef QERL_RING
#define QERL_RING 4
#endif
constexpr int kRing = QERL_RING;  // weight chunks in flight per wave (m <= 16)

// counter words at the head of the workspace; kCtrErr is the segment's error
// word (kGemmErrWaitTimeout when a bounded wait gave up), read by
// gemm_workspace_check and cleared by gemm_workspace_reset
constexpr int kCtrProd = 0, kCtrTReady = 1, kCtrDone = 2, kCtrErr = kGemmCtrErrWord, kCtrRow = 4;
static_assert(kCtrErr == 3, "the error word sits between the fixed counters and the row counters");
constexpr int64_t kMaxRowBlocks = kSegCtrBytes / 4 - kCtrRow;

struct DecodePlan {
    int mt, nw, px;
    int64_t rows_per_unit, row_blocks;
    int64_t chunks, full_chunks;   // chunks of K (the last may be partial), full chunks
    int64_t cps, slices, units;    // chunks per slice (a multiple of 4/nw)
    int64_t producers, jt, rp;     // LoRA producers, 16-wide rank tiles, rank padded to 32
    int64_t prod_kr, prod_groups;  // producers: K ranges x (m-tile, rank-tile pair) groups
    int64_t xpitch, sc_pitch;      // LDS pitches: BF16 elements per x row, bytes per scale row
    int64_t sc_lds_off, lds_bytes;
    int64_t unit_sc_pitch;         // 16 < m: LDS pitch of the unit's scale tile
    bool unit_sc;                  // 16 < m: scales staged in LDS
    int64_t part_off, tpart_off, t_off, bytes;
    // RMSNorm prologue (m <= 16): the producers' per-K-range sums of squares
    // [prod_kr][16] at ss_off, and the rows' 1 / rms [16] after t16 at inv_off
    bool norm;
    int64_t ss_off, inv_off;
    // m <= 16 with few producer K ranges (and r <= 64): the epilogue sums the
    // producers' partial tiles itself, so t costs no last-producer stage
    bool direct;
    // the bounded wait for t: polls before giving up, and a count added to
    // the value waited for (nonzero only when the host forces every such wait
    // to give up, to test that failure is reported)
    uint32_t spin_limit, wait_bias;
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
    p.mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    p.nw = p.mt == 1 ? 1 : kUnitWaves * 4 / kWaves;  // 16 < m: MFMA units of 64 kUnitWaves weight rows
    p.rows_per_unit = 16 * kWaves * (int64_t)p.nw;
    p.row_blocks = (n + p.rows_per_unit - 1) / p.rows_per_unit;
    if (p.row_blocks > kMaxRowBlocks) p.row_blocks = 0;  // one counter per row block: rejected at launch
    p.chunks = (k + kChunkK - 1) / kChunkK;
    p.full_chunks = k / kChunkK;
    p.px = 1;
    p.jt = (r + 15) / 16;
    p.rp = (r + 31) / 32 * 32;
    p.prod_kr = (p.chunks + kProdChunks - 1) / kProdChunks;
    p.prod_groups = p.mt * ((p.jt + kProdTiles - 1) / kProdTiles);
    p.norm = norm && p.mt == 1;
    p.spin_limit = g_force_wait_timeout ? 1u : kSpinLimit;
    p.wait_bias = g_force_wait_timeout ? 1u : 0u;
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
        // fewer row blocks than CUs split K as above; more keep at least
        // kUnitMinChunks chunks per unit but still split K (several units
        // per CU keep more loads in flight than one long unit)
        const int64_t s_work = p.chunks / kUnitMinChunks;
        if (s < s_work) s = s_work < s_cap ? s_work : s_cap;
        p.cps = (p.chunks + s - 1) / s;
        p.slices = (p.chunks + p.cps - 1) / p.cps;
        p.units = p.row_blocks * p.slices;
        int64_t scp = (p.cps * 8 + 15) / 16;  // rows an odd multiple of 16 bytes apart
        if (scp % 2 == 0) ++scp;
        p.unit_sc_pitch = scp * 16;
        p.unit_sc = p.rows_per_unit * p.unit_sc_pitch <= kUnitScBytes;
        p.part_off = 0;  // offsets from the segment's data (after the counter head)
        p.tpart_off = align256(p.part_off + p.units * tile);
        p.t_off = align256(p.tpart_off + p.prod_kr * (int64_t)p.mt * p.jt * 64 * 16);
        p.bytes = align256(p.t_off + m * (int64_t)r * 4);
        return p;
    }
    // m <= 16: stream_kernel, the unit's x slice and scales resident in LDS
    const int64_t win = 4;  // chunks per slice are a multiple of this
    int64_t cps = (p.chunks + s - 1) / s;
    cps = (cps + win - 1) / win * win;
    int64_t cps_max = kScBudget * 16 / (p.rows_per_unit * kChunkK) / win * win;
    const int64_t x_max = (kXBudget / (2 * m) - kXPad) / kChunkK / win * win;
    if (cps_max > x_max) cps_max = x_max;
    if (cps > cps_max) cps = cps_max;
    if (cps < win) cps = win;
    p.cps = cps;
    p.slices = (p.chunks + cps - 1) / cps;
    p.units = p.row_blocks * p.slices;
    // short units reach their epilogue before a last-producer stage could
    // publish t: those sum the producers' partials themselves
    p.direct = p.producers > 0 && p.prod_kr <= kDirectMaxKr && p.jt <= 4 && p.cps <= kDirectMaxCps;
    // LDS: the x slice, then the scales (rows an odd multiple of 16 bytes
    // apart, so the 16 rows a wave reads fall in distinct banks)
    p.xpitch = cps * kChunkK + kXPad;
    const int64_t x_bytes = m * p.xpitch * 2;
    int64_t scp = (cps * 8 + 15) / 16;
    if (scp % 2 == 0) ++scp;
    p.sc_pitch = scp * 16;
    p.sc_lds_off = (x_bytes + 15) / 16 * 16;
    int64_t lds = p.sc_lds_off + p.rows_per_unit * p.sc_pitch;
    const int64_t epi = 16 * p.rp * 2 * 2;  // t16 in the one-launch epilogue
    const int64_t prod = (int64_t)kWaves * kProdTiles * 64 * 16 + kWaves * 16 * 4;  // producer wave reductions
    if (lds < epi) lds = epi;
    if (lds < prod) lds = prod;
    p.lds_bytes = lds;
    // workspace after the counters: partial tiles, producer partials, t
    p.part_off = 0;  // offsets from the segment's data (after the counter head)
    p.tpart_off = align256(p.part_off + (p.slices > 1 ? p.units * tile : 0));
    p.ss_off = align256(p.tpart_off + p.prod_kr * (int64_t)p.mt * p.jt * 64 * 16);
    p.t_off = align256(p.ss_off + (p.norm ? p.prod_kr * 16 * 4 : 0));
    p.inv_off = p.t_off + 2 * 16 * p.rp * 2;  // after t16: BF16 hi/lo [2][16][rp]
    p.bytes = align256(p.inv_off + (p.norm ? 16 * 4 : 0));
    return p;
}

struct Decode {
    GemmArgs a;      // a.workspace: this segment's data region
    DecodePlan p;
    uint32_t *ctrs;  // this segment's counters in the workspace head
    __device__ uint32_t *ctr() const { return ctrs; }
    __device__ float *part() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.part_off); }
    __device__ float *tpart() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.tpart_off); }
    __device__ float *t32() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.t_off); }
    __device__ float *ssp() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.ss_off); }
    __device__ float *inv() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.inv_off); }
};

// One launch over up to kMaxSegments GEMMs that share x (m, k, ldx): the
// segment is a grid dimension (y for the main kernels, z for finish_kernel),
// so a workgroup reads its segment's fields without first reading a table;
// the grid is as wide as the widest segment and the surplus workgroups of
// the others exit at once.  Each segment has its own counters and data.
// A one-segment launch takes a one-segment set, so its kernel arguments stay
// as small as one plan.
constexpr int kMaxSegments = QERL_MAX_SEGMENTS;
static_assert(kMaxSegments * kSegCtrBytes == kGemmCtrBytes, "one counter block per segment");
template <int NS>
struct DecodeSetN {
    Decode seg[NS];
    int nseg;
};
using DecodeSet = DecodeSetN<kMaxSegments>;

// ---- device-coherent access: agent scope, no cache write-back or invalidate ----
constexpr int kSc1 = 16;  // cache-policy bit: coherent at device scope

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void store_f4_coherent(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
    i32x4_t b;
    __builtin_memcpy(&b, &v, 16);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off, 0, kSc1);
}
__device__ __forceinline__ void store_u16_coherent(__amdgpu_buffer_rsrc_t r, int off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kSc1);
}
__device__ __forceinline__ i32x4_t load_i4_coherent(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t load_f4_coherent(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
    f32x4_t v;
    __builtin_memcpy(&v, &b, 16);
    return v;
}
__device__ __forceinline__ void store_f32_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_f32_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_add(uint32_t *c, uint32_t v) {
    return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_load(uint32_t *c) {
    return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctr_store(uint32_t *c, uint32_t v) {
    __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every global store and load this wave issued has completed
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// Producer p covers one range of kProdChunks chunks of K for one 16-row
// m-tile and kProdTiles 16-rank tiles (the producers of a launch enumerate
// K ranges x m-tiles x rank-tile groups); its 4 waves take interleaved
// 32-element steps.  A lane supplies x row
// 16*mt + (lane % 16) and A row 16*jt + (lane % 16), 8 elements at
// 8*(lane / 16) of the step, so MFMA tile (mt, jt) holds
// t[16 mt + 4 (lane/16) + v][16 jt + lane % 16] in element v.
// NORM (m <= 16): x enters as bf16(x * norm_w) and the first group of each K
// range also sums the squares of x over the range; the last producer turns
// the sums into 1 / rms per row, scales t by it and publishes both.
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
    const int64_t kb = kr * kProdChunks * kChunkK;
    const int64_t ke = kb + kProdChunks * kChunkK < a.k ? kb + kProdChunks * kChunkK : a.k;
    const int64_t tile_floats = (int64_t)MT * JT * 64 * 4;
    const __amdgpu_buffer_rsrc_t rs_own = coherent_rsrc(d.tpart() + kr * tile_floats);
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [wave][2 tiles][64 lanes]
    float *red_ss = reinterpret_cast<float *>(lds + kWaves * kProdTiles * 64 * 16);  // [wave][16]
    // one m-tile and two rank tiles, so the producer path never needs more
    // registers than the streaming path; each wave's steps (32 elements,
    // every 4th of the range) in groups of PS with all loads of a group
    // issued before its products
    constexpr int PS = 4;
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
            // the four waves' tiles, summed in wave order by wave 0 and published
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
                    store_f4_coherent(rs_own, ((mt * JT + jg + jj) * 64 + lane) * 16, t);
                }
                if (NORM && sum_sq && lane < 16) {
                    float tot = red_ss[lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) tot += red_ss[w * 16 + lane];
                    store_f32_coherent(d.ssp() + kr * 16 + lane, tot);
                }
            }
            __syncthreads();
        }
    }
    if (wave == 0) wait_vm();
    __shared__ uint32_t s_last;
    __shared__ float s_inv[16];
    __syncthreads();
    if (tid == 0) s_last = ctr_add(d.ctr() + kCtrProd, 1u) == (uint32_t)(d.p.producers - 1);
    __syncthreads();
    if (!s_last || d.p.direct) return;  // direct: the consumers read the count and the partials
    if (tid == 0) ctr_store(d.ctr() + kCtrProd, 0u);  // every producer has counted
    if (NORM) {  // 1 / rms of the 16 rows (rows past m repeat row m - 1), sums in K-range order
        if (tid < 16) {
            float tot = 0.0f;
            for (int64_t q = 0; q < d.p.prod_kr; ++q) tot += load_f32_coherent(d.ssp() + q * 16 + tid);
            const float inv = 1.0f / sqrtf(tot * (1.0f / (float)a.k) + a.norm_eps);
            s_inv[tid] = inv;
            store_f32_coherent(d.inv() + tid, inv);
        }
        __syncthreads();
    }
    // The last producer sums the partials in K-range order (tile i goes to
    // wave i % 4, kBatch ranges in flight).  16 < m: into t [m, r] in FP32,
    // read after the kernel boundary.  m <= 16: into t16 [2][16][rp], the BF16
    // hi and lo halves of t in the layout the consumers' epilogue multiplies,
    // published to this launch's consumers by the ready flag.
    const __amdgpu_buffer_rsrc_t rt = coherent_rsrc(d.t32());
    for (int i = wave; wave < kWaves && i < MT * JT; i += kWaves) {
        f32x4_t sum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t q0 = 0; q0 < d.p.prod_kr; q0 += kBatch) {
            f32x4_t v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t q = q0 + u < d.p.prod_kr ? q0 + u : d.p.prod_kr - 1;
                v[u] = load_f4_coherent(coherent_rsrc(d.tpart() + q * tile_floats), (i * 64 + lane) * 16);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (q0 + u < d.p.prod_kr) sum = sum + v[u];
        }
        const int mt = i / JT, jt = i - mt * JT;
        const int64_t j = 16 * jt + lr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = 16 * mt + 4 * lq + v;
            if (MT == 1) {  // all 16 rows (rows past m repeat row m - 1 and are never output)
                const float tv = NORM ? sum[v] * s_inv[m] : sum[v];
                const uint16_t hi = f32_to_bf16_bits(tv);
                const int off = (int)((m * d.p.rp + j) * 2);
                store_u16_coherent(rt, off, hi);
                store_u16_coherent(rt, off + (int)(16 * d.p.rp * 2),
                                   f32_to_bf16_bits(tv - __uint_as_float((uint32_t)hi << 16)));
            } else if (m < a.m && j < a.r) {
                d.t32()[m * a.r + j] = sum[v];
            }
        }
    }
    if (MT == 1) {
        // rank columns past the tiles (r rounded up to 16 vs to 32) are zero
        const int pad = (int)(d.p.rp - 16 * JT);
        for (int i = tid; i < 2 * 16 * pad; i += kThreadsD) {
            const int h = i / (16 * pad), m = (i / pad) % 16, j = 16 * JT + i % pad;
            store_u16_coherent(rt, (int)(((h * 16 + m) * d.p.rp + j) * 2), 0);
        }
        wait_vm();
        __syncthreads();
        if (tid == 0) ctr_store(d.ctr() + kCtrTReady, 1u);
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
struct XNormItem {
    uint4 x;
    float4 w0, w1;
};
template <bool NORM>
__device__ void stage_x_slice(const GemmArgs &a, uint16_t *xs, int64_t pitch, int64_t k0, int64_t width) {
    if (!NORM) {
        batched_copy_2d<uint4>(
            (int)a.m, (int)(width / 8),
            [&](int m, int pc) {
                const int64_t col = k0 + 8 * pc;
                return col < a.k ? *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + col) : make_uint4(0, 0, 0, 0);
            },
            [&](int m, int pc, const uint4 &v) { *reinterpret_cast<uint4 *>(xs + m * pitch + 8 * pc) = v; });
        return;
    }
    batched_copy_2d<XNormItem>(
        (int)a.m, (int)(width / 8),
        [&](int m, int pc) {
            const int64_t col = k0 + 8 * pc;
            XNormItem it{make_uint4(0, 0, 0, 0), make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
            if (col < a.k) {
                it.x = *reinterpret_cast<const uint4 *>(a.x + m * a.ldx + col);
                it.w0 = *reinterpret_cast<const float4 *>(a.norm_w + col);
                it.w1 = *reinterpret_cast<const float4 *>(a.norm_w + col + 4);
            }
            return it;
        },
        [&](int m, int pc, const XNormItem &it) {
            const uint4 v = it.x;
            const uint4 o = make_uint4(pack_bf16x2(bf16lo_to_f32(v.x) * it.w0.x, bf16hi_to_f32(v.x) * it.w0.y),
                                       pack_bf16x2(bf16lo_to_f32(v.y) * it.w0.z, bf16hi_to_f32(v.y) * it.w0.w),
                                       pack_bf16x2(bf16lo_to_f32(v.z) * it.w1.x, bf16hi_to_f32(v.z) * it.w1.y),
                                       pack_bf16x2(bf16lo_to_f32(v.w) * it.w1.z, bf16hi_to_f32(v.w) * it.w1.w));
            *reinterpret_cast<uint4 *>(xs + m * pitch + 8 * pc) = o;
        });
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

// One chunk: x fragments from the LDS window, weights from registers.
// sc_off[g]: LDS byte offset of this lane's scale pair for row group g at the
// unit's first chunk; cl: chunk index within the unit; col: x column of the
// chunk within the window.  The x fragments of the chunk are read once and
// reused over the row groups; each row group's weights are decoded just
// before use, which bounds the registers of the larger tiles.
template <int MT, int NW>
__device__ __forceinline__ void mma_chunk(const uint4 (&w)[NW], const uint8_t *sc, const int (&sc_off)[NW],
                                          int64_t cl, const uint16_t *xb, int64_t pitch, int64_t col, int m_last,
                                          int lr, int lq, f32x4_t (&acc)[MT][NW]) {
    bf16x8_t xa[4][MT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + lr < m_last ? 16 * mt + lr : m_last;
            xa[j][mt] = *reinterpret_cast<const bf16x8_t *>(xb + (m * pitch + col + 32 * lq + 8 * j));
        }
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        const uint32_t s2 = *reinterpret_cast<const uint16_t *>(sc + sc_off[g] + cl * 8);
        const float sv0 = QERL_E4M3_F32(s2, 0), sv1 = QERL_E4M3_F32(s2, 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t q = j == 0 ? w[g].x : j == 1 ? w[g].y : j == 2 ? w[g].z : w[g].w;
            const bf16x8_t b = dequant8_d(q, j < 2 ? sv0 : sv1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j][mt], b, acc[mt][g], 0, 0, 0);
        }
    }
}

// K32: k % 32 == 0; SPLIT: K is split over several units per row block
// (slices > 1); LORA: r > 0.
template <int NS, bool K32, bool SPLIT, bool LORA, bool NORM>
__global__ __launch_bounds__(kThreadsD) void stream_kernel(DecodeSetN<NS> ds) {
    constexpr int MT = 1, NW = 1;  // one 16-row m-tile, one 16-row weight group per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.y];
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    const int64_t bx = blockIdx.x;
    if (NS > 1 && bx >= p.producers + p.units) return;  // past a narrower segment
    // (segments of one launch may differ; a one-segment launch has LORA == (r > 0))
    const bool lora = LORA && (NS == 1 || a.r > 0);
    const bool wait_t = lora || NORM;  // producers publish t and / or 1 / rms behind the ready flag
    if (wait_t && bx < p.producers) {
        lora_producer<MT, NORM>(d, bx, lds);
        return;
    }
    uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
    uint8_t *sc = lds + p.sc_lds_off;
    const int64_t u = bx - p.producers;
    const int64_t slice = u / p.row_blocks, rblk = u - slice * p.row_blocks;
    const int64_t c_begin = slice * p.cps;
    const int64_t c_end = c_begin + p.cps < p.chunks ? c_begin + p.cps : p.chunks;
    const int64_t c_full_end = c_end < p.full_chunks ? c_end : p.full_chunks;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t R = p.rows_per_unit;
    const int64_t n_unit = rblk * R;
    const int64_t n0 = n_unit + (int64_t)wave * 16 * NW;
    const int m_last = (int)a.m - 1;

    int sc_off[NW];
#pragma unroll
    for (int g = 0; g < NW; ++g) sc_off[g] = (int)((wave * 16 * NW + 16 * g + lr) * p.sc_pitch + 2 * lq);

    f32x4_t acc[MT][NW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t c_last = c_full_end - 1;  // the unit's last full chunk (< c_begin: none)
    const int64_t sb0 = c_begin * 8;
    const int64_t sb1 = c_end * 8 < (a.k >> 4) ? c_end * 8 : (a.k >> 4);
    // ---- x and scales of the whole unit resident in LDS; the weights
    // stream through a ring of DR chunks with no barrier ----
    constexpr int DR = kRing;
    uint4 w[DR][NW];
    if (c_full_end > c_begin) {
#pragma unroll
        for (int s = 0; s < DR; ++s)
            load_chunk<NW, K32>(a, n0, c_begin + s < c_last ? c_begin + s : c_last, lr, lq, w[s]);
    }
    stage_x_slice<NORM>(a, xs, p.xpitch, c_begin * kChunkK, (c_end - c_begin) * kChunkK);
    stage_scales(a, sc, p.sc_pitch, n_unit, R, sb0, sb1 - sb0);
    if (c_end > c_full_end) {  // scale bytes of the partial last chunk past k: zero
        const int z0 = (int)((a.k >> 4) - sb0), zn = (int)(p.full_chunks * 8 + 8 - (a.k >> 4));  // zn < 8
        for (int rr = tid >> 3; rr < R; rr += kThreadsD / 8)
            if ((tid & 7) < zn) sc[rr * p.sc_pitch + z0 + (tid & 7)] = 0;
    }
    __syncthreads();
    int64_t c = c_begin;
    for (; c + 2 * DR <= c_full_end; c += DR) {
#pragma unroll
        for (int s = 0; s < DR; ++s) {
            mma_chunk<MT, NW>(w[s], sc, sc_off, c + s - c_begin, xs, p.xpitch, (c + s - c_begin) * kChunkK,
                              m_last, lr, lq, acc);
            load_chunk<NW, K32>(a, n0, c + s + DR, lr, lq, w[s]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (c_full_end - c > DR) {  // DR < rest < 2 DR: one more reloading round (clamped)
#pragma unroll
        for (int s = 0; s < DR; ++s) {
            mma_chunk<MT, NW>(w[s], sc, sc_off, c + s - c_begin, xs, p.xpitch, (c + s - c_begin) * kChunkK,
                              m_last, lr, lq, acc);
            load_chunk<NW, K32>(a, n0, c + s + DR < c_last ? c + s + DR : c_last, lr, lq, w[s]);
            __builtin_amdgcn_sched_barrier(0);
        }
        c += DR;
    }
    // Whether t is published, read while the last chunks multiply: the
    // producers lead the grid and are done by now as a rule, so t can be
    // loaded without a round trip of its own.
    uint32_t t_seen = 0;
    // (direct: ready once every producer has counted; else the ready flag)
    const bool direct = wait_t && p.direct;
    uint32_t *ready_ctr = d.ctr() + (direct ? kCtrProd : kCtrTReady);
    const uint32_t ready_at = (direct ? (uint32_t)p.producers : 1u) + p.wait_bias;
    if (wait_t && tid == 0) t_seen = ctr_load(ready_ctr) >= ready_at;
#pragma unroll
    for (int s = 0; s < DR; ++s)
        if (c + s < c_full_end)  // uniform
            mma_chunk<MT, NW>(w[s], sc, sc_off, c + s - c_begin, xs, p.xpitch, (c + s - c_begin) * kChunkK,
                              m_last, lr, lq, acc);
    if (c_end > c_full_end) {  // the partial last chunk of K (k % 128 != 0)
        uint4 wt[NW];
        load_chunk_tail<NW>(a, n0, p.full_chunks, lr, lq, wt);
        mma_chunk<MT, NW>(wt, sc, sc_off, p.full_chunks - c_begin, xs, p.xpitch, (p.full_chunks - c_begin) * kChunkK,
                          m_last, lr, lq, acc);
    }
    const int64_t tile_floats = R * 16;
    const int wave_off = wave * 64;  // f32x4 slots before this wave's in a tile
    // B [n, j] for this lane's rows and ranks 8 lq .. 8 lq + 7 of the block jb
    auto load_b = [&](int g, int64_t jb) -> bf16x8_t {
        int64_t nb = n0 + 16 * g + lr;
        nb = nb < a.n ? nb : a.n - 1;
        const uint16_t *br = a.lora_b + nb * a.r;
        const int64_t j0 = jb + 8 * lq;
        uint4 v = make_uint4(0, 0, 0, 0);
        if ((a.r & 7) == 0) {
            if (j0 < a.r) v = *reinterpret_cast<const uint4 *>(br + j0);
        } else {
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = j0 + i < a.r ? br[j0 + i] : (uint16_t)0;
            __builtin_memcpy(&v, e, 16);
        }
        return as_bf16x8_d(v);
    };
    bf16x8_t b0[NW];  // the first rank block (read-only input: loaded early)
    if (lora)
#pragma unroll
        for (int g = 0; g < NW; ++g) b0[g] = load_b(g, 0);
    __shared__ uint32_t s_flag, s_ready, s_timeout;
    // ---- split K: the last unit of the row block to arrive sums the slices ----
    if (SPLIT) {
        {
            const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(d.part() + u * tile_floats);
            if (4 * lq < a.m) store_f4_coherent(rs, (wave_off + lane) * 16, acc[0][0]);
            wait_vm();
        }
        if (tid == 0) s_ready = t_seen;
        __syncthreads();
        if (tid == 0) s_flag = ctr_add(d.ctr() + kCtrRow + rblk, 1u) == (uint32_t)(p.slices - 1);
        __syncthreads();
        if (!s_flag) return;
        if (tid == 0) ctr_store(d.ctr() + kCtrRow + rblk, 0u);
    } else {
        if (tid == 0) s_ready = t_seen;
        __syncthreads();
    }
    // A wait that gives up leaves t (or 1 / rms) unknown: the row block's
    // outputs are written as NaN and the segment's error word is set, which
    // gemm_workspace_check reports.
    bool timed_out = false;
    if (wait_t && !s_ready) {  // uniform; rare: wait for the last producer
        if (tid == 0) {
            uint32_t it = 0;
            while (ctr_load(ready_ctr) < ready_at && ++it < p.spin_limit) __builtin_amdgcn_s_sleep(2);
            s_timeout = ctr_load(ready_ctr) < ready_at;
            if (s_timeout) ctr_store(d.ctr() + kCtrErr, kGemmErrWaitTimeout);
        }
        __syncthreads();
        timed_out = s_timeout;
    }
    // The slices' partial tiles and t16 are loaded together (one round trip
    // in the usual case; more than kRedP slices take more), then summed in
    // slice order; t16 goes to LDS as it is.
    constexpr int kRedP = 12;
    auto part_at = [&](int64_t sl) { return coherent_rsrc(d.part() + (sl * p.row_blocks + rblk) * tile_floats); };
    const int t_pieces = (int)(16 * p.rp * 2 * 2 / 16);  // 16-byte pieces of t16 (<= 512)
    // Every load is issued unconditionally; the buffer resources end where
    // the data does, so a load past the slices or past t16 returns zeros
    // without a memory access (and with no branch for the compiler to fold
    // the sums into).
    f32x4_t pv[kRedP];
    i32x4_t tq[2], iq;
    f32x4_t dq[kDirectMaxKr];  // direct: tile (wave) of each K range's partial t
    float sq[kDirectMaxKr];    // direct + NORM: row (tid < 16) of each K range's sum of squares
    if (SPLIT) {
        const int64_t sstride = p.row_blocks * tile_floats * 4;  // bytes between slices of a row block
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            d.part() + rblk * tile_floats, 0, (int)(sstride * (p.slices < kRedP ? p.slices : kRedP)), 0x00020000);
#pragma unroll
        for (int v = 0; v < kRedP; ++v)
            pv[v] = load_f4_coherent(rp, (int)(v * sstride) + (wave_off + lane) * 16);
    }
    const int64_t ptile = (int64_t)p.jt * 64 * 4;  // floats of one K range's partial tiles
    if (direct) {
        if (lora && wave < p.jt) {  // (uniform) tile `wave`, K ranges past prod_kr read as zeros
            const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                d.tpart(), 0, (int)(p.prod_kr * ptile * 4), 0x00020000);
#pragma unroll
            for (int q = 0; q < kDirectMaxKr; ++q)
                dq[q] = load_f4_coherent(rq, (int)((q * ptile + (wave * 64 + lane) * 4) * 4));
        }
        if (NORM) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                d.ssp(), 0, (int)(p.prod_kr * 16 * 4), 0x00020000);
#pragma unroll
            for (int q = 0; q < kDirectMaxKr; ++q)
                sq[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (q * 16 + (tid & 15)) * 4, 0, kSc1));
        }
    } else {
        if (lora) {
            const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(d.t32(), 0, t_pieces * 16, 0x00020000);
            tq[0] = load_i4_coherent(rt, tid * 16);
            tq[1] = load_i4_coherent(rt, (tid + kThreadsD) * 16);
        }
        if (NORM) iq = load_i4_coherent(coherent_rsrc(d.inv()), (tid & 3) * 16);  // 1 / rms of the 16 rows
    }
    // The values are taken here, after every load has been issued: without
    // this the compiler folds the sums below into the conditional loads and
    // waits for each load before issuing the next.
    if (SPLIT)
#pragma unroll
        for (int v = 0; v < kRedP; ++v) asm volatile("" : "+v"(pv[v]));
    if (direct) {
        if (lora && wave < p.jt)
#pragma unroll
            for (int q = 0; q < kDirectMaxKr; ++q) asm volatile("" : "+v"(dq[q]));
        if (NORM)
#pragma unroll
            for (int q = 0; q < kDirectMaxKr; ++q) asm volatile("" : "+v"(sq[q]));
    } else {
        if (lora) asm volatile("" : "+v"(tq[0]), "+v"(tq[1]));
        if (NORM) asm volatile("" : "+v"(iq));
    }
    if (SPLIT) {
        acc[0][0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < kRedP; ++v) acc[0][0] = acc[0][0] + pv[v];  // zeros past the slices
        for (int64_t s0 = kRedP; s0 < p.slices; s0 += kRedP) {
#pragma unroll
            for (int v = 0; v < kRedP; ++v) {
                const int64_t sl = s0 + v < p.slices ? s0 + v : p.slices - 1;
                pv[v] = load_f4_coherent(part_at(sl), (wave_off + lane) * 16);
            }
#pragma unroll
            for (int v = 0; v < kRedP; ++v)
                if (s0 + v < p.slices) acc[0][0] = acc[0][0] + pv[v];
        }
    }

    // ---- LoRA epilogue (lora_scale * t B^T on the MFMA, t as BF16 hi + lo) and output ----
    uint16_t *th = reinterpret_cast<uint16_t *>(lds);  // t16 [2][16][rp]: hi, then lo
    uint16_t *tl = th + 16 * p.rp;
    __shared__ __attribute__((aligned(16))) float s_inv[16];
    if (direct) {
        // t = the K ranges' partial tiles summed in K-range order (scaled by
        // 1 / rms with the norm), into LDS as BF16 hi + lo in the t16 layout
        if (NORM) {
            if (tid < 16) {
                float tot = 0.0f;
#pragma unroll
                for (int q = 0; q < kDirectMaxKr; ++q) tot += sq[q];  // zeros past prod_kr
                s_inv[tid] = 1.0f / sqrtf(tot * (1.0f / (float)a.k) + a.norm_eps);
            }
            __syncthreads();
        }
        if (lora) {
            if (wave < p.jt) {
                f32x4_t t = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int q = 0; q < kDirectMaxKr; ++q) t = t + dq[q];
                const int64_t j = 16 * wave + lr;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 4 * lq + v;
                    const float tv = NORM ? t[v] * s_inv[m] : t[v];
                    const uint16_t hi = f32_to_bf16_bits(tv);
                    th[m * p.rp + j] = hi;
                    tl[m * p.rp + j] = f32_to_bf16_bits(tv - __uint_as_float((uint32_t)hi << 16));
                }
            }
            // rank columns past the tiles (r rounded up to 16 vs to 32) are zero
            const int pad = (int)(p.rp - 16 * p.jt);
            for (int i = tid; i < 2 * 16 * pad; i += kThreadsD) {
                const int h = i / (16 * pad), m = (i / pad) % 16, j = 16 * (int)p.jt + i % pad;
                th[(h * 16 + m) * p.rp + j] = 0;
            }
        }
    } else {
        if (lora) {  // (the pieces past t16 were loaded as zeros and are not stored)
            if (tid < t_pieces) reinterpret_cast<i32x4_t *>(th)[tid] = tq[0];
            if (tid + kThreadsD < t_pieces) reinterpret_cast<i32x4_t *>(th)[tid + kThreadsD] = tq[1];
        }
        if (NORM && tid < 4) reinterpret_cast<i32x4_t *>(s_inv)[tid] = iq;
    }
    if (wait_t) __syncthreads();
    const float st = *a.tensor_scale, lam = a.lora_scale;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4_t l = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            for (int64_t jb = 0; jb < p.rp; jb += 32) {
                const bf16x8_t bfrag = jb == 0 ? b0[g] : load_b(g, jb);
                const int64_t off = (16 * mt + lr) * p.rp + jb + 8 * lq;
                l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t *>(th + off), bfrag, l,
                                                            0, 0, 0);
                l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t *>(tl + off), bfrag, l,
                                                            0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = 16 * mt + 4 * lq + v;
                const int64_t n = n0 + 16 * g + lr;
                const float base = NORM ? st * s_inv[m] * acc[mt][g][v] : st * acc[mt][g][v];
                if (m < a.m && n < a.n)
                    a.y[m * a.ldy + n] = timed_out ? (uint16_t)0x7FC0 : f32_to_bf16_bits(base + lam * l[v]);
            }
        }
    }
    // this row block is done with t16; the last one clears the ready flag
    // and this count for the next call
    if (wait_t && tid == 0 && ctr_add(d.ctr() + kCtrDone, 1u) == (uint32_t)(p.row_blocks - 1)) {
        ctr_store(ready_ctr, 0u);  // (direct: the producers' count)
        ctr_store(d.ctr() + kCtrDone, 0u);
    }
}

// 16 < m: y[m, n] = bf16(s_t * sum over slices of the partial tiles (in slice
// order) + lora_scale * sum_j t[m][j] B[n][j]).  Thread (n, quad) handles the
// rows 4 quad .. 4 quad + 3 of column n, which one lane of one tile holds as a
// float4.  Workgroup: 64 columns x 4 quads (16 rows); t of its rows in LDS.
template <int NS, int MT, int NW>
__global__ __launch_bounds__(256) void finish_kernel(DecodeSetN<NS> ds) {
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.z];
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    const int64_t bx = blockIdx.x;
    if (NS > 1 && bx * 64 >= a.n) return;  // past a narrower segment
    __shared__ float ts[16][kMaxRank];
    const int tid = threadIdx.x;
    const int64_t n = bx * 64 + (tid & 63);
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int64_t quad = blockIdx.y * 4 + (tid >> 6);
    for (int64_t i = tid; i < 16 * (int64_t)a.r; i += 256) {
        const int64_t mm = i / a.r, j = i - mm * a.r;
        ts[mm][j] = m0 + mm < a.m ? d.t32()[(m0 + mm) * a.r + j] : 0.0f;
    }
    __syncthreads();
    if (n >= a.n || 4 * quad >= a.m) return;
    const int64_t R = p.rows_per_unit;
    const int64_t rblk = n / R, rem = n - rblk * R;
    const int64_t wave = rem / (16 * NW), g = (rem / 16) % NW, lr = rem % 16;
    const int64_t mt = quad / 4, lq = quad % 4;
    const int64_t slot = ((wave * MT + mt) * NW + g) * 64 + lq * 16 + lr;
    const int64_t tile_floats = R * 16 * MT;
    const float *part = d.part();
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t s0 = 0; s0 < p.slices; s0 += kBatch) {  // kBatch slices in flight, summed in order
        f32x4_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t s = s0 + u < p.slices ? s0 + u : p.slices - 1;
            v[u] = *reinterpret_cast<const f32x4_t *>(part + (s * p.row_blocks + rblk) * tile_floats + slot * 4);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (s0 + u < p.slices) acc = acc + v[u];
    }
    float lora[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *br = a.lora_b + n * a.r;
    const int q0 = (int)(tid >> 6) * 4;  // this thread's first row in ts
    int j = 0;
    if ((a.r & 7) == 0) {
        for (; j < a.r; j += 8) {
            const uint4 b8 = *reinterpret_cast<const uint4 *>(br + j);
            const uint32_t bw[4] = {b8.x, b8.y, b8.z, b8.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    lora[v] = __builtin_fmaf(ts[q0 + v][j + 2 * e], bf16lo_to_f32(bw[e]), lora[v]);
                    lora[v] = __builtin_fmaf(ts[q0 + v][j + 2 * e + 1], bf16hi_to_f32(bw[e]), lora[v]);
                }
        }
    }
    for (; j < a.r; ++j) {
        const float b = bf16lo_to_f32(br[j]);
#pragma unroll
        for (int v = 0; v < 4; ++v) lora[v] = __builtin_fmaf(ts[q0 + v][j], b, lora[v]);
    }
    const float st = *a.tensor_scale, lam = a.lora_scale;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t m = 4 * quad + v;
        if (m < a.m) a.y[m * a.ldy + n] = f32_to_bf16_bits(st * acc[v] + lam * lora[v]);
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
        lora_producer<MT>(d, bx, g_dxtile0);
        return;
    }
    constexpr int NW = 4 * kUnitWaves / kWaves;  // n-tiles per wave of the four-wave tile layout
    constexpr int kPer = kUnitWaves / kWaves;     // unit waves per layout wave
    const int64_t u = bx - p.producers;
    const int64_t slice = u / p.row_blocks, rblk = u - slice * p.row_blocks;
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
    mfma_kloop<MT, kUnitWaves, 1, SCL>(a.x, a.m, a.ldx, a.packed + n0 * kb, a.scales + n0 * ks, a.n - n0, a.k,
                                       c_begin, fast_end, g_dxtile0, g_dxtile1, acc, g_dsc, (int)p.unit_sc_pitch);
    // the rest of the slice (the partial last chunk of K, or all of it for
    // very wide x rows)
    const int64_t nw = n0 + wave * 64 + lr;
    plain_kloop<MT, kUnitWaves>(
        fast_end * kChunkK, c_end * kChunkK < a.k ? c_end * kChunkK : a.k, g_dxtile0,
        [&](int row, int64_t kk) {
            uint4 o = make_uint4(0, 0, 0, 0);
            if (row < a.m && kk < a.k) o = *reinterpret_cast<const uint4 *>(a.x + row * a.ldx + kk);
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
            if (16 * i + 4 * lq < a.m) tile[(((wave / kPer) * MT + i) * NW + (4 * wave + j) % NW) * 64] = acc[i][j];
}

template <int NS, int MT, bool SCL>
__global__ __launch_bounds__(64 * kUnitWaves) void mfma_unit_kernel(DecodeSetN<NS> ds) {
    const Decode &d = ds.seg[NS == 1 ? 0u : blockIdx.y];
    if (NS > 1 && (int64_t)blockIdx.x >= d.p.producers + d.p.units) return;  // past a narrower segment
    mfma_unit<MT, SCL>(d, blockIdx.x);
}

template <int MT, int NS>
hipError_t launch_mfma_units(const DecodeSetN<NS> &ds, hipStream_t stream) {
    const Decode &d = ds.seg[0];  // the unit shape and scale staging are shared by the segments
    int64_t blocks = 0, fblocks = 0;
    for (int i = 0; i < ds.nseg; ++i) {
        const int64_t b = ds.seg[i].p.producers + ds.seg[i].p.units, f = (ds.seg[i].a.n + 63) / 64;
        blocks = b > blocks ? b : blocks;
        fblocks = f > fblocks ? f : fblocks;
    }
    const dim3 grid((unsigned)blocks, (unsigned)ds.nseg);
    if (d.p.unit_sc)
        hipLaunchKernelGGL((mfma_unit_kernel<NS, MT, true>), grid, dim3(64 * kUnitWaves), 0, stream, ds);
    else
        hipLaunchKernelGGL((mfma_unit_kernel<NS, MT, false>), grid, dim3(64 * kUnitWaves), 0, stream, ds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 fgrid((unsigned)fblocks, (unsigned)((d.a.m + 15) / 16), (unsigned)ds.nseg);
    hipLaunchKernelGGL((finish_kernel<NS, MT, 4 * kUnitWaves / kWaves>), fgrid, dim3(256), 0, stream, ds);
    return hipGetLastError();
}

template <bool K32, bool SPLIT, bool LORA, bool NORM, int NS>
hipError_t launch_stream(const DecodeSetN<NS> &ds, int64_t lds_bytes, hipStream_t stream) {
    auto kern = stream_kernel<NS, K32, SPLIT, LORA, NORM>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    if (attr != hipSuccess) return attr;
    int64_t blocks = 0;
    for (int i = 0; i < ds.nseg; ++i) {
        const int64_t b = ds.seg[i].p.producers + ds.seg[i].p.units;
        blocks = b > blocks ? b : blocks;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks, (unsigned)ds.nseg), dim3(kThreadsD), (size_t)lds_bytes, stream, ds);
    return hipGetLastError();
}

template <bool K32, int NS>
hipError_t launch_stream(const DecodeSetN<NS> &ds, int64_t lds_bytes, bool lora, hipStream_t stream) {
    const bool split = ds.seg[0].p.slices > 1;  // the same for every segment
    if (ds.seg[0].p.norm) {  // the norm prologue: k % 32 == 0 only (checked by the caller)
        if constexpr (K32) {
            if (split)
                return lora ? launch_stream<K32, true, true, true>(ds, lds_bytes, stream)
                            : launch_stream<K32, true, false, true>(ds, lds_bytes, stream);
            return lora ? launch_stream<K32, false, true, true>(ds, lds_bytes, stream)
                        : launch_stream<K32, false, false, true>(ds, lds_bytes, stream);
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (split)
        return lora ? launch_stream<K32, true, true, false>(ds, lds_bytes, stream)
                    : launch_stream<K32, true, false, false>(ds, lds_bytes, stream);
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
    int64_t data = kGemmCtrBytes;
    for (int i = 0; i < nseg; ++i) {
        ds.seg[i].a = segs[i];
        ds.seg[i].p = make_decode_plan(segs[i].m, segs[i].n, segs[i].k, segs[i].r, rows, norm);
        ds.seg[i].ctrs = reinterpret_cast<uint32_t *>(base + i * kSegCtrBytes);
        ds.seg[i].a.workspace = base + data;
        data += align256(ds.seg[i].p.bytes);
    }
    return ds;
}

template <int NS>
hipError_t launch_checked(const DecodeSetN<NS> &ds, int64_t lds, bool lora, hipStream_t stream) {
    const Decode &d0 = ds.seg[0];
    if (d0.p.mt == 2) return launch_mfma_units<2>(ds, stream);
    if (d0.p.mt == 4) return launch_mfma_units<4>(ds, stream);
    return (d0.a.k & 31) == 0 ? launch_stream<true>(ds, lds, lora, stream) : launch_stream<false>(ds, lds, lora, stream);
}

hipError_t launch_decode_set(const DecodeSet &ds, hipStream_t stream) {
    int64_t lds = 0;
    bool lora = false;
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
    }
    for (int i = 0; i < ds.nseg; ++i)
        if (ds.seg[i].p.producers + ds.seg[i].p.units > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (ds.nseg == 1) return launch_checked(DecodeSetN<1>{{ds.seg[0]}, 1}, lds, lora, stream);
    return launch_checked(ds, lds, lora, stream);
}

// the counter head of a GEMM workspace to zero, 16 bytes per thread
__global__ __launch_bounds__(256) void zero_head_kernel(uint4 *head) {
    head[(int64_t)blockIdx.x * 256 + threadIdx.x] = make_uint4(0, 0, 0, 0);
}
static_assert(kGemmCtrBytes % (256 * 16) == 0, "whole workgroups of 16-byte stores");

}  // namespace

std::atomic<int> g_force_wait_timeout{0};

hipError_t launch_gemm_workspace_reset(void *workspace, hipStream_t stream) {
    hipLaunchKernelGGL(zero_head_kernel, dim3((unsigned)(kGemmCtrBytes / (256 * 16))), dim3(256), 0, stream,
                       static_cast<uint4 *>(workspace));
    return hipGetLastError();
}

size_t decode_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    return (size_t)(kGemmCtrBytes + make_decode_plan(m, n, k, r).bytes);
}

hipError_t launch_decode(const GemmArgs &a, hipStream_t stream) {
    return launch_decode_set(make_decode_set(&a, 1), stream);
}

size_t decode_multi_workspace_bytes(int64_t m, int64_t k, const int64_t *n, const int *r, int nseg, bool norm) {
    int64_t rows = 0;
    for (int j = 0; j < nseg; ++j) rows += make_decode_plan(m, n[j], k, r[j], 0, norm).row_blocks;
    int64_t bytes = kGemmCtrBytes;
    for (int j = 0; j < nseg; ++j) bytes += align256(make_decode_plan(m, n[j], k, r[j], rows, norm).bytes);
    return (size_t)bytes;
}

hipError_t launch_decode_multi(const GemmArgs *segs, int nseg, hipStream_t stream) {
    if (nseg < 1 || nseg > kMaxSegments) return hipErrorInvalidValue;
    return launch_decode_set(make_decode_set(segs, nseg), stream);
}

}  // namespace qerl
