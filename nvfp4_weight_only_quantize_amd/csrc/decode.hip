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
// which are read exactly once.  Two launches, no inter-workgroup waiting:
//
//  stream_kernel  work units = (block of 64*NW weight rows) x (slice of K).
//                 Each of the 4 waves owns 16*NW rows and streams them over
//                 the slice in 128-element chunks (64 packed bytes + 8 scale
//                 bytes per row), keeping kDepth chunks in flight in a
//                 register ring.  The x columns of the slice pass through a
//                 double-buffered LDS segment shared by the 4 waves; LDS reads
//                 are counted separately from global loads, so waiting for x
//                 never waits for the weight prefetch.  Weights are decoded to
//                 exact BF16 (e2m1 * e4m3) and multiplied on the 16x16x32 BF16
//                 MFMA; each unit writes FP32 partial sums of its slice.
//                 Extra "producer" workgroups of the same launch compute the
//                 LoRA down-projection t = x A^T in FP32.
//  finish_kernel  y = bf16(s_t * sum over slices of the partials (in slice
//                 order: deterministic) + lora_scale * t B^T).
#include "device_common.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreadsD = kWaves * 64;
constexpr int64_t kChunkK = 128;   // K elements per chunk
constexpr int kDepth = 4;          // chunks in flight per wave
constexpr int kXPad = 8;           // LDS row padding of the staged x (BF16 elements)
constexpr int64_t kLdsBudget = 64 * 1024 - 1024;  // dynamic LDS for x (static LDS stays below 1 KB)
constexpr int64_t kTargetUnits = 640;
constexpr int kProdMG = 2;         // activation rows per LoRA producer workgroup
constexpr int kMaxRank = 128;      // LoRA rank limit of the C ABI

struct DecodePlan {
    int mt, nw;
    int64_t rows_per_unit, row_blocks, slices, kslice;
    int64_t units, producers;
    int64_t part_off, t_off, bytes, lds_bytes;
};

// The whole x slice of a unit is staged in LDS once, so its K extent is
// bounded by the LDS budget: m * (kslice + pad) * 2 bytes <= kLdsBudget.
DecodePlan make_decode_plan(int64_t m, int64_t n, int64_t k, int r) {
    DecodePlan p{};
    p.mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    p.nw = p.mt;  // x fragments are reused over nw column groups
    p.rows_per_unit = 16 * kWaves * (int64_t)p.nw;
    p.row_blocks = (n + p.rows_per_unit - 1) / p.rows_per_unit;
    const int64_t chunks = (k + kChunkK - 1) / kChunkK;
    int64_t max_chunks = (kLdsBudget / (2 * m) - kXPad) / kChunkK;  // LDS bound on the slice
    if (max_chunks < 1) max_chunks = 1;
    // split K so the grid covers the chip, keeping FP32 partials small next to
    // the weights where the LDS bound allows it (S * m * n * 4 <= weight bytes / 4)
    int64_t s = (kTargetUnits + p.row_blocks - 1) / p.row_blocks;
    int64_t s_cap = (k * 9) / (256 * m);
    if (s_cap < 1) s_cap = 1;
    if (s > s_cap) s = s_cap;
    const int64_t s_min = (chunks + max_chunks - 1) / max_chunks;
    if (s < s_min) s = s_min;
    if (s > chunks) s = chunks;
    if (s < 1) s = 1;
    p.kslice = (chunks + s - 1) / s * kChunkK;
    p.slices = (k + p.kslice - 1) / p.kslice;
    p.units = p.row_blocks * p.slices;
    p.producers = r > 0 ? (int64_t)r * ((m + kProdMG - 1) / kProdMG) : 0;
    p.part_off = 0;
    p.t_off = (p.slices * m * n * 4 + 255) & ~(int64_t)255;
    p.bytes = p.t_off + ((m * (int64_t)r * 4 + 255) & ~(int64_t)255);
    p.lds_bytes = m * (p.kslice + kXPad) * 2;
    return p;
}

struct Decode {
    GemmArgs a;
    DecodePlan p;
    __device__ float *partials() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.part_off); }
    __device__ float *t32() const { return reinterpret_cast<float *>(static_cast<char *>(a.workspace) + p.t_off); }
};

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

// One full chunk of the weights for lane (lr, lq) of column group g: row n,
// elements 128c + 32lq .. +32 (16 packed bytes, 2 scale bytes).  Rows past n
// are clamped (their outputs are discarded), so the loads carry no branch and
// the compiler's in-order wait counting stays exact.  K32: k % 32 == 0, so
// packed rows are 16-byte and scale rows 2-byte aligned.
template <int NW, bool K32>
__device__ __forceinline__ void load_chunk_full(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq,
                                                uint4 (&w)[NW], uint32_t (&sc)[NW]) {
    const int64_t e0 = c * kChunkK + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        int64_t n = n0 + 16 * g + lr;
        n = n < a.n ? n : a.n - 1;
        const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
        const uint8_t *srow = a.scales + n * (a.k >> 4) + (e0 >> 4);
        if (K32) {
            w[g] = *reinterpret_cast<const uint4 *>(prow);
            sc[g] = *reinterpret_cast<const uint16_t *>(srow);
        } else {
            const uint2 lo = reinterpret_cast<const uint2 *>(prow)[0];
            const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
            w[g] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            sc[g] = (uint32_t)srow[0] | ((uint32_t)srow[1] << 8);
        }
    }
}

// The last chunk of a row when k % 128 != 0 (k % 16 == 0): elements past k
// read as zero.
template <int NW>
__device__ __forceinline__ void load_chunk_tail(const GemmArgs &a, int64_t n0, int64_t c, int lr, int lq,
                                                uint4 (&w)[NW], uint32_t (&sc)[NW]) {
    const int64_t e0 = c * kChunkK + 32 * lq;
#pragma unroll
    for (int g = 0; g < NW; ++g) {
        int64_t n = n0 + 16 * g + lr;
        n = n < a.n ? n : a.n - 1;
        const uint8_t *prow = a.packed + n * (a.k >> 1) + (e0 >> 1);
        const uint8_t *srow = a.scales + n * (a.k >> 4) + (e0 >> 4);
        w[g] = make_uint4(0, 0, 0, 0);
        sc[g] = 0;
        if (e0 + 16 <= a.k) {
            const uint2 lo = *reinterpret_cast<const uint2 *>(prow);
            w[g].x = lo.x;
            w[g].y = lo.y;
            sc[g] = srow[0];
            if (e0 + 32 <= a.k) {
                const uint2 hi = reinterpret_cast<const uint2 *>(prow)[1];
                w[g].z = hi.x;
                w[g].w = hi.y;
                sc[g] |= (uint32_t)srow[1] << 8;
            }
        }
    }
}

// LoRA down-projection for rows [m0, m0 + kProdMG) and rank j: the 256 lanes
// split K, four 16-byte steps in flight per lane.
__device__ void lora_producer(const Decode &d, int64_t job) {
    const GemmArgs &a = d.a;
    const int64_t j = job % a.r;
    const int64_t m0 = (job / a.r) * kProdMG;
    const uint16_t *ar = a.lora_a + j * a.k;
    float acc[kProdMG];
#pragma unroll
    for (int i = 0; i < kProdMG; ++i) acc[i] = 0.0f;
    const uint16_t *xr[kProdMG];
#pragma unroll
    for (int i = 0; i < kProdMG; ++i) {
        const int64_t m = m0 + i < a.m ? m0 + i : a.m - 1;
        xr[i] = a.x + m * a.ldx;
    }
    const int64_t step = (int64_t)kThreadsD * 8;
    int64_t kk = (int64_t)threadIdx.x * 8;
    for (; kk + 3 * step < a.k; kk += 4 * step) {
        uint4 av[4], xv[4][kProdMG];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[u] = *reinterpret_cast<const uint4 *>(ar + kk + u * step);
#pragma unroll
            for (int i = 0; i < kProdMG; ++i) xv[u][i] = *reinterpret_cast<const uint4 *>(xr[i] + kk + u * step);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < kProdMG; ++i) {
                acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u][i].x), as_bf16x2(av[u].x), acc[i], false);
                acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u][i].y), as_bf16x2(av[u].y), acc[i], false);
                acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u][i].z), as_bf16x2(av[u].z), acc[i], false);
                acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[u][i].w), as_bf16x2(av[u].w), acc[i], false);
            }
    }
    for (; kk < a.k; kk += step) {  // k % 16 == 0: a vector never straddles the end
        const uint4 av = *reinterpret_cast<const uint4 *>(ar + kk);
#pragma unroll
        for (int i = 0; i < kProdMG; ++i) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xr[i] + kk);
            acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.x), as_bf16x2(av.x), acc[i], false);
            acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.y), as_bf16x2(av.y), acc[i], false);
            acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.z), as_bf16x2(av.z), acc[i], false);
            acc[i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv.w), as_bf16x2(av.w), acc[i], false);
        }
    }
    __shared__ float red[kProdMG][4];
#pragma unroll
    for (int i = 0; i < kProdMG; ++i) {
        const float v = wave_sum(acc[i]);
        if ((threadIdx.x & 63) == 0) red[i][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if (threadIdx.x < kProdMG && m0 + threadIdx.x < a.m) {
        const int i = threadIdx.x;
        d.t32()[(m0 + i) * a.r + j] = (red[i][0] + red[i][1]) + (red[i][2] + red[i][3]);
    }
}

template <int MT, int NW>
__device__ __forceinline__ void mma_chunk_lds(const uint4 (&w)[NW], const uint32_t (&sc)[NW],
                                              const uint16_t *lds, int64_t base, int64_t pitch, int64_t col,
                                              int m_last, int lr, int lq, f32x4_t (&acc)[MT][NW]) {
    float sv[NW][2];
#pragma unroll
    for (int gi = 0; gi < NW; ++gi) {
        sv[gi][0] = QERL_E4M3_F32(sc[gi], 0);
        sv[gi][1] = QERL_E4M3_F32(sc[gi], 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bf16x8_t xa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + lr < m_last ? 16 * mt + lr : m_last;
            xa[mt] = *reinterpret_cast<const bf16x8_t *>(lds + (base + m * pitch + col + 32 * lq + 8 * j));
        }
#pragma unroll
        for (int gi = 0; gi < NW; ++gi) {
            const uint32_t q = j == 0 ? w[gi].x : j == 1 ? w[gi].y : j == 2 ? w[gi].z : w[gi].w;
            const bf16x8_t b = dequant8_d(q, sv[gi][j >> 1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt], b, acc[mt][gi], 0, 0, 0);
        }
    }
}

// Stage x[:, k0 .. kend) of every row into LDS (row pitch kslice + pad;
// columns past kend as zero).  Thread t moves 16-byte pieces t, t + 256, ...;
// addresses are clamped into range so every load is unconditional.
template <int PIECES>
__device__ __forceinline__ void stage_x(const GemmArgs &a, uint16_t *lds, int64_t k0, int64_t kend,
                                        int64_t width, int64_t pitch) {
    const int64_t per_row = width / 8;
    uint4 v[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        const int64_t piece = threadIdx.x + (int64_t)i * kThreadsD;
        const int64_t m = piece / per_row, col = (piece - m * per_row) * 8;
        const int64_t mm = m < a.m ? m : a.m - 1;
        const int64_t kk = k0 + col < kend ? k0 + col : kend - 8;
        v[i] = *reinterpret_cast<const uint4 *>(a.x + mm * a.ldx + kk);
        if (!(m < a.m && k0 + col < kend)) v[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        const int64_t piece = threadIdx.x + (int64_t)i * kThreadsD;
        const int64_t m = piece / per_row, col = (piece - m * per_row) * 8;
        if (m < a.m) *reinterpret_cast<uint4 *>(lds + (m * pitch + col)) = v[i];
    }
}

// PIECES >= ceil(m * kslice / 8 / 256): 16-byte staging pieces per thread
template <int MT, int NW, int PIECES, bool K32>
__global__ __launch_bounds__(kThreadsD) void stream_kernel(Decode d) {
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    if ((int64_t)blockIdx.x < p.producers) {  // LoRA producers go first so they start early
        lora_producer(d, blockIdx.x);
        return;
    }
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_lds[];
    const int64_t u = blockIdx.x - p.producers;
    const int64_t slice = u / p.row_blocks, rblk = u - slice * p.row_blocks;
    const int64_t k_begin = slice * p.kslice;
    const int64_t k_end = k_begin + p.kslice < a.k ? k_begin + p.kslice : a.k;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t n0 = rblk * p.rows_per_unit + (int64_t)wave * 16 * NW;
    const int64_t pitch = p.kslice + kXPad;
    const int m_last = (int)a.m - 1;

    f32x4_t acc[MT][NW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t c_begin = k_begin / kChunkK;
    const int64_t c_end = (k_end + kChunkK - 1) / kChunkK;
    const int64_t full_chunks = a.k / kChunkK;
    const int64_t c_full_end = c_end < full_chunks ? c_end : full_chunks;

    // ring prologue (chunk indices clamped into the slice's full chunks), then x
    uint4 w[kDepth][NW];
    uint32_t sc[kDepth][NW];
    if (c_full_end > c_begin) {  // uniform
        const int64_t c_last = c_full_end - 1;
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            const int64_t c = c_begin + s < c_last ? c_begin + s : c_last;
            load_chunk_full<NW, K32>(a, n0, c, lr, lq, w[s], sc[s]);
        }
    }
    stage_x<PIECES>(a, xs_lds, k_begin, k_end, p.kslice, pitch);
    __syncthreads();

    if (c_full_end > c_begin) {  // uniform
        const int64_t c_last = c_full_end - 1;
        for (int64_t c0 = c_begin; c0 < c_full_end; c0 += kDepth) {
#pragma unroll
            for (int s = 0; s < kDepth; ++s) {
                const int64_t c = c0 + s;
                if (c < c_full_end)  // uniform; the compute only, loads stay unconditional
                    mma_chunk_lds<MT, NW>(w[s], sc[s], xs_lds, 0, pitch, (c - c_begin) * kChunkK, m_last, lr,
                                          lq, acc);
                const int64_t cn = c + kDepth < c_last ? c + kDepth : c_last;
                load_chunk_full<NW, K32>(a, n0, cn, lr, lq, w[s], sc[s]);
            }
        }
    }
    if (c_end > c_full_end) {  // the partial last chunk of K (k % 128 != 0)
        uint4 wt[NW];
        uint32_t st[NW];
        load_chunk_tail<NW>(a, n0, full_chunks, lr, lq, wt, st);
        mma_chunk_lds<MT, NW>(wt, st, xs_lds, 0, pitch, (full_chunks - c_begin) * kChunkK, m_last, lr, lq, acc);
    }

    // FP32 partial sums of this slice: P[slice][m][n]
    float *part = d.partials() + slice * a.m * a.n;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int gi = 0; gi < NW; ++gi)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = 16 * mt + 4 * lq + v;
                const int64_t n = n0 + 16 * gi + lr;
                if (m < a.m && n < a.n) part[m * a.n + n] = acc[mt][gi][v];
            }
}

// y[m, n] = bf16(s_t * sum_s P[s][m][n] + lora_scale * sum_j t[m][j] B[n][j]);
// one thread per output, partials summed in slice order.
__global__ __launch_bounds__(256) void finish_kernel(Decode d) {
    const GemmArgs &a = d.a;
    const DecodePlan &p = d.p;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m = blockIdx.y;
    __shared__ float ts[kMaxRank];
    for (int j = threadIdx.x; j < a.r; j += 256) ts[j] = d.t32()[m * a.r + j];
    __syncthreads();
    if (n >= a.n) return;
    const float *part = d.partials() + m * a.n + n;
    const int64_t stride = a.m * a.n;
    float acc = 0.0f;
    int64_t s = 0;
    for (; s + 8 <= p.slices; s += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = part[(s + i) * stride];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; s < p.slices; ++s) acc += part[s * stride];
    float lora = 0.0f;
    const uint16_t *br = a.lora_b + n * a.r;
    if ((a.r & 7) == 0) {
        for (int j = 0; j < a.r; j += 8) {
            const uint4 b = *reinterpret_cast<const uint4 *>(br + j);
            lora = __builtin_fmaf(ts[j + 0], bf16lo_to_f32(b.x), lora);
            lora = __builtin_fmaf(ts[j + 1], bf16hi_to_f32(b.x), lora);
            lora = __builtin_fmaf(ts[j + 2], bf16lo_to_f32(b.y), lora);
            lora = __builtin_fmaf(ts[j + 3], bf16hi_to_f32(b.y), lora);
            lora = __builtin_fmaf(ts[j + 4], bf16lo_to_f32(b.z), lora);
            lora = __builtin_fmaf(ts[j + 5], bf16hi_to_f32(b.z), lora);
            lora = __builtin_fmaf(ts[j + 6], bf16lo_to_f32(b.w), lora);
            lora = __builtin_fmaf(ts[j + 7], bf16hi_to_f32(b.w), lora);
        }
    } else {
        for (int j = 0; j < a.r; ++j) lora = __builtin_fmaf(ts[j], bf16lo_to_f32(br[j]), lora);
    }
    a.y[m * a.ldy + n] = f32_to_bf16_bits(*a.tensor_scale * acc + a.lora_scale * lora);
}

template <int MT, int NW, int PIECES, bool K32>
hipError_t launch_stream(const Decode &d, hipStream_t stream) {
    auto kern = stream_kernel<MT, NW, PIECES, K32>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
    if (attr != hipSuccess) return attr;
    const int64_t grid = d.p.producers + d.p.units;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreadsD), (size_t)d.p.lds_bytes, stream, d);
    return hipGetLastError();
}

template <int MT, int NW, bool K32>
hipError_t launch_stream_pieces(const Decode &d, int64_t pieces, hipStream_t stream) {
    if (pieces <= 2) return launch_stream<MT, NW, 2, K32>(d, stream);
    if (pieces <= 4) return launch_stream<MT, NW, 4, K32>(d, stream);
    if (pieces <= 8) return launch_stream<MT, NW, 8, K32>(d, stream);
    if (pieces <= 16) return launch_stream<MT, NW, 16, K32>(d, stream);
    return hipErrorInvalidConfiguration;
}

template <int MT, int NW>
hipError_t launch_stream_k(const Decode &d, int64_t pieces, hipStream_t stream) {
    return (d.a.k & 31) == 0 ? launch_stream_pieces<MT, NW, true>(d, pieces, stream)
                             : launch_stream_pieces<MT, NW, false>(d, pieces, stream);
}

}  // namespace

size_t decode_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
    return (size_t)make_decode_plan(m, n, k, r).bytes;
}

hipError_t launch_decode(const GemmArgs &a, hipStream_t stream) {
    const Decode d{a, make_decode_plan(a.m, a.n, a.k, a.r)};
    if (d.p.producers + d.p.units > 0x7FFFFFFF || d.p.lds_bytes > kLdsBudget) return hipErrorInvalidConfiguration;
    // 16-byte staging pieces per thread for the unit's x slice
    const int64_t pieces = (a.m * d.p.kslice / 8 + kThreadsD - 1) / kThreadsD;
    hipError_t e;
    if (d.p.mt == 1) e = launch_stream_k<1, 1>(d, pieces, stream);
    else if (d.p.mt == 2) e = launch_stream_k<2, 2>(d, pieces, stream);
    else e = launch_stream_k<4, 4>(d, pieces, stream);
    if (e != hipSuccess) return e;
    const dim3 fgrid((unsigned)((a.n + 255) / 256), (unsigned)a.m);
    hipLaunchKernelGGL(finish_kernel, fgrid, dim3(256), 0, stream, d);
    return hipGetLastError();
}

}  // namespace qerl
