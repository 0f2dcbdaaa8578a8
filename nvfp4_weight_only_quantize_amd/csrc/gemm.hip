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
//   prefill_kernel   256 x 128 output tiles, x tiles double-buffered in LDS,
//                    weights decoded to exact BF16 (e2m1 * e4m3) in registers,
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
// Workgroup tile 128 (rows of x) x 256 (weight rows); four waves side by
// side along n, each the full 128 x 64 (8 x 4 MFMA 16x16x32 tiles), so no
// weight fragment is fetched twice.  Each wave decodes its own weight
// fragments straight from global memory into registers (e2m1 * e4m3 is exact
// in BF16); x tiles go from global memory to LDS by DMA (buffer loads with
// the LDS bit), double-buffered in two LDS arrays, and no register holds x in
// flight.
//
// The main loop takes K in blocks of 128 and permutes K inside a block: the
// sum over K does not depend on its order, so lane quarter q of both operands
// takes the 32 columns 32q .. 32q+31 -- 16 packed bytes and two scale bytes,
// one load each -- split over the block's four MFMA steps.  The loads of
// block s+1 are in flight while block s multiplies.  What is left of K past
// the last full block, and the LoRA product as 2r extra K columns (t hi/lo x
// B twice), go through a plain loop of 32 columns a step.
//
// LDS x tile: 128 rows of 256 bytes, no padding; 16-byte chunk c of row r
// holds global chunk c ^ (r % 16), so that the 16 rows one MFMA operand read
// touches fall in 16 distinct bank groups.
constexpr int PBM = 128, PBN = 256, PBK = 128;
constexpr int kXTileBytes = PBM * PBK * 2;
constexpr int kSlowPitch = 40;  // BF16 elements per row in the plain loop's x tile

__shared__ __attribute__((aligned(1024))) uint8_t g_xtile0[kXTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_xtile1[kXTileBytes];

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

// exact BF16 of e2m1 * e4m3 for the 8 elements of one packed 32-bit word
__device__ __forceinline__ bf16x8_t dequant8_p(uint32_t q, float s) {
    const f32x2_t f0 = QERL_FP4_PAIR_F32(q, 0), f1 = QERL_FP4_PAIR_F32(q, 1);
    const f32x2_t f2 = QERL_FP4_PAIR_F32(q, 2), f3 = QERL_FP4_PAIR_F32(q, 3);
    const uint4 u = make_uint4(pack_bf16x2(f0.x * s, f0.y * s), pack_bf16x2(f1.x * s, f1.y * s),
                               pack_bf16x2(f2.x * s, f2.y * s), pack_bf16x2(f3.x * s, f3.y * s));
    bf16x8_t v;
    __builtin_memcpy(&v, &u, 16);
    return v;
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

typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(256, 2) void prefill_kernel(Gemm g) {
    const GemmArgs &a = g.a;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous range of tiles (n fastest), so the workgroups sharing an x
    // row block also share that XCD's L2
    const int64_t tiles_n = (a.n + PBN - 1) / PBN, tiles = tiles_n * ((a.m + PBM - 1) / PBM);
    const int64_t b = blockIdx.x, x8 = b % 8, q8 = tiles / 8, r8 = tiles % 8;
    const int64_t tile = x8 * q8 + (x8 < r8 ? x8 : r8) + b / 8;
    const int64_t m0 = (tile / tiles_n) * PBM, n0 = (tile % tiles_n) * PBN;
    const int64_t klora = 2 * (int64_t)a.r;
    const int64_t ktot = a.k + klora;

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- main K range, 128 columns a block ----
    // Operands come through buffer loads: one resource per operand for the
    // whole tile, per-lane 32-bit offsets, the block and the row group in the
    // uniform offset.  Rows past m or n lie past the resource's end and read
    // as zeros (their outputs are discarded).  The 32-bit offsets need
    // 256 * ldx < 2^31; wider rows take the plain loop.
    const int64_t rows_m = a.m - m0 < PBM ? a.m - m0 : PBM, rows_n = a.n - n0 < PBN ? a.n - n0 : PBN;
    const int64_t kb = a.k >> 1, ks = a.k >> 4;
    const int64_t blocks = a.ldx <= ((int64_t)1 << 22) ? a.k / PBK : 0;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x + m0 * a.ldx), 0, (int)(blocks ? rows_m * a.ldx * 2 : 0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.packed + n0 * kb), 0, (int)(blocks ? rows_n * kb : 0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.scales + n0 * ks), 0, (int)(blocks ? rows_n * ks : 0), 0x00020000);
    // x DMA: instruction v (< 8) of wave w fills LDS bytes [1024 (8w + v), +1024)
    // = rows 4q .. 4q+3 with q = 8w + v; lane l writes chunk l % 16 of row
    // 4q + l / 16, i.e. global chunk (l % 16) ^ (row % 16), and row % 16 only
    // depends on v % 4
    int xoff[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int row = 4 * (8 * wave + v) + (lane >> 4);
        xoff[v] = (int)((row * a.ldx + 8 * ((lane & 15) ^ (row & 15))) * 2);
    }
    const int xrow16 = (int)(16 * a.ldx * 2);
    // weight fragments of this lane: rows 64*wave + 16j + lr, columns 32lq ..
    // 32lq+31 of each block
    const int wrow = wave * 64 + lr;
    const int qoff = (int)(wrow * kb + 16 * lq), soff = (int)(wrow * ks + 2 * lq);
    const int qrow16 = (int)(16 * kb), srow16 = (int)(16 * ks);
    // A operand of MFMA step t, m-tile i: row 16i + lr, global chunk 4lq + t
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = lr * 256 + (((4 * lq + t) ^ lr) << 4);

    auto dma_x = [&](uint8_t *dst, int64_t s) {
        const int k0 = (int)(s * PBK);
#pragma unroll
        for (int v = 0; v < 8; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(dst + 1024 * (8 * wave + v)), 16,
                                                     xoff[v & 3], 2 * k0 + (v >> 2) * xrow16, 0, 0);
    };
    uint4 qn0, qn1, qn2, qn3;
    uint32_t sn0, sn1, sn2, sn3;
    auto ldq16 = [&](int j, int kq) {
        const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, kq + j * qrow16, 0);
        uint4 o;
        __builtin_memcpy(&o, &v, 16);
        return o;
    };
    auto lds2 = [&](int j, int kq) { return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, soff, kq + j * srow16, 0); };
    auto load_w = [&](int64_t s) {
        const int k0 = (int)(s * PBK);
        qn0 = ldq16(0, k0 >> 1);
        qn1 = ldq16(1, k0 >> 1);
        qn2 = ldq16(2, k0 >> 1);
        qn3 = ldq16(3, k0 >> 1);
        sn0 = lds2(0, k0 >> 4);
        sn1 = lds2(1, k0 >> 4);
        sn2 = lds2(2, k0 >> 4);
        sn3 = lds2(3, k0 >> 4);
    };
    // one MFMA step over the 8 x 4 tiles; A row 16i + lr at byte pa + 4096 i
    auto mma_t = [&](const uint8_t *pa, const bf16x8_t &b0, const bf16x8_t &b1, const bf16x8_t &b2,
                     const bf16x8_t &b3, int pitch_bytes) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(pa + 16 * i * pitch_bytes);
            acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b0, acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b1, acc[i][1], 0, 0, 0);
            acc[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b2, acc[i][2], 0, 0, 0);
            acc[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b3, acc[i][3], 0, 0, 0);
        }
    };
    uint4 qc0, qc1, qc2, qc3;
    uint32_t sc0, sc1, sc2, sc3;
    // block s from LDS tile cur while block s+1 streams into nxt
    auto block = [&](const uint8_t *cur, uint8_t *nxt, int64_t s) {
        const bool more = s + 1 < blocks;  // uniform
        if (more) {
            dma_x(nxt, s + 1);
            load_w(s + 1);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool hi = t >= 2;  // scale byte 1 covers the last 16 of the lane's 32 columns
            const float f0 = hi ? QERL_E4M3_F32(sc0, 1) : QERL_E4M3_F32(sc0, 0);
            const float f1 = hi ? QERL_E4M3_F32(sc1, 1) : QERL_E4M3_F32(sc1, 0);
            const float f2 = hi ? QERL_E4M3_F32(sc2, 1) : QERL_E4M3_F32(sc2, 0);
            const float f3 = hi ? QERL_E4M3_F32(sc3, 1) : QERL_E4M3_F32(sc3, 0);
            const uint32_t w0 = t == 0 ? qc0.x : t == 1 ? qc0.y : t == 2 ? qc0.z : qc0.w;
            const uint32_t w1 = t == 0 ? qc1.x : t == 1 ? qc1.y : t == 2 ? qc1.z : qc1.w;
            const uint32_t w2 = t == 0 ? qc2.x : t == 1 ? qc2.y : t == 2 ? qc2.z : qc2.w;
            const uint32_t w3 = t == 0 ? qc3.x : t == 1 ? qc3.y : t == 2 ? qc3.z : qc3.w;
            mma_t(cur + aoff[t], dequant8_p(w0, f0), dequant8_p(w1, f1), dequant8_p(w2, f2), dequant8_p(w3, f3),
                  256);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more) {
            qc0 = qn0; qc1 = qn1; qc2 = qn2; qc3 = qn3;
            sc0 = sn0; sc1 = sn1; sc2 = sn2; sc3 = sn3;
        }
        // this wave's DMA into nxt must land before any wave reads it
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    if (blocks > 0) {
        dma_x(g_xtile0, 0);
        load_w(0);
        qc0 = qn0; qc1 = qn1; qc2 = qn2; qc3 = qn3;
        sc0 = sn0; sc1 = sn1; sc2 = sn2; sc3 = sn3;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int64_t s = 0; s < blocks; s += 2) {
            block(g_xtile0, g_xtile1, s);
            if (s + 1 < blocks) block(g_xtile1, g_xtile0, s + 1);
        }
    }
    // ---- the rest: K past the last full block and the LoRA columns, 32 a
    // step in natural order (lane quarter q: columns 8q .. 8q+7) ----
    uint16_t *sx = reinterpret_cast<uint16_t *>(g_xtile0);  // [PBM][kSlowPitch]
    const int xr2 = tid >> 2, xc2 = (tid & 3) * 8;
    for (int64_t k0 = blocks * PBK; k0 < ktot; k0 += 32) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<uint4 *>(sx + (xr2 + 64 * u) * kSlowPitch + xc2) =
                x_piece_ext(g, m0 + xr2 + 64 * u, k0 + xc2, klora);
        const int64_t kk = k0 + 8 * lq, nw = n0 + wave * 64 + lr;
        const bf16x8_t b0 = w_frag_ext(a, nw, kk, klora);
        const bf16x8_t b1 = w_frag_ext(a, nw + 16, kk, klora);
        const bf16x8_t b2 = w_frag_ext(a, nw + 32, kk, klora);
        const bf16x8_t b3 = w_frag_ext(a, nw + 48, kk, klora);
        __syncthreads();
        mma_t(reinterpret_cast<const uint8_t *>(sx + lr * kSlowPitch + 8 * lq), b0, b1, b2, b3, kSlowPitch * 2);
        __syncthreads();
    }
    const float st_scale = *a.tensor_scale;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + 16 * i + 4 * lq + v;
                const int64_t n = n0 + wave * 64 + 16 * j + lr;
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
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace qerl
