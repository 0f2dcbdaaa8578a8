// mfma_tile.h -- the K loops of the large-m W4A16 GEMM (gemm.hip) on gfx950.
//
// A workgroup of four waves owns 256 consecutive weight rows; wave w owns
// rows 64w .. 64w+63 (four 16-row MFMA n-tiles) against all 16*MTW rows of
// its x tile (MTW 16-row m-tiles), accumulating in FP32 with BF16 MFMA
// 16x16x32.  e2m1 * e4m3 is exact in BF16, so the weights are decoded to
// BF16 in registers without rounding; the tensor scale s_t is left to the
// caller.
//
// Main loop (mfma_kloop): K in blocks of 128, with K permuted inside a block.
// The sum over K does not depend on its order, so lane quarter q of both MFMA
// operands takes the 32 columns 32q .. 32q+31 of the block -- 16 packed bytes
// and two scale bytes, one load each -- spread over the block's four MFMA
// steps (8 columns each).  Each wave reads its weight fragments straight from
// global memory into registers; the x tile goes global -> LDS by buffer DMA
// into one of two LDS tiles, so no register holds x in flight.  The loads of
// block s+1 are in flight while block s multiplies.
//
// LDS x tile: 16*MTW rows of 256 bytes, no padding; 16-byte chunk c of row r
// holds global chunk c ^ (r % 16), so the 16 rows that one MFMA operand read
// touches fall in 16 distinct bank groups.
//
// Plain loop (plain_kloop): 32 columns a step in natural order (lane quarter
// q: columns 8q .. 8q+7), operands from caller-supplied functions, for what
// the main loop does not cover.
#pragma once

#include "device_common.h"

namespace qerl {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTileK = 128;                 // K columns per main-loop block
constexpr int kTileRowBytes = kTileK * 2;   // bytes per x row of an LDS tile
constexpr int kPlainPitch = 40;             // BF16 elements per x row in the plain loop
constexpr int64_t kTileMaxLdx = (int64_t)1 << 22;  // main loop: 32-bit buffer offsets

// exact BF16 of e2m1 * e4m3 for the 8 elements of one packed 32-bit word
// (element 2i in the low nibble of byte i)
__device__ __forceinline__ bf16x8_t dequant8_p(uint32_t q, float s) {
    const f32x2_t f0 = QERL_FP4_PAIR_F32(q, 0), f1 = QERL_FP4_PAIR_F32(q, 1);
    const f32x2_t f2 = QERL_FP4_PAIR_F32(q, 2), f3 = QERL_FP4_PAIR_F32(q, 3);
    const uint4 u = make_uint4(pack_bf16x2(f0.x * s, f0.y * s), pack_bf16x2(f1.x * s, f1.y * s),
                               pack_bf16x2(f2.x * s, f2.y * s), pack_bf16x2(f3.x * s, f3.y * s));
    bf16x8_t v;
    __builtin_memcpy(&v, &u, 16);
    return v;
}

// acc[i][j] += (rows 16i.. of the LDS tile at pa, pitch_bytes apart) x (b_j)
template <int MTW>
__device__ __forceinline__ void mfma_step(const uint8_t *pa, int pitch_bytes, const bf16x8_t &b0, const bf16x8_t &b1,
                                          const bf16x8_t &b2, const bf16x8_t &b3, f32x4_t (&acc)[MTW][4]) {
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(pa + 16 * i * pitch_bytes);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b1, acc[i][1], 0, 0, 0);
        acc[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b2, acc[i][2], 0, 0, 0);
        acc[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b3, acc[i][3], 0, 0, 0);
    }
}

// Main loop over the full K blocks [b0, b1) (b1 * 128 <= k).
//   x_tile: row 0 of the x tile; rows at or past x_rows are read as zeros
//   w_packed, w_scales: row 0 of the workgroup's 256 weight rows; rows at or
//     past w_rows are read as zeros
//   t0, t1: two LDS tiles of 16 * MTW * 256 bytes, distinct arrays
// Needs ldx <= kTileMaxLdx and uniform arguments; ends with a barrier.
template <int MTW>
__device__ __forceinline__ void mfma_kloop(const uint16_t *x_tile, int64_t x_rows, int64_t ldx,
                                           const uint8_t *w_packed, const uint8_t *w_scales, int64_t w_rows,
                                           int64_t k, int64_t b0, int64_t b1, uint8_t *t0, uint8_t *t1,
                                           f32x4_t (&acc)[MTW][4]) {
    static_assert(MTW == 2 || MTW == 4 || MTW == 8, "x tile of 32, 64 or 128 rows");
    if (b0 >= b1) return;
    constexpr int kXRows = 16 * MTW;
    constexpr int kDma = MTW;  // DMA instructions per wave per block (1 KB = 4 rows each)
    // the wave index as a scalar: the DMA's LDS address must be uniform
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15,
              lq = lane >> 4;
    if (x_rows > kXRows) x_rows = kXRows;
    if (w_rows > 256) w_rows = 256;
    const int64_t kb = k >> 1, ks = k >> 4;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x_tile), 0,
                                                                         (int)(x_rows * ldx * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(w_packed), 0,
                                                                         (int)(w_rows * kb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(w_scales), 0,
                                                                         (int)(w_rows * ks), 0x00020000);
    // x DMA: instruction v of wave w fills LDS bytes [1024 (kDma w + v), +1024),
    // i.e. rows 4q .. 4q+3 with q = kDma w + v; lane l writes chunk l % 16 of
    // row 4q + l / 16 from global chunk (l % 16) ^ (row % 16).  Rows 16 apart
    // share the swizzle, so instruction v + 4 reuses the offset of v.
    constexpr int kXo = kDma < 4 ? kDma : 4;
    int xoff[kXo];
#pragma unroll
    for (int v = 0; v < kXo; ++v) {
        const int row = 4 * (kDma * wave + v) + (lane >> 4);
        xoff[v] = (int)((row * ldx + 8 * ((lane & 15) ^ (row & 15))) * 2);
    }
    const int xrow16 = (int)(16 * ldx * 2);
    // weight fragments of this lane: rows 64 wave + 16j + lr, columns 32lq ..
    // 32lq+31 of each block
    const int wrow = wave * 64 + lr;
    const int qoff = (int)(wrow * kb + 16 * lq), soff = (int)(wrow * ks + 2 * lq);
    const int qrow16 = (int)(16 * kb), srow16 = (int)(16 * ks);
    // A operand of MFMA step t, m-tile i: row 16i + lr, global chunk 4lq + t
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = lr * kTileRowBytes + (((4 * lq + t) ^ lr) << 4);

    auto dma_x = [&](uint8_t *dst, int64_t s) {
        const int k0 = (int)(s * kTileK);
#pragma unroll
        for (int v = 0; v < kDma; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(dst + 1024 * (kDma * wave + v)), 16,
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
    auto lds2 = [&](int j, int kq) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, soff, kq + j * srow16, 0);
    };
    auto load_w = [&](int64_t s) {
        const int k0 = (int)(s * kTileK);
        qn0 = ldq16(0, k0 >> 1);
        qn1 = ldq16(1, k0 >> 1);
        qn2 = ldq16(2, k0 >> 1);
        qn3 = ldq16(3, k0 >> 1);
        sn0 = lds2(0, k0 >> 4);
        sn1 = lds2(1, k0 >> 4);
        sn2 = lds2(2, k0 >> 4);
        sn3 = lds2(3, k0 >> 4);
    };
    uint4 qc0, qc1, qc2, qc3;
    uint32_t sc0, sc1, sc2, sc3;
    // block s from LDS tile cur while block s+1 streams into nxt
    auto block = [&](const uint8_t *cur, uint8_t *nxt, int64_t s) {
        const bool more = s + 1 < b1;  // uniform
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
            mfma_step<MTW>(cur + aoff[t], kTileRowBytes, dequant8_p(w0, f0), dequant8_p(w1, f1), dequant8_p(w2, f2),
                           dequant8_p(w3, f3), acc);
            // keep each step's decode next to its MFMAs (hoisting them all
            // raises register use past the budget)
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
    dma_x(t0, b0);
    load_w(b0);
    qc0 = qn0; qc1 = qn1; qc2 = qn2; qc3 = qn3;
    sc0 = sn0; sc1 = sn1; sc2 = sn2; sc3 = sn3;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int64_t s = b0; s < b1; s += 2) {
        block(t0, t1, s);
        if (s + 1 < b1) block(t1, t0, s + 1);
    }
}

// Plain loop over K columns [k0, k1) in steps of 32 (k0 % 8 == 0).
//   xpiece(m, kk): uint4, 8 BF16 of x tile row m at columns kk .. kk+7
//   wfrag(j, kk):  bf16x8_t, this lane's weight row 64 wave + 16j + lr at
//                  columns kk .. kk+7
//   tile: LDS of at least 16 * MTW * kPlainPitch * 2 bytes
// Uniform arguments; ends with a barrier.
template <int MTW, typename XPiece, typename WFrag>
__device__ __forceinline__ void plain_kloop(int64_t k0, int64_t k1, uint8_t *tile, XPiece xpiece, WFrag wfrag,
                                            f32x4_t (&acc)[MTW][4]) {
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    uint16_t *sx = reinterpret_cast<uint16_t *>(tile);  // [16 MTW][kPlainPitch]
    for (int64_t kc = k0; kc < k1; kc += 32) {
        for (int i = tid; i < 64 * MTW; i += 256) {
            const int row = i >> 2, col = (i & 3) * 8;
            *reinterpret_cast<uint4 *>(sx + row * kPlainPitch + col) = xpiece(row, kc + col);
        }
        const int64_t kk = kc + 8 * lq;
        const bf16x8_t b0 = wfrag(0, kk), b1 = wfrag(1, kk), b2 = wfrag(2, kk), b3 = wfrag(3, kk);
        __syncthreads();
        mfma_step<MTW>(reinterpret_cast<const uint8_t *>(sx + lr * kPlainPitch + 8 * lq), kPlainPitch * 2, b0, b1,
                       b2, b3, acc);
        __syncthreads();
    }
}

}  // namespace qerl
