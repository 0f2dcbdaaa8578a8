// mfma_tile.h -- the K loops of the large-m W4A16 GEMM (gemm.hip) on gfx950.
//
// A workgroup of NWV waves (4 or 8) owns 64 NWV consecutive weight rows;
// wave w owns rows 64w .. 64w+63 (four 16-row MFMA n-tiles) against all
// 16*MTW rows of its x tile (MTW 16-row m-tiles), accumulating in FP32 with
// BF16 MFMA 16x16x32.  e2m1 * e4m3 is exact in BF16, so the weights are decoded to
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

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).  Unlike an
// inline-asm wait, the compiler's own wait analysis takes this one into
// account.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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
//   w_packed, w_scales: row 0 of the workgroup's 64 NWV weight rows; rows at
//     or past w_rows are read as zeros
//   t0, t1: two LDS tiles of 16 * MTW * 256 bytes, distinct arrays
//   SCL: the scales come from an LDS tile (sc_tile: row r of the workgroup's
//     rows at sc_tile + r * sc_pitch, the 8 bytes of block b0 + i at 8 i),
//     staged and made visible by the caller, instead of 2-byte global loads
// Needs ldx <= kTileMaxLdx and uniform arguments; ends with a barrier.
//   SCD: the scales travel by DMA in chunks of four blocks (32 contiguous
//     bytes per weight row) into the LDS tiles sd0, sd1 (64 NWV rows of 32
//     bytes each), one chunk ahead, and each block reads its pairs from
//     there: one 16-byte DMA lane per half row instead of a 2-byte load per
//     lane and block (16 cache lines an instruction).  Needs k % 256 == 0 and
//     b0 even (16-byte aligned sources); the range check of the buffer
//     (offset + soffset against its size) zero-fills what a chunk reads past
//     the last row.
template <int MTW, int NWV = 4, int WD = 1, bool SCL = false, bool SCD = false>
__device__ __forceinline__ void mfma_kloop(const uint16_t *x_tile, int64_t x_rows, int64_t ldx,
                                           const uint8_t *w_packed, const uint8_t *w_scales, int64_t w_rows,
                                           int64_t k, int64_t b0, int64_t b1, uint8_t *t0, uint8_t *t1,
                                           f32x4_t (&acc)[MTW][4], const uint8_t *sc_tile = nullptr,
                                           int sc_pitch = 0, uint8_t *sd0 = nullptr, uint8_t *sd1 = nullptr) {
    static_assert(!SCD || (WD == 1 && !SCL), "scales by DMA: weights one block ahead, no LDS scale tile");
    static_assert(MTW == 2 || MTW == 4 || MTW == 8, "x tile of 32, 64 or 128 rows");
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    static_assert(4 * MTW % NWV == 0, "whole DMA instructions per wave");
    static_assert(WD == 1 || WD == 2, "weights one or two blocks ahead");
    static_assert(!SCL || WD == 1, "LDS scales with weights one block ahead");
    if (b0 >= b1) return;
    constexpr int kXRows = 16 * MTW;
    constexpr int kDma = 4 * MTW / NWV;  // DMA instructions per wave per block (1 KB = 4 rows each)
    // the wave index as a scalar: the DMA's LDS address must be uniform
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15,
              lq = lane >> 4;
    if (x_rows > kXRows) x_rows = kXRows;
    if (w_rows > 64 * NWV) w_rows = 64 * NWV;
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
    auto ldq16 = [&](int j, int kq) {
        const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, kq + j * qrow16, 0);
        uint4 o;
        __builtin_memcpy(&o, &v, 16);
        return o;
    };
    auto lds2 = [&](int j, int kq) { return __builtin_amdgcn_raw_buffer_load_b16(rs, soff, kq + j * srow16, 0); };
    // the weight fragments of one block: named members (an array of them
    // ends up in scratch memory), one set per block in flight; the sets
    // rotate statically over an unrolled loop, since copying a set would
    // make the compiler wait for the loads that fill it.  The scale pairs stay
    // 16-bit until used: widened at the loop head, they would be waited for
    // there.
    struct WSet {
        uint4 q0, q1, q2, q3;
        uint16_t c0, c1, c2, c3;
    };
    auto load_w = [&](WSet &w, int64_t s) {
        const int k0 = (int)(s * kTileK);
        w.q0 = ldq16(0, k0 >> 1);
        w.q1 = ldq16(1, k0 >> 1);
        w.q2 = ldq16(2, k0 >> 1);
        w.q3 = ldq16(3, k0 >> 1);
        if (SCD) {  // the block reads its scale pairs from the DMA'd chunk
        } else if (SCL) {
            const uint8_t *sp = sc_tile + wrow * sc_pitch + (int)(s - b0) * 8 + 2 * lq;
            w.c0 = *reinterpret_cast<const uint16_t *>(sp);
            w.c1 = *reinterpret_cast<const uint16_t *>(sp + 16 * sc_pitch);
            w.c2 = *reinterpret_cast<const uint16_t *>(sp + 32 * sc_pitch);
            w.c3 = *reinterpret_cast<const uint16_t *>(sp + 48 * sc_pitch);
        } else {
            w.c0 = lds2(0, k0 >> 4);
            w.c1 = lds2(1, k0 >> 4);
            w.c2 = lds2(2, k0 >> 4);
            w.c3 = lds2(3, k0 >> 4);
        }
    };
    // block s from LDS tile cur and weight set wc while x of block s+1 streams
    // into nxt and the weights of block s+WD into wl.  Every block issues its
    // weight loads (clamped past the end), so the wait at its end always
    // leaves exactly the 8 loads of block s+WD in flight when WD == 2.
    // SCD chunk DMA, instruction i of wave w: lane l copies half l % 2 of the
    // 32 bytes of row 64w + 32i + l / 2 (LDS rows of 32 bytes, 1 KB an
    // instruction)
    int sdoff = 0;
    if (SCD) sdoff = (int)(((int64_t)wave * 64 + (lane >> 1)) * ks + 16 * (lane & 1));
    auto dma_sc = [&](uint8_t *dst, int64_t s) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + 2048 * wave + 1024 * i), 16, sdoff,
                                                     (int)(8 * s + 32 * i * ks), 0, 0);
    };
    // SCD: sdc holds the chunk of block s; when cn, s ends its chunk and the
    // next chunk goes to sdn (both uniform)
    auto block = [&](const uint8_t *cur, uint8_t *nxt, const WSet &wc, WSet &wl, int64_t s,
                     const uint8_t *sdc = nullptr, uint8_t *sdn = nullptr, bool cn = false) {
        uint16_t c0 = wc.c0, c1 = wc.c1, c2 = wc.c2, c3 = wc.c3;
        if (SCD && s < b1) {  // uniform: the scale pairs, before any load is issued
            const uint8_t *sp = sdc + wrow * 32 + (int)((s - b0) & 3) * 8 + 2 * lq;
            c0 = *reinterpret_cast<const uint16_t *>(sp);
            c1 = *reinterpret_cast<const uint16_t *>(sp + 16 * 32);
            c2 = *reinterpret_cast<const uint16_t *>(sp + 32 * 32);
            c3 = *reinterpret_cast<const uint16_t *>(sp + 48 * 32);
        }
        if (s + 1 < b1) dma_x(nxt, s + 1);  // uniform
        if (SCD && cn && s + 1 < b1) dma_sc(sdn, s + 1);
        load_w(wl, s + WD < b1 ? s + WD : b1 - 1);
        if (s < b1) {  // uniform
            // step t's MFMAs are issued interleaved with the decode of step
            // t+1: one wave issues in order, so a decode placed wholly before
            // or after a run of MFMAs would leave one of the two pipes idle
            auto decode_step = [&](int t, bf16x8_t &d0, bf16x8_t &d1, bf16x8_t &d2, bf16x8_t &d3) {
                const bool hi = t >= 2;  // scale byte 1 covers the last 16 of the lane's 32 columns
                const float f0 = hi ? QERL_E4M3_F32(c0, 1) : QERL_E4M3_F32(c0, 0);
                const float f1 = hi ? QERL_E4M3_F32(c1, 1) : QERL_E4M3_F32(c1, 0);
                const float f2 = hi ? QERL_E4M3_F32(c2, 1) : QERL_E4M3_F32(c2, 0);
                const float f3 = hi ? QERL_E4M3_F32(c3, 1) : QERL_E4M3_F32(c3, 0);
                d0 = dequant8_p(t == 0 ? wc.q0.x : t == 1 ? wc.q0.y : t == 2 ? wc.q0.z : wc.q0.w, f0);
                d1 = dequant8_p(t == 0 ? wc.q1.x : t == 1 ? wc.q1.y : t == 2 ? wc.q1.z : wc.q1.w, f1);
                d2 = dequant8_p(t == 0 ? wc.q2.x : t == 1 ? wc.q2.y : t == 2 ? wc.q2.z : wc.q2.w, f2);
                d3 = dequant8_p(t == 0 ? wc.q3.x : t == 1 ? wc.q3.y : t == 2 ? wc.q3.z : wc.q3.w, f3);
            };
            constexpr int kMf = 4 * MTW;                  // MFMAs per step
            constexpr int kVa = (68 + kMf - 1) / kMf;     // decode VALU per MFMA slot
            bf16x8_t e0, e1, e2, e3, o0, o1, o2, o3;      // decoded fragments of even / odd steps
            decode_step(0, e0, e1, e2, e3);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t == 0) decode_step(1, o0, o1, o2, o3);
                if (t == 1) decode_step(2, e0, e1, e2, e3);
                if (t == 2) decode_step(3, o0, o1, o2, o3);
                if (t % 2 == 0)
                    mfma_step<MTW>(cur + aoff[t], kTileRowBytes, e0, e1, e2, e3, acc);
                else
                    mfma_step<MTW>(cur + aoff[t], kTileRowBytes, o0, o1, o2, o3, acc);
                __builtin_amdgcn_sched_group_barrier(0x100, MTW, 0);  // the step's x fragment reads
#pragma unroll
                for (int i = 0; i < kMf; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);  // then a share of the decode
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // this wave's DMA into nxt and the weights of block s+1 must land
        // before the next block; with WD == 2 the loads just issued may not
        if (WD == 1)
            wait_vmcnt<0>();
        else
            wait_vmcnt<8>();
        __syncthreads();
    };
    WSet w0, w1, w2;
    dma_x(t0, b0);
    if (SCD) dma_sc(sd0, b0);
    load_w(w0, b0);
    if (WD == 2) load_w(w1, b0 + 1 < b1 ? b0 + 1 : b1 - 1);
    wait_vmcnt<0>();
    __syncthreads();
    if (SCD) {  // chunks of four blocks alternate between sd0 and sd1
        for (int64_t s = b0; s < b1; s += 8) {
            block(t0, t1, w0, w1, s, sd0, sd1, false);
            block(t1, t0, w1, w0, s + 1, sd0, sd1, false);
            block(t0, t1, w0, w1, s + 2, sd0, sd1, false);
            block(t1, t0, w1, w0, s + 3, sd0, sd1, true);
            block(t0, t1, w0, w1, s + 4, sd1, sd0, false);
            block(t1, t0, w1, w0, s + 5, sd1, sd0, false);
            block(t0, t1, w0, w1, s + 6, sd1, sd0, false);
            block(t1, t0, w1, w0, s + 7, sd1, sd0, true);
        }
    } else if (WD == 1) {
        for (int64_t s = b0; s < b1; s += 2) {
            block(t0, t1, w0, w1, s);
            block(t1, t0, w1, w0, s + 1);
        }
    } else {
        for (int64_t s = b0; s < b1; s += 6) {
            block(t0, t1, w0, w2, s);
            block(t1, t0, w1, w0, s + 1);
            block(t0, t1, w2, w1, s + 2);
            block(t1, t0, w0, w2, s + 3);
            block(t0, t1, w1, w0, s + 4);
            block(t1, t0, w2, w1, s + 5);
        }
    }
}

// Plain loop over K columns [k0, k1) in steps of 32 (k0 % 8 == 0).
//   xpiece(m, kk): uint4, 8 BF16 of x tile row m at columns kk .. kk+7
//   wfrag(j, kk):  bf16x8_t, this lane's weight row 64 wave + 16j + lr at
//                  columns kk .. kk+7
//   tile: LDS of at least 16 * MTW * kPlainPitch * 2 bytes
// Uniform arguments; ends with a barrier.
template <int MTW, int NWV = 4, typename XPiece, typename WFrag>
__device__ __forceinline__ void plain_kloop(int64_t k0, int64_t k1, uint8_t *tile, XPiece xpiece, WFrag wfrag,
                                            f32x4_t (&acc)[MTW][4]) {
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    uint16_t *sx = reinterpret_cast<uint16_t *>(tile);  // [16 MTW][kPlainPitch]
    for (int64_t kc = k0; kc < k1; kc += 32) {
        for (int i = tid; i < 64 * MTW; i += 64 * NWV) {
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
