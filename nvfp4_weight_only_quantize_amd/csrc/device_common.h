// device_common.h -- small device helpers shared by the gfx950 kernels of
// libqerl (vector types, BF16 packing, wave/block reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qerl {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even FP32 -> BF16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    uint16_t u;
    __builtin_memcpy(&u, &b, 2);
    return u;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
    bf16x2_t v;
    __builtin_memcpy(&v, &u, 4);
    return v;
}

// E2M1 pair decode: byte `sel` of `src` -> two BF16 values (low nibble in .x).
// The scale operand of the conversion contributes only its exponent, so 1.0f
// gives the plain E2M1 values.
#define QERL_FP4_PAIR_BF16(src, sel) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((src), 1.0f, (sel))
#define QERL_FP4_PAIR_F32(src, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((src), 1.0f, (sel))
// OCP E4M3 ("FN") byte `sel` of `src` -> FP32.
#define QERL_E4M3_F32(src, sel) __builtin_amdgcn_cvt_f32_fp8((int)(src), (sel))

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (T)__shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum over a 256-thread workgroup; every thread receives the total.
__device__ __forceinline__ float block_sum_256(float v, float *scratch /* >= 4 floats of LDS */) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // scratch may still be read by a previous call
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

// Counter-based Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): round
// multipliers and key increments (Weyl sequence constants) as published.
struct U64x4 { uint64_t v[4]; };
__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
    constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
    constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull, kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t hi0 = __umul64hi(kMul0, c0), lo0 = kMul0 * c0;
        const uint64_t hi1 = __umul64hi(kMul1, c2), lo1 = kMul1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    return U64x4{{c0, c1, c2, c3}};
}

}  // namespace qerl
