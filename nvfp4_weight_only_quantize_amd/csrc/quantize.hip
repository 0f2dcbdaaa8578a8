// quantize.hip -- BF16 -> NVFP4 quantizer for gfx950.
//
// Block scaling of the cuDNN formula quoted on "QeRL: NVFP4-Quantized
// Reinforcement Learning -- Redefining Efficiency in AI Training and
// Inference", section "NVFP4: NVIDIA's FP4 Format": per block of 16 values
// along K, scale = round_up(amax / 6) as an E4M3 byte (relative to an FP32
// tensor scale, the second level of the same section) and each value rounded
// to nearest-even on the E2M1 grid.
//
// Two HBM passes (the tensor amax must be known before any block is encoded):
//   pass 1  amax_kernel: 16-byte loads, integer max of (bits & 0x7FFF) -- exact
//           for BF16 magnitudes and >= 0x7F80 exactly when a value is Inf/NaN;
//           one partial per workgroup into the workspace.
//   pass 2  encode_kernel: every workgroup folds the partials into s_t, then
//           each thread encodes one 16-element block: 32 B in, 8 B + 1 B out.
//
// Exactness: s_t = fl32(amax / 2688) is computed as a double quotient rounded
// to float (double rounding is harmless since 53 >= 2*24 + 2).  Block-scale
// decisions compare E4M3 * 6 * s_t (<= 30 significant bits) with the block
// amax in double, exactly.  Element decisions compare |w| with c * E4M3 * s_t
// for the seven E2M1 midpoints c through the sign of one fused multiply-add
// fmaf(c * E4M3, s_t, -|w|): c * E4M3 is exact in float and the fma rounds the
// exact difference once, so its sign is exact whenever the difference cannot
// fall below the float subnormal range -- guaranteed for s_t >= 2^-90 (all
// operands are then multiples of 2^-133).  Smaller s_t takes a double path.
//
// Fast element path (deterministic rounding, s_t in [2^-80, 2^80] with more
// than 8 significant bits): the hardware FP32 -> E2M1 conversion rounds to
// nearest-even on the E2M1 grid and saturates at 6 (checked exhaustively over
// every float in [2^-9, 16) and its negative), so it decides each element
// from a quotient q ~ w / (e s_t) that is on the same side of every midpoint
// c as the exact one.  Why that holds: with s_t of more than 8 significant
// bits, c e s_t has more significant bits than any BF16 |w|, so |w| is never
// a midpoint exactly, and when |w| != c e s_t the two differ by at least
// 2^-33 relative (|w| has 8 significant bits, c e s_t at most 33).  1 /
// (e s_t), taken in double, is split into r_hi of 16 significant bits and r_lo
// = fl(r - r_hi), together within 2^-39 relative of it; w r_hi is exact (8 + 16
// bits) and s = fma(w, r_lo, w r_hi) rounds w (r_hi + r_lo) once, so s is on
// the exact side of every midpoint or equal to one (midpoints are floats and
// rounding is monotone), and an element whose s is equal to one (low 21
// mantissa bits zero) is decided again by the comparisons above.
#include "device_common.h"
#include "qerl_internal.h"

namespace qerl {
namespace {

constexpr int kThreads = 256;
// amax pass: loads in flight per thread and workgroups (two per CU on 256
// CUs; 7% faster over a 32B-shaped layer than four loads on 1024 workgroups)
constexpr int kAmaxLoads = 8;
constexpr int kAmaxBlocks = 512;
static_assert(kAmaxBlocks <= kAmaxMaxBlocks, "partial maxima fit the workspace");

__device__ __forceinline__ uint32_t absmax_pair(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}
__device__ __forceinline__ uint32_t absmax_vec(uint4 v) {
    return max(max(absmax_pair(v.x), absmax_pair(v.y)), max(absmax_pair(v.z), absmax_pair(v.w)));
}

// max of (bits & 0x7FFF) over the 16 BF16 values of two vectors, two at a
// time in 16-bit halves
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t abs_pair16(uint32_t w) {
    u16x2_t h;
    const uint32_t a = w & 0x7FFF7FFFu;
    __builtin_memcpy(&h, &a, 4);
    return h;
}
__device__ __forceinline__ uint32_t absmax16(uint4 v0, uint4 v1) {
    u16x2_t m = __builtin_elementwise_max(abs_pair16(v0.x), abs_pair16(v0.y));
    m = __builtin_elementwise_max(m, abs_pair16(v0.z));
    m = __builtin_elementwise_max(m, abs_pair16(v0.w));
    m = __builtin_elementwise_max(m, abs_pair16(v1.x));
    m = __builtin_elementwise_max(m, abs_pair16(v1.y));
    m = __builtin_elementwise_max(m, abs_pair16(v1.z));
    m = __builtin_elementwise_max(m, abs_pair16(v1.w));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t *__restrict__ w, int64_t n,
                                                        int64_t k, int64_t ldw,
                                                        uint32_t *__restrict__ partial) {
    uint32_t m = 0;
    const int64_t vpr = k >> 3;  // 16-byte vectors per row
    if (ldw == k) {
        const uint4 *p = reinterpret_cast<const uint4 *>(w);
        const int64_t total = n * vpr;
        const int64_t stride = (int64_t)gridDim.x * kThreads;
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        // kAmaxLoads 16-byte loads in flight per thread, non-temporal: this
        // pass reads the weight once and nothing re-reads it before the
        // encoder's own pass over the whole tensor
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t *pv = reinterpret_cast<const u32x4_t *>(w);
        for (; i + (kAmaxLoads - 1) * stride < total; i += kAmaxLoads * stride) {
            u32x4_t v[kAmaxLoads];
#pragma unroll
            for (int u = 0; u < kAmaxLoads; ++u) v[u] = __builtin_nontemporal_load(pv + i + u * stride);
#pragma unroll
            for (int u = 0; u < kAmaxLoads; ++u) m = max(m, absmax_vec(make_uint4(v[u].x, v[u].y, v[u].z, v[u].w)));
        }
        for (; i < total; i += stride) m = max(m, absmax_vec(p[i]));
    } else {
        for (int64_t row = blockIdx.x; row < n; row += gridDim.x) {
            const uint4 *p = reinterpret_cast<const uint4 *>(w + row * ldw);
            for (int64_t c = threadIdx.x; c < vpr; c += kThreads) m = max(m, absmax_vec(p[c]));
        }
    }
    __shared__ uint32_t red[kThreads / kWave];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Exact E4M3 value of code c in 0..126 (non-negative, non-NaN).
__device__ __forceinline__ float e4m3_value(int c) {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? (float)m * 0x1p-9f
                  : __uint_as_float(((uint32_t)(e + 120) << 23) | ((uint32_t)m << 20));
}

// 1 / E4M3(c) rounded to double, c = 1 .. 126 (0 for c = 0): a power of two
// times the rounded inverse of the 3-bit mantissa's significand (normal
// codes), or 512 / c (subnormal codes); the quotients are compile-time
// constants.
__device__ __forceinline__ double e4m3_inverse(int c) {
    constexpr double kNorm[8] = {8.0 / 8, 8.0 / 9, 8.0 / 10, 8.0 / 11, 8.0 / 12, 8.0 / 13, 8.0 / 14, 8.0 / 15};
    constexpr double kSub[8] = {0.0, 512.0 / 1, 512.0 / 2, 512.0 / 3, 512.0 / 4, 512.0 / 5, 512.0 / 6, 512.0 / 7};
    if (c <= 0 || c > 126) return 0.0;
    const int e = c >> 3, m = c & 7;
    return e == 0 ? kSub[m] : __builtin_ldexp(kNorm[m], 7 - e);  // E4M3(c) = 2^(e-7) (8 + m) / 8
}

// Approximate least E4M3 code with value >= t (t >= 0); corrected exactly below.
__device__ __forceinline__ int e4m3_ceil_code_guess(float t) {
    if (!(t > 0.0f)) return 0;
    if (t >= 448.0f) return 126;
    if (t < 0x1p-6f) return min((int)ceilf(t * 512.0f), 8);
    const uint32_t u = __float_as_uint(t);
    int c = (((int)(u >> 23) - 120) << 3) | (int)((u >> 20) & 7);
    if (u & 0xFFFFFu) ++c;
    return min(c, 126);
}

// Least E4M3 code v with E4M3(v) * 6 * s_t >= amax_b (saturating at 448).
// inv6st ~ 1 / (6 s_t) seeds the search (any approximation is corrected).
__device__ __forceinline__ int scale_code_round_up(float amax_b, float st, float inv6st) {
    const double s6 = 6.0 * (double)st;  // exact
    const double a = (double)amax_b;
    if (448.0 * s6 < a) return 126;
    int c = e4m3_ceil_code_guess(amax_b * inv6st);
    while (c > 0 && (double)e4m3_value(c - 1) * s6 >= a) --c;
    while (c < 126 && (double)e4m3_value(c) * s6 < a) ++c;
    return c;
}

// Nearest E4M3 value to amax_b / (6 s_t), ties to the even code, saturating.
__device__ __forceinline__ int scale_code_rne(float amax_b, float st, float inv6st) {
    const double s6 = 6.0 * (double)st;
    const double a = (double)amax_b;
    const int hi = scale_code_round_up(amax_b, st, inv6st);
    const double vhi = (double)e4m3_value(hi);
    if (vhi * s6 < a) return 126;
    if (hi == 0 || vhi * s6 == a) return hi;
    const double vlo = (double)e4m3_value(hi - 1);
    const double two_a = 2.0 * a, mid = (vlo + vhi) * s6;  // both exact
    if (two_a < mid) return hi - 1;
    if (two_a > mid) return hi;
    return ((hi - 1) & 1) ? hi : hi - 1;
}

// The same two decisions in float for s_t >= 2^-90, each comparison the sign
// of one fma: 6 E4M3(c) and 6 (E4M3(c-1) + E4M3(c)) are exact in float, and
// fmaf(x, s_t, -amax_b) rounds the exact difference once, so its sign is
// exact (as for the elements below).  The guess from amax_b * inv6st is
// within one code of the answer (its relative error, ~2^-22, is far below
// the 1/15 spacing of E4M3 values), so one step corrects it.
__device__ __forceinline__ int scale_code_round_up_f32(float amax_b, float st, float inv6st) {
    int c = e4m3_ceil_code_guess(amax_b * inv6st);
    if (c > 0 && __builtin_fmaf(6.0f * e4m3_value(c - 1), st, -amax_b) >= 0.0f) --c;
    else if (c < 126 && __builtin_fmaf(6.0f * e4m3_value(c), st, -amax_b) < 0.0f) ++c;
    return c;
}

__device__ __forceinline__ int scale_code_rne_f32(float amax_b, float st, float inv6st) {
    const int hi = scale_code_round_up_f32(amax_b, st, inv6st);
    const float vhi = e4m3_value(hi);
    const float dhi = __builtin_fmaf(6.0f * vhi, st, -amax_b);
    if (dhi < 0.0f) return 126;  // above 448: saturate
    if (hi == 0 || dhi == 0.0f) return hi;
    // 2 amax_b against (vlo + vhi) 6 s_t: the sum of neighbours is exact
    const float d = __builtin_fmaf(6.0f * (e4m3_value(hi - 1) + vhi), st, -2.0f * amax_b);
    if (d > 0.0f) return hi - 1;
    if (d < 0.0f) return hi;
    return ((hi - 1) & 1) ? hi : hi - 1;
}

// E2M1 midpoints between grid neighbours and which side a tie takes: at .75,
// 1.75 and 3.5 the upper neighbour has the even code, elsewhere the lower.
__device__ __forceinline__ uint32_t e2m1_mag_f32(float a, const float (&ce)[7], float st) {
    uint32_t mag = 0;
    mag += __builtin_fmaf(ce[0], st, -a) < 0.0f;
    mag += __builtin_fmaf(ce[1], st, -a) <= 0.0f;
    mag += __builtin_fmaf(ce[2], st, -a) < 0.0f;
    mag += __builtin_fmaf(ce[3], st, -a) <= 0.0f;
    mag += __builtin_fmaf(ce[4], st, -a) < 0.0f;
    mag += __builtin_fmaf(ce[5], st, -a) <= 0.0f;
    mag += __builtin_fmaf(ce[6], st, -a) < 0.0f;
    return mag;
}

__device__ __forceinline__ uint32_t e2m1_mag_f64(float a, const float (&ce)[7], float st) {
    const double d = (double)a, s = (double)st;
    uint32_t mag = 0;
    mag += (double)ce[0] * s < d;
    mag += (double)ce[1] * s <= d;
    mag += (double)ce[2] * s < d;
    mag += (double)ce[3] * s <= d;
    mag += (double)ce[4] * s < d;
    mag += (double)ce[5] * s <= d;
    mag += (double)ce[6] * s < d;
    return mag;
}

// Stochastic rounding of |w| (a) in a block of scale S = e * s_t: between the
// neighbouring grid points lo <= a / S < hi, up with probability
// (a / S - lo) / (hi - lo): up <=> u (hi - lo) S < a - lo S, where u is the
// element's 24-bit uniform.  Exact in double: S has at most 28 significant
// bits, (hi - lo) is a power of two, and a - lo S is exact (lo S <= a < 2 lo S
// when lo > 0).  Values at or above 6 S take 6.
__device__ __forceinline__ uint32_t e2m1_mag_sr(float a, float e, float st, uint32_t u24) {
    const double S = (double)e * (double)st, d = (double)a;
    constexpr double g[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    uint32_t lo = 0;
#pragma unroll
    for (int i = 1; i < 8; ++i) lo += g[i] * S <= d;
    if (lo == 7) return 7;
    double glo = 0.0, gap = 0.5;
#pragma unroll
    for (int i = 1; i < 7; ++i)
        if (lo == (uint32_t)i) {
            glo = g[i];
            gap = g[i + 1] - g[i];
        }
    const double u = (double)u24 * 0x1p-24;
    return lo + (u * (gap * S) < d - glo * S ? 1u : 0u);
}

struct EncodeParams {
    const uint16_t *w;
    int64_t n, k, ldw;
    uint8_t *packed;
    uint8_t *scales;
    float *tensor_scale_out;
    const float *tensor_scale_in;
    const uint32_t *partial;
    int num_partials;
    uint32_t flags;
    uint64_t seed;  // SR: the stochastic-rounding stream
};

// SR: stochastic element rounding; the uniform of element e (row-major index
// row * k + col) is the top 24 bits of word e % 4 of Philox4x64-10 with key
// (seed, 0) and counter (e / 4, 0, 1, 0).
// s_t admits the fast element path: in range for the float-float quotient,
// and more than 8 significant bits (no BF16 value is an exact midpoint)
__device__ __forceinline__ bool fast_path_scale(float st) {
    if (!(st >= 0x1p-80f && st <= 0x1p80f)) return false;
    const uint32_t sig = (__float_as_uint(st) & 0x7FFFFFu) | 0x800000u;  // normal: 24-bit significand
    return __builtin_ctz(sig) < 16;  // odd part of at least 9 bits
}

// q ~ f / (e s_t) as fl(f (r_hi + r_lo)): r_hi + r_lo ~ 1 / (e s_t), r_hi of
// 16 significant bits, so f r_hi is exact for a BF16 f
__device__ __forceinline__ float fast_quotient(float f, float rh, float rl) {
    return __builtin_fmaf(f, rl, f * rh);
}

// s is E2M1-grid aligned (a midpoint or grid value: low 21 mantissa bits
// zero) and non-zero: the hardware's tie rule might not be the exact
// decision, so the element is decided again by comparisons
__device__ __forceinline__ uint32_t fast_suspect(float s) {
    // lowest set bit of the bits of s at 21 .. 30 <=> low 21 bits zero and s
    // neither +0 (no bit) nor -0 (bit 31); a zero element gives a zero s
    return (uint32_t)__builtin_ffs((int)__float_as_uint(s)) - 22u <= 9u;
}

// byte SEL of `old` <- the codes of the two BF16 elements of `word` (low
// half -> low nibble); bits J and J + 1 of `suspect` flag their quotients
template <int SEL, int J>
__device__ __forceinline__ uint32_t fast_pair(uint32_t old, uint32_t word, float rh, float rl, uint32_t &suspect) {
    const float f0 = __uint_as_float(word << 16), f1 = __uint_as_float(word & 0xFFFF0000u);
    const float s0 = fast_quotient(f0, rh, rl), s1 = fast_quotient(f1, rh, rl);
    suspect |= fast_suspect(s0) << J | fast_suspect(s1) << (J + 1);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, s0, s1, 1.0f, SEL);
}

// the 32-bit code word of elements J .. J + 7 (4 BF16 words)
template <int J>
__device__ __forceinline__ uint32_t fast_codes4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, float rh,
                                                float rl, uint32_t &suspect) {
    uint32_t c = fast_pair<0, J>(0u, w0, rh, rl, suspect);
    c = fast_pair<1, J + 2>(c, w1, rh, rl, suspect);
    c = fast_pair<2, J + 4>(c, w2, rh, rl, suspect);
    return fast_pair<3, J + 6>(c, w3, rh, rl, suspect);
}

template <bool SR>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeParams p) {
    __shared__ float s_st;
    __shared__ double s_inv_st;
    __shared__ double s_inv_e[128];  // 1 / E4M3(c), c = 1 .. 126
    if (!SR && threadIdx.x < 128) s_inv_e[threadIdx.x] = e4m3_inverse((int)threadIdx.x);
    // the partial maxima: every thread loads its share at once (at most
    // kAmaxMaxBlocks / kThreads), the waves' maxima meet in LDS
    __shared__ uint32_t s_red[kThreads / kWave];
    if (!p.tensor_scale_in) {
        constexpr int kPer = kAmaxMaxBlocks / kThreads;
        uint32_t v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = threadIdx.x + u * kThreads;
            v[u] = i < p.num_partials ? p.partial[i] : 0u;
        }
        uint32_t m = v[0];
#pragma unroll
        for (int u = 1; u < kPer; ++u) m = max(m, v[u]);
        m = wave_max(m);
        if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = m;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        float st;
        if (p.tensor_scale_in) {
            st = *p.tensor_scale_in;
            if (!(st > 0.0f && st < INFINITY)) st = __builtin_nanf("");
        } else {
            uint32_t m = s_red[0];
#pragma unroll
            for (int w = 1; w < kThreads / kWave; ++w) m = max(m, s_red[w]);
            if (m >= 0x7F80u) st = __builtin_nanf("");
            else if (m == 0) st = 1.0f;
            else st = (float)((double)__uint_as_float(m << 16) / 2688.0);
        }
        s_st = st;
        s_inv_st = 1.0 / (double)st;
        if (blockIdx.x == 0) *p.tensor_scale_out = st;
    }
    __syncthreads();
    const float st = s_st;
    if (!(st > 0.0f && st < INFINITY)) return;  // non-finite input: outputs unspecified
    const bool fma_exact = st >= 0x1p-90f;
    const bool rne = (p.flags & 1u) != 0;
    const bool fast = !SR && fast_path_scale(st);
    const double inv_st = s_inv_st;
    const float inv6st = (float)(inv_st / 6.0);  // scale-code guesses
    const int64_t bpr = p.k >> 4;
    const int64_t total = p.n * bpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < total; b += stride) {
        const uint16_t *src;
        if (p.ldw == p.k) {
            src = p.w + b * 16;
        } else {
            const int64_t row = b / bpr;
            src = p.w + row * p.ldw + (b - row * bpr) * 16;
        }
        const uint4 v0 = reinterpret_cast<const uint4 *>(src)[0];
        const uint4 v1 = reinterpret_cast<const uint4 *>(src)[1];
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const uint32_t am = absmax16(v0, v1);
        const float amax_b = __uint_as_float(am << 16);
        int sb;
        if (fast)  // (uniform)
            sb = rne ? scale_code_rne_f32(amax_b, st, inv6st) : scale_code_round_up_f32(amax_b, st, inv6st);
        else
            sb = rne ? scale_code_rne(amax_b, st, inv6st) : scale_code_round_up(amax_b, st, inv6st);
        const float e = e4m3_value(sb);
        uint32_t lo = 0, hi = 0;
        if (SR && e != 0.0f) {
            const int64_t row = b / bpr;
            const uint64_t e0 = (uint64_t)(row * p.k + (b - row * bpr) * 16);  // a multiple of 16
            uint32_t u[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const U64x4 r = philox4x64_10(e0 / 4 + q, 0, 1, 0, p.seed, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) u[4 * q + i] = (uint32_t)(r.v[i] >> 40);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t bits = (j & 1) ? (wd[j >> 1] >> 16) : (wd[j >> 1] & 0xFFFFu);
                const float a = __uint_as_float((bits & 0x7FFFu) << 16);
                const uint32_t code = e2m1_mag_sr(a, e, st, u[j]) | ((bits >> 12) & 8u);
                if (j < 8) lo |= code << (4 * j);
                else hi |= code << (4 * (j - 8));
            }
        } else if (e != 0.0f) {
            bool done = false;
            if (fast && am < 0x7F80u) {  // (finite block)
                const double r = inv_st * s_inv_e[sb];
                const float rh = __uint_as_float(__float_as_uint((float)r) & 0xFFFFFF00u);  // 16 significant bits
                const float rl = (float)(r - (double)rh);
                if (amax_b * rh < 0x1p100f) {
                    uint32_t suspect = 0;  // bit j: element j's quotient fell on an aligned value
                    lo = fast_codes4<0>(wd[0], wd[1], wd[2], wd[3], rh, rl, suspect);
                    hi = fast_codes4<8>(wd[4], wd[5], wd[6], wd[7], rh, rl, suspect);
                    if (suspect) {
                        // those elements again by the comparisons (the quotient
                        // lies within 2^-24 of a midpoint whenever |w| / (e s_t)
                        // is a short binary fraction times fl(s_t) / s_t's exact
                        // value, which s_t = fl(amax / 2688) makes common)
                        const float ce[7] = {0.25f * e, 0.75f * e, 1.25f * e, 1.75f * e,
                                             2.5f * e,  3.5f * e,  5.0f * e};
                        do {
                            const int j = __builtin_ctz(suspect);
                            suspect &= suspect - 1;
                            const int wi = j >> 1;
                            const uint32_t word = wi == 0 ? wd[0] : wi == 1 ? wd[1] : wi == 2 ? wd[2] : wi == 3 ? wd[3]
                                                : wi == 4 ? wd[4] : wi == 5 ? wd[5] : wi == 6 ? wd[6] : wd[7];
                            const uint32_t bits = (j & 1) ? (word >> 16) : (word & 0xFFFFu);
                            const float a = __uint_as_float((bits & 0x7FFFu) << 16);
                            const uint32_t code = e2m1_mag_f32(a, ce, st) | ((bits >> 12) & 8u);
                            const int sh = 4 * (j & 7);
                            if (j < 8) lo = (lo & ~(0xFu << sh)) | code << sh;
                            else hi = (hi & ~(0xFu << sh)) | code << sh;
                        } while (suspect);
                    }
                    done = true;
                }
            }
            if (!done) {
                lo = hi = 0;
                const float ce[7] = {0.25f * e, 0.75f * e, 1.25f * e, 1.75f * e,
                                     2.5f * e,  3.5f * e,  5.0f * e};
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t bits = (j & 1) ? (wd[j >> 1] >> 16) : (wd[j >> 1] & 0xFFFFu);
                    const float a = __uint_as_float((bits & 0x7FFFu) << 16);
                    const uint32_t mag = fma_exact ? e2m1_mag_f32(a, ce, st) : e2m1_mag_f64(a, ce, st);
                    const uint32_t code = mag | ((bits >> 12) & 8u);
                    if (j < 8) lo |= code << (4 * j);
                    else hi |= code << (4 * (j - 8));
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t bits = (j & 1) ? (wd[j >> 1] >> 16) : (wd[j >> 1] & 0xFFFFu);
                const uint32_t code = (bits >> 12) & 8u;
                if (j < 8) lo |= code << (4 * j);
                else hi |= code << (4 * (j - 8));
            }
        }
        reinterpret_cast<uint2 *>(p.packed)[b] = make_uint2(lo, hi);
        p.scales[b] = (uint8_t)sb;
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

}  // namespace

size_t quantize_workspace_bytes(int64_t, int64_t) { return kAmaxMaxBlocks * sizeof(uint32_t); }

hipError_t launch_nvfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                                 uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                 const float *tensor_scale_in, uint32_t flags, void *workspace,
                                 hipStream_t stream, bool stochastic, uint64_t seed) {
    uint32_t *partial = static_cast<uint32_t *>(workspace);
    int g1 = 0;
    if (!tensor_scale_in) {
        const int64_t vecs = n * (k >> 3);
        const int64_t want = ldw == k ? (vecs + kThreads * kAmaxLoads - 1) / (kThreads * kAmaxLoads) : n;
        g1 = (int)(want < kAmaxBlocks ? (want < 1 ? 1 : want) : kAmaxBlocks);
        hipLaunchKernelGGL(amax_kernel, dim3(g1), dim3(kThreads), 0, stream, w, n, k, ldw, partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    EncodeParams p{w, n, k, ldw, packed, scales, tensor_scale, tensor_scale_in, partial, g1, flags, seed};
    const int64_t blocks16 = n * (k >> 4);
    const int64_t want = (blocks16 + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)num_cus() * 16;
    const int g2 = (int)(want < cap ? want : cap);
    if (stochastic)
        hipLaunchKernelGGL(encode_kernel<true>, dim3(g2), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(encode_kernel<false>, dim3(g2), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// ---- MXFP4 (OCP MX v1.0): 32-element blocks along K, E8M0 scale ----
// One thread per block: 64 B in, 16 B of codes and 1 scale byte out.  The
// scale is 2^(floor(log2 amax) - 2) (E8M0 byte clamped to [0, 254], 0 for an
// all-zero block, 0xFF for a block with Inf/NaN and zero codes); |w| / X is
// exact (X a power of two) and rounds to nearest-even on the E2M1 grid with
// the midpoint comparisons of the NVFP4 encoder, saturating at 6.
__global__ __launch_bounds__(kThreads) void mxfp4_encode_kernel(const uint16_t *__restrict__ w, int64_t n,
                                                                int64_t k, int64_t ldw, uint8_t *__restrict__ packed,
                                                                uint8_t *__restrict__ scales) {
    const int64_t bpr = k >> 5, total = n * bpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < total; b += stride) {
        const int64_t row = b / bpr;
        const uint4 *src = reinterpret_cast<const uint4 *>(w + row * ldw + (b - row * bpr) * 32);
        const uint4 v[4] = {src[0], src[1], src[2], src[3]};
        const uint32_t am = max(max(absmax_vec(v[0]), absmax_vec(v[1])), max(absmax_vec(v[2]), absmax_vec(v[3])));
        uint4 out = make_uint4(0, 0, 0, 0);
        uint32_t code = 0;
        if (am >= 0x7F80u) {
            code = 0xFF;
        } else if (am != 0) {
            const int ef = (int)(am >> 7);  // BF16 exponent field
            const int fl = ef > 0 ? ef - 127 : (31 - __builtin_clz(am & 0x7Fu)) - 133;  // floor(log2 amax)
            int c = fl - 2 + 127;
            c = c < 0 ? 0 : (c > 254 ? 254 : c);
            code = (uint32_t)c;
            // 1 / X = 2^(127 - c), a normal float for c <= 253 (BF16 amax gives c <= 252)
            const float r = c <= 253 ? __uint_as_float((uint32_t)(254 - c) << 23) : 0x1p-127f;
            uint32_t wd[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wd[4 * q] = v[q].x;
                wd[4 * q + 1] = v[q].y;
                wd[4 * q + 2] = v[q].z;
                wd[4 * q + 3] = v[q].w;
            }
            uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t bits = (j & 1) ? (wd[j >> 1] >> 16) : (wd[j >> 1] & 0xFFFFu);
                const float a = __uint_as_float((bits & 0x7FFFu) << 16) * r;  // |w| / X, exact
                uint32_t mag = 0;
                mag += a > 0.25f;
                mag += a >= 0.75f;
                mag += a > 1.25f;
                mag += a >= 1.75f;
                mag += a > 2.5f;
                mag += a >= 3.5f;
                mag += a > 5.0f;
                o[j >> 3] |= (mag | ((bits >> 12) & 8u)) << (4 * (j & 7));
            }
            out = make_uint4(o[0], o[1], o[2], o[3]);
        } else {  // all zero: signed zero codes
            uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint4 q = v[j >> 3];
                const uint32_t word = ((j >> 1) & 3) == 0 ? q.x : ((j >> 1) & 3) == 1 ? q.y : ((j >> 1) & 3) == 2 ? q.z : q.w;
                const uint32_t bits = (j & 1) ? (word >> 16) : (word & 0xFFFFu);
                o[j >> 3] |= ((bits >> 12) & 8u) << (4 * (j & 7));
            }
            out = make_uint4(o[0], o[1], o[2], o[3]);
        }
        reinterpret_cast<uint4 *>(packed + row * (k >> 1))[b - row * bpr] = out;
        scales[b] = (uint8_t)code;
    }
}

hipError_t launch_mxfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw, uint8_t *packed,
                                 uint8_t *scales, hipStream_t stream) {
    const int64_t blocks32 = n * (k >> 5);
    const int64_t want = (blocks32 + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)num_cus() * 16;
    const int g = (int)(want < cap ? (want < 1 ? 1 : want) : cap);
    hipLaunchKernelGGL(mxfp4_encode_kernel, dim3(g), dim3(kThreads), 0, stream, w, n, k, ldw, packed, scales);
    return hipGetLastError();
}

namespace {

// ---- NVFP4 -> BF16 ----
// What an unfused update-phase forward needs before a BF16 GEMM.  One thread
// per 16-element block: 8 code bytes and 1 scale byte in, 32 B out, coalesced
// across the wave.  e2m1 * e4m3 is exact in float (<= 6 significant bits) and
// its product with s_t exact in double (<= 30 bits); that value is rounded
// once to BF16: to float with round-to-odd (24 bits >= 8 + 2 keeps the later
// rounding correct), then to BF16 nearest-even.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
    if (v != v) return 0x7FC0;
    float f = (float)v;  // nearest-even
    uint32_t b = __float_as_uint(f);
    if ((double)f != v && (b & 0x7F800000u) != 0x7F800000u && (b & 1u) == 0)
        b = fabs(v) > fabs((double)f) ? b + 1u : b - 1u;  // the odd neighbour on v's side
    return f32_to_bf16_bits(__uint_as_float(b));
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *__restrict__ packed,
                                                           const uint8_t *__restrict__ scales,
                                                           const float *__restrict__ tensor_scale, int64_t n,
                                                           int64_t k, uint16_t *__restrict__ out, int64_t ldo) {
    const int64_t bpr = k >> 4, total = n * bpr;
    const double st = (double)*tensor_scale;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < total; b += stride) {
        const int64_t row = b / bpr, col = b - row * bpr;
        const uint2 c = *reinterpret_cast<const uint2 *>(packed + row * (k >> 1) + col * 8);
        const double s = (double)QERL_E4M3_F32(scales[b], 0) * st;  // exact: 4 x 24 bits
        float e[16];
        const auto p0 = QERL_FP4_PAIR_F32(c.x, 0), p1 = QERL_FP4_PAIR_F32(c.x, 1);
        const auto p2 = QERL_FP4_PAIR_F32(c.x, 2), p3 = QERL_FP4_PAIR_F32(c.x, 3);
        const auto p4 = QERL_FP4_PAIR_F32(c.y, 0), p5 = QERL_FP4_PAIR_F32(c.y, 1);
        const auto p6 = QERL_FP4_PAIR_F32(c.y, 2), p7 = QERL_FP4_PAIR_F32(c.y, 3);
        e[0] = p0[0], e[1] = p0[1], e[2] = p1[0], e[3] = p1[1], e[4] = p2[0], e[5] = p2[1], e[6] = p3[0];
        e[7] = p3[1], e[8] = p4[0], e[9] = p4[1], e[10] = p5[0], e[11] = p5[1], e[12] = p6[0], e[13] = p6[1];
        e[14] = p7[0], e[15] = p7[1];
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = (uint32_t)f64_to_bf16_rne((double)e[2 * i] * s) |
                   ((uint32_t)f64_to_bf16_rne((double)e[2 * i + 1] * s) << 16);
        uint4 *dst = reinterpret_cast<uint4 *>(out + row * ldo + col * 16);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

}  // namespace

hipError_t launch_nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                   int64_t n, int64_t k, uint16_t *out, int64_t ldo, hipStream_t stream) {
    const int64_t blocks16 = n * (k >> 4);
    const int64_t want = (blocks16 + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)num_cus() * 16;
    const int g = (int)(want < cap ? (want < 1 ? 1 : want) : cap);
    hipLaunchKernelGGL(dequant_kernel, dim3(g), dim3(kThreads), 0, stream, packed, scales, tensor_scale, n, k, out,
                       ldo);
    return hipGetLastError();
}

}  // namespace qerl
