/*
 * qerl_oracle.c -- plain CPU oracle for the NVFP4 weight-only (W4A16) + LoRA
 * linear layer and the adaptive-quantization-noise (AQN) RMSNorm of QeRL.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; the two meet only through seeded inputs.
 *
 * Everything here is the plain definition, evaluated in fp64 (exact where
 * the text says so), with no blocking, fusion or reordering beyond what the
 * definition states.  Worker threads only split independent output rows.
 *
 * Sources (page title -- section):
 *  [BoA-NVFP4]  "QeRL: NVFP4-Quantized Reinforcement Learning -- Redefining
 *               Efficiency in AI Training and Inference", section "NVFP4:
 *               NVIDIA's FP4 Format" (block size 16; one FP8 E4M3 scale per
 *               block plus an FP32 tensor scale; cuDNN block scaling: scale =
 *               quantize_round_up(amax(vals)/vmax_otype), value =
 *               round_to_even(vals/scale)).
 *  [BoA-LoRA]   same page, section "LoRA (Low-Rank Adaptation)" (W + dW with
 *               a rank-r product of two small matrices).
 *  [BoA-Impl]   same page, "Implementation and Practical Details" (weight-only
 *               quantization; NVFP4 + LoRA summation in the kernel).
 *  [README-Ack] "NVlabs/QeRL" README mirror, "Acknowledgement" (the rollout
 *               kernel multiplies NVFP4 weights by BF16 activations).
 *  [README-Hint] same page, "Hints for QeRL training", item 3 (the noise
 *               knobs sigma_start, sigma_end, num_stages).
 *  [1kp-Sum]    "Paper 2510.11696 -- QeRL: Beyond Efficiency", "In brief /
 *               Summary" (AQN: channel-wise Gaussian noise injected through
 *               the normalization layer, exponential decay schedule).
 *  [Dfc-Test]   "QERL: NVFP4-intensive learning (RL) brings 32B LLM training
 *               to H100", section on findings (the noise lives in the norm's
 *               scale parameters, so no extra weights are needed).
 *  [OCP-MX]     OCP Microscaling Formats (MX) v1.0, element formats FP4 E2M1
 *               and FP8 E4M3 (the "FN" variant: no infinities, NaN = S.1111.111).
 *  [Philox]     Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *               as 1, 2, 3", SC'11 -- Philox4x64 with 10 rounds.
 *  [BoxMuller]  Box & Muller, "A Note on the Generation of Random Normal
 *               Deviates", Ann. Math. Stat. 29 (1958).
 *
 * Readings where the pages are silent are listed next to the code they
 * shape; each is also listed in the design notes of the repository.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* worker threads: split [0, count) into contiguous chunks                  */
/* ------------------------------------------------------------------------ */
typedef void (*range_fn)(void *ctx, int64_t begin, int64_t end);
typedef struct { range_fn fn; void *ctx; int64_t begin, end; } range_job;

static void *range_trampoline(void *p) {
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static int resolve_threads(int threads) {
    if (threads > 0) return threads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static void parallel_range(int threads, int64_t count, range_fn fn, void *ctx) {
    threads = resolve_threads(threads);
    if (threads > 256) threads = 256;
    if (count <= 0) return;
    if ((int64_t)threads > count) threads = (int)count;
    if (threads <= 1) { fn(ctx, 0, count); return; }
    pthread_t tid[256];
    range_job job[256];
    int started[256];
    for (int t = 0; t < threads; ++t) {
        job[t].fn = fn;
        job[t].ctx = ctx;
        job[t].begin = count * t / threads;
        job[t].end = count * (t + 1) / threads;
        started[t] = pthread_create(&tid[t], NULL, range_trampoline, &job[t]) == 0;
        if (!started[t]) range_trampoline(&job[t]);
    }
    for (int t = 0; t < threads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* element codecs                                                            */
/* ------------------------------------------------------------------------ */

/* BF16 is the upper half of an IEEE binary32; decoding is exact. */
double oracle_bf16_decode(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP4 E2M1 [OCP-MX]: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no Inf/NaN.
 * Exponent field 0 is subnormal (0 or 0.5); otherwise 2^(e-1) * (1 + m/2). */
double oracle_e2m1_decode(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3 "FN" [OCP-MX]: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; max 448. */
double oracle_e4m3_decode(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* E4M3 block-scale rounding                                                 */
/* ------------------------------------------------------------------------ */
/* The non-negative, non-NaN E4M3 codes 0x00..0x7E are increasing in value.
 * Each decision below is a comparison of exact products in fp64: an E4M3
 * value (4 significant bits) times 6 (2 bits) times the FP32 tensor scale
 * (24 bits) has at most 30 significant bits, so it is exact in a double.   */

#define E4M3_MAX_CODE 0x7E /* 448 */

/* least code v with decode(v) * 6 * s_t >= amax_b ("quantize_round_up" of
 * amax/vmax in [BoA-NVFP4]); saturates at 448 when no code is large enough */
static int e4m3_round_up_code(double amax_b, double s_t) {
    if (448.0 * 6.0 * s_t < amax_b) return E4M3_MAX_CODE;
    int lo = 0, hi = E4M3_MAX_CODE; /* invariant: answer in [lo, hi] */
    while (lo < hi) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode(mid) * 6.0 * s_t >= amax_b) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

/* nearest E4M3 value to t* = amax_b / (6 s_t); ties to the even code;
 * saturates at 448 (round-to-nearest-even option for the block scale) */
static int e4m3_rne_code(double amax_b, double s_t) {
    int hi = e4m3_round_up_code(amax_b, s_t);
    double vhi = oracle_e4m3_decode(hi);
    if (vhi * 6.0 * s_t < amax_b) return E4M3_MAX_CODE;   /* saturated */
    if (hi == 0 || vhi * 6.0 * s_t == amax_b) return hi;  /* exact hit */
    int lo = hi - 1;
    double vlo = oracle_e4m3_decode(lo);
    /* t* - vlo  vs  vhi - t*   <=>   2*amax_b  vs  (vlo + vhi) * 6 * s_t */
    double two_amax = 2.0 * amax_b;
    double mid6s = (vlo + vhi) * 6.0 * s_t;
    if (two_amax < mid6s) return lo;
    if (two_amax > mid6s) return hi;
    return (lo & 1) ? hi : lo;
}

/* exposed for the codec tests: the scale byte chosen for a block with
 * amax amax_b under tensor scale s_t (flags bit 0: nearest-even instead of
 * round-up) */
int oracle_e4m3_block_scale_code(double amax_b, float s_t, unsigned flags) {
    return (flags & 1u) ? e4m3_rne_code(amax_b, (double)s_t) : e4m3_round_up_code(amax_b, (double)s_t);
}

/* ------------------------------------------------------------------------ */
/* E2M1 element rounding                                                     */
/* ------------------------------------------------------------------------ */
/* Magnitude code of round_to_even(|w| / S) on the E2M1 grid
 * {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6.  The midpoints between
 * neighbours are .25 .75 1.25 1.75 2.5 3.5 5; at a midpoint the neighbour
 * whose code is even (mantissa bit 0) wins, so the lower neighbour wins at
 * .25 1.25 2.5 5 and the upper one at .75 1.75 3.5.  Values above 6 clamp.
 * Each comparison |w| vs c*S is exact in fp64 (c has at most 3 significant
 * bits, S = E4M3 * s_t at most 28).                                        */
static int e2m1_rne_mag(double aw, double S) {
    if (S == 0.0) return 0;
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    static const int ties_up[7] = {0, 1, 0, 1, 0, 1, 0};
    int mag = 0;
    for (int i = 0; i < 7; ++i) {
        double t = mid[i] * S;
        if (aw > t || (ties_up[i] && aw == t)) mag = i + 1;
    }
    return mag;
}

/* exposed for the codec tests: full 4-bit code of element w in a block whose
 * scale (E4M3 value times tensor scale) is S */
int oracle_e2m1_code(double w, double S) {
    return ((signbit(w) ? 1 : 0) << 3) | e2m1_rne_mag(fabs(w), S);
}

/* ------------------------------------------------------------------------ */
/* BF16 -> NVFP4 quantizer                                                   */
/* ------------------------------------------------------------------------ */
/* Layout: packed[n, k/2] with element 2j in the low nibble of byte j and
 * element 2j+1 in the high nibble; scales[n, k/16] one E4M3 byte per block of
 * 16 consecutive elements along K; *s_t_out the FP32 tensor scale.  The
 * dequantized weight is e2m1(code) * e4m3(scale byte) * s_t.
 *
 * Reading (pages silent): the tensor scale maps the largest block scale to
 * the top of the E4M3 range, s_t = fl32(amax_t / (6 * 448)).  amax_t == 0
 * gives s_t = 1.  A non-finite weight gives s_t = NaN and the other outputs
 * are unspecified (left untouched here).                                    */

#define ORACLE_SCALE_RNE 1u

typedef struct {
    const uint16_t *w; int64_t n, k, ldw;
    uint8_t *packed, *scales;
    double s_t; unsigned flags;
    int stochastic; uint64_t seed;   /* element rounding: stochastic (see below) */
} quant_ctx;

static double sr_uniform(uint64_t seed, int64_t e);
static int e2m1_sr_mag(double aw, double S, double u);
void oracle_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]);

static void quant_rows(void *p, int64_t r0, int64_t r1) {
    quant_ctx *c = (quant_ctx *)p;
    const int64_t nb = c->k / 16;
    for (int64_t row = r0; row < r1; ++row) {
        const uint16_t *wr = c->w + row * c->ldw;
        for (int64_t b = 0; b < nb; ++b) {
            double amax_b = 0.0;
            for (int i = 0; i < 16; ++i) {
                double a = fabs(oracle_bf16_decode(wr[b * 16 + i]));
                if (a > amax_b) amax_b = a;
            }
            int sb = (c->flags & ORACLE_SCALE_RNE) ? e4m3_rne_code(amax_b, c->s_t)
                                                   : e4m3_round_up_code(amax_b, c->s_t);
            c->scales[row * nb + b] = (uint8_t)sb;
            double S = oracle_e4m3_decode(sb) * c->s_t;   /* exact */
            for (int i = 0; i < 16; i += 2) {
                int code[2];
                for (int h = 0; h < 2; ++h) {
                    uint16_t bits = wr[b * 16 + i + h];
                    double v = oracle_bf16_decode(bits);
                    int sign = (bits >> 15) & 1;              /* signbit(w) */
                    int mag = c->stochastic
                                  ? e2m1_sr_mag(fabs(v), S, sr_uniform(c->seed, row * c->k + b * 16 + i + h))
                                  : e2m1_rne_mag(fabs(v), S);
                    code[h] = (sign << 3) | mag;
                }
                c->packed[row * (c->k / 2) + (b * 16 + i) / 2] =
                    (uint8_t)(code[0] | (code[1] << 4));
            }
        }
    }
}

/* returns 0 on success, -1 on bad arguments */
static int quantize_impl(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                         const float *s_t_in, unsigned flags, int stochastic, uint64_t seed,
                         uint8_t *packed, uint8_t *scales, float *s_t_out, int threads) {
    if (!w || !packed || !scales || !s_t_out || n <= 0 || k <= 0 || k % 16 || ldw < k)
        return -1;
    float s_t;
    if (s_t_in) {
        s_t = *s_t_in;
        if (!(s_t > 0.0f) || isinf(s_t)) { *s_t_out = NAN; return 0; }
    } else {
        /* tensor amax; any non-finite element poisons the tensor scale */
        float amax = 0.0f;
        for (int64_t r = 0; r < n; ++r)
            for (int64_t i = 0; i < k; ++i) {
                double v = oracle_bf16_decode(w[r * ldw + i]);
                if (!isfinite(v)) { *s_t_out = NAN; return 0; }
                if (fabs(v) > amax) amax = (float)fabs(v);
            }
        /* one IEEE binary32 division, correctly rounded */
        s_t = (amax == 0.0f) ? 1.0f : amax / 2688.0f;
    }
    *s_t_out = s_t;
    quant_ctx c = {w, n, k, ldw, packed, scales, (double)s_t, flags, stochastic, seed};
    parallel_range(threads, n, quant_rows, &c);
    return 0;
}

int oracle_nvfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                          const float *s_t_in, unsigned flags,
                          uint8_t *packed, uint8_t *scales, float *s_t_out,
                          int threads) {
    return quantize_impl(w, n, k, ldw, s_t_in, flags, 0, 0, packed, scales, s_t_out, threads);
}

/* ------------------------------------------------------------------------ */
/* Stochastic element rounding ([BoA-NVFP4]: the FP4 training work it cites   */
/* pairs 16-value blocks with stochastic rounding)                           */
/* ------------------------------------------------------------------------ */
/* Reading (self-defined stream, the pages name the method only): with
 * lo <= |w|/S < hi the neighbouring E2M1 grid points, the element rounds up to
 * hi with probability (|w|/S - lo) / (hi - lo), else down to lo, so that the
 * expected dequantized value is w.  Values at or above 6 S saturate to 6; grid
 * values stay.  The uniform of element e (row-major index row * k + col) is
 * u = (r >> 40) * 2^-24 for word e % 4 of Philox4x64-10 with key (seed, 0)
 * and counter (e / 4, 0, 1, 0).  Rounding up <=> u * (hi - lo) * S < |w| - lo * S,
 * evaluated exactly in fp64: (hi - lo) is a power of two, u has 24
 * significant bits and S = E4M3 * s_t at most 28; |w| - lo * S is exact by
 * Sterbenz's lemma (lo * S <= |w| < hi * S <= 2 lo * S when lo > 0).        */
static double sr_uniform(uint64_t seed, int64_t e) {
    const uint64_t ctr[4] = {(uint64_t)e / 4, 0, 1, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t r[4];
    oracle_philox4x64_10(ctr, key, r);
    return (double)(r[e % 4] >> 40) * 0x1p-24;
}

static int e2m1_sr_mag(double aw, double S, double u) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (S == 0.0) return 0;
    int lo = 0;
    for (int i = 1; i < 8; ++i)
        if (grid[i] * S <= aw) lo = i;
    if (lo == 7) return 7;
    return u * (grid[lo + 1] - grid[lo]) * S < aw - grid[lo] * S ? lo + 1 : lo;
}

/* exposed for the tests: the uniform element e draws, and the magnitude code
 * of |w| in a block of scale S given that uniform */
double oracle_sr_uniform(uint64_t seed, int64_t e) { return sr_uniform(seed, e); }
int oracle_e2m1_sr_mag(double aw, double S, double u) { return e2m1_sr_mag(aw, S, u); }

int oracle_nvfp4_quantize_sr(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                             const float *s_t_in, unsigned flags, uint64_t seed,
                             uint8_t *packed, uint8_t *scales, float *s_t_out, int threads) {
    return quantize_impl(w, n, k, ldw, s_t_in, flags, 1, seed, packed, scales, s_t_out, threads);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 (OCP MX v1.0): blocks of 32 along K, one E8M0 scale each             */
/* ------------------------------------------------------------------------ */
/* [BoA-NVFP4] contrasts NVFP4's 16-value blocks with MXFP4's 32.
 * [OCP-MX] conversion: X = 2^(floor(log2(amax_b)) - emax) with emax = 2 for
 * E2M1, stored as the E8M0 byte floor(log2(amax_b)) - 2 + 127 (clamped to
 * [0, 254]; an all-zero block gets byte 0); elements round to nearest-even on
 * the E2M1 grid of |w| / X, saturating at 6, sign = signbit(w).  A block with
 * a non-finite element gets the NaN byte 0xFF and unspecified elements.
 * Layout as NVFP4: packed[n, k/2] (even element in the low nibble),
 * scales[n, k/32].                                                          */
int oracle_mxfp4_quantize(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                          uint8_t *packed, uint8_t *scales) {
    if (!w || !packed || !scales || n <= 0 || k <= 0 || k % 32 || ldw < k) return -1;
    for (int64_t row = 0; row < n; ++row) {
        const uint16_t *wr = w + row * ldw;
        for (int64_t b = 0; b < k / 32; ++b) {
            double amax = 0.0;
            int finite = 1;
            for (int i = 0; i < 32; ++i) {
                double v = oracle_bf16_decode(wr[b * 32 + i]);
                if (!isfinite(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            if (!finite) { scales[row * (k / 32) + b] = 0xFF; continue; }
            int code = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1 */
                code = (ex - 1) - 2 + 127;
                if (code < 0) code = 0;
                if (code > 254) code = 254;
            }
            scales[row * (k / 32) + b] = (uint8_t)code;
            double X = ldexp(1.0, code - 127);
            for (int i = 0; i < 32; i += 2) {
                int c2[2];
                for (int h = 0; h < 2; ++h) {
                    uint16_t bits = wr[b * 32 + i + h];
                    c2[h] = (((bits >> 15) & 1) << 3) | e2m1_rne_mag(fabs(oracle_bf16_decode(bits)), X);
                }
                packed[row * (k / 2) + (b * 32 + i) / 2] = (uint8_t)(c2[0] | (c2[1] << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 -> BF16 dequantization                                              */
/* ------------------------------------------------------------------------ */
/* The value a stored weight stands for is e2m1(code) * e4m3(block scale) *
 * s_t (bitsofall page, "NVFP4: NVIDIA's FP4 Format": a 4-bit element, one
 * E4M3 scale per 16 values, an FP32 tensor scale).  The update phase of QeRL
 * turns the weights back into 16-bit values before its GEMMs (README "Hints
 * for QeRL training", item 2; bitsofall page, "Workflow: Rollout, Update,
 * Quantization"); the BF16 result is that exact product (fp64:
 * 6 significant bits times 24) rounded to the nearest BF16 value, ties to the
 * even code.                                                               */

/* The BF16 value of code c (0 <= c <= 0x7F80, sign clear); 0x7F80 counts as
 * 2^128, the next step past the largest finite value, so that a magnitude
 * from half a step above that value up rounds to infinity as IEEE 754 says. */
static double bf16_mag(uint16_t c) {
    return c == 0x7F80 ? ldexp(1.0, 128) : oracle_bf16_decode(c);
}

/* Nearest BF16 to v, ties to the even code: the largest magnitude code not
 * above |v| by bisection over the ordered codes, then the nearer of it and
 * its successor. */
uint16_t oracle_bf16_nearest_even(double v) {
    if (isnan(v)) return 0x7FC0;
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a >= bf16_mag(0x7F80)) return sign | 0x7F80;
    uint16_t lo = 0, hi = 0x7F80; /* bf16_mag(lo) <= a < bf16_mag(hi) */
    while (hi - lo > 1) {
        const uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (bf16_mag(mid) <= a) lo = mid; else hi = mid;
    }
    const double below = a - bf16_mag(lo), above = bf16_mag(hi) - a;
    uint16_t c;
    if (below < above) c = lo;
    else if (above < below) c = hi;
    else c = (lo & 1) ? hi : lo;
    return sign | c;
}

/* packed [n, k/2] (even element in the low nibble), scales [n, k/16], s_t ->
 * out_f64 [n, k] (exact values, may be NULL) and out_bf16 [n, k] (may be NULL). */
int oracle_nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, float s_t, int64_t n, int64_t k,
                            double *out_f64, uint16_t *out_bf16) {
    if (n < 0 || k < 0 || k % 16 != 0) return 1;
    for (int64_t row = 0; row < n; ++row)
        for (int64_t j = 0; j < k; ++j) {
            const uint8_t byte = packed[row * (k / 2) + j / 2];
            const int code = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
            const double v = oracle_e2m1_decode(code) * oracle_e4m3_decode(scales[row * (k / 16) + j / 16]) * (double)s_t;
            if (out_f64) out_f64[row * k + j] = v;
            if (out_bf16) out_bf16[row * k + j] = oracle_bf16_nearest_even(v);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* W4A16 + LoRA linear layer, fp64                                           */
/* ------------------------------------------------------------------------ */
/* y[m, n] = sum_k x[m,k] * what[n,k]  +  lora_scale * sum_j t[m,j] * B[n,j],
 * t[m, j] = sum_k x[m,k] * A[j,k],  what = e2m1 * e4m3 * s_t (exact in fp64).
 * x is [M, K] bf16 (row stride ldx) -- or fp64 for oracle_w4a16_lora_gemm_f64,
 * the same definition on activations given in fp64 (the output of a norm
 * before any rounding) --, A is [r, K] bf16, B is [N, r] bf16.
 * The layer has no bias.  Only the rows listed in rows[] (or all rows when
 * rows is NULL) are evaluated; y is [nrows, N] fp64.                        */

/* x[m, kk]: the fp64 activations when given, else the BF16 ones */
static double x_elem(const uint16_t *xb, const double *xd, int64_t ldx, int64_t m, int64_t kk) {
    return xd ? xd[m * ldx + kk] : oracle_bf16_decode(xb[m * ldx + kk]);
}

typedef struct {
    const uint16_t *x; const double *xd; int64_t k, ldx;
    const uint8_t *packed, *scales; double s_t; int64_t n;
    const uint16_t *b; int r; double lora_scale;
    const int64_t *rows; int64_t nrows;
    const double *t;      /* [nrows, r] */
    double *y;            /* [nrows, n] */
} gemm_ctx;

static void gemm_cols(void *p, int64_t n0, int64_t n1) {
    gemm_ctx *c = (gemm_ctx *)p;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)c->k);
    if (!wrow) return;
    for (int64_t n = n0; n < n1; ++n) {
        /* dequantize weight row n */
        for (int64_t kk = 0; kk < c->k; ++kk) {
            uint8_t byte = c->packed[n * (c->k / 2) + kk / 2];
            int code = (kk & 1) ? (byte >> 4) : (byte & 15);
            double sc = oracle_e4m3_decode(c->scales[n * (c->k / 16) + kk / 16]);
            wrow[kk] = oracle_e2m1_decode(code) * sc * c->s_t;
        }
        for (int64_t i = 0; i < c->nrows; ++i) {
            int64_t m = c->rows ? c->rows[i] : i;
            double acc = 0.0;
            for (int64_t kk = 0; kk < c->k; ++kk) acc += x_elem(c->x, c->xd, c->ldx, m, kk) * wrow[kk];
            double lora = 0.0;
            for (int j = 0; j < c->r; ++j)
                lora += c->t[i * c->r + j] * oracle_bf16_decode(c->b[n * c->r + j]);
            c->y[i * c->n + n] = acc + c->lora_scale * lora;
        }
    }
    free(wrow);
}

static int gemm_impl(const uint16_t *x, const double *xd, int64_t m, int64_t k, int64_t ldx,
                     const uint8_t *packed, const uint8_t *scales, float s_t, int64_t n,
                     const uint16_t *lora_a, const uint16_t *lora_b, int r, float lora_scale,
                     const int64_t *rows, int64_t nrows, double *y, int threads) {
    if ((!x && !xd) || !packed || !scales || !y || m <= 0 || n <= 0 || k <= 0 || k % 16 || ldx < k || r < 0)
        return -1;
    if (r > 0 && (!lora_a || !lora_b)) return -1;
    if (!rows) nrows = m;
    if (nrows <= 0) return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= m) return -1;
    /* LoRA down-projection t = x A^T for the requested rows */
    double *t = (double *)calloc((size_t)(nrows * (r > 0 ? r : 1)), sizeof(double));
    if (!t) return -2;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t mm = rows ? rows[i] : i;
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk)
                acc += x_elem(x, xd, ldx, mm, kk) * oracle_bf16_decode(lora_a[(int64_t)j * k + kk]);
            t[i * r + j] = acc;
        }
    }
    gemm_ctx c = {x, xd, k, ldx, packed, scales, (double)s_t, n, lora_b, r, (double)lora_scale,
                  rows, nrows, t, y};
    parallel_range(threads, n, gemm_cols, &c);
    free(t);
    return 0;
}

int oracle_w4a16_lora_gemm(const uint16_t *x, int64_t m, int64_t k, int64_t ldx,
                           const uint8_t *packed, const uint8_t *scales, float s_t, int64_t n,
                           const uint16_t *lora_a, const uint16_t *lora_b, int r, float lora_scale,
                           const int64_t *rows, int64_t nrows, double *y, int threads) {
    if (!x) return -1;
    return gemm_impl(x, NULL, m, k, ldx, packed, scales, s_t, n, lora_a, lora_b, r, lora_scale, rows, nrows, y,
                     threads);
}

int oracle_w4a16_lora_gemm_f64(const double *x, int64_t m, int64_t k, int64_t ldx,
                               const uint8_t *packed, const uint8_t *scales, float s_t, int64_t n,
                               const uint16_t *lora_a, const uint16_t *lora_b, int r, float lora_scale,
                               const int64_t *rows, int64_t nrows, double *y, int threads) {
    if (!x) return -1;
    return gemm_impl(NULL, x, m, k, ldx, packed, scales, s_t, n, lora_a, lora_b, r, lora_scale, rows, nrows, y,
                     threads);
}

/* ------------------------------------------------------------------------ */
/* Backward of the layer (the update phase trains the LoRA; W is frozen)     */
/* ------------------------------------------------------------------------ */
/* With y = x what^T + lambda t B^T and t = x A^T (forward above), and an
 * upstream gradient dy [M, N], the chain rule gives (g = dy B, [M, r]):
 *   dx = dy what + lambda g A          [M, K]
 *   dA = lambda g^T x                   [r, K]
 *   dB = lambda dy^T t                  [N, r]
 * (what is dequantized exactly; W itself gets no gradient, as in the pages'
 * LoRA training, [BoA-LoRA]).  Any of dx, dA, dB may be NULL.  All fp64.    */
typedef struct {
    const uint16_t *dy, *x; int64_t m, n, k;
    const uint8_t *packed, *scales; double s_t;
    const uint16_t *a, *b; int r; double lam;
    double *t, *g, *dx, *da, *db;
} bwd_ctx;

/* t[i, :] = x[i, :] A^T and g[i, :] = dy[i, :] B for rows i in [i0, i1) */
static void bwd_rank_rows(void *p, int64_t i0, int64_t i1) {
    bwd_ctx *c = (bwd_ctx *)p;
    for (int64_t i = i0; i < i1; ++i)
        for (int j = 0; j < c->r; ++j) {
            double at = 0.0, ag = 0.0;
            for (int64_t kk = 0; kk < c->k; ++kk)
                at += oracle_bf16_decode(c->x[i * c->k + kk]) * oracle_bf16_decode(c->a[(int64_t)j * c->k + kk]);
            for (int64_t nn = 0; nn < c->n; ++nn)
                ag += oracle_bf16_decode(c->dy[i * c->n + nn]) * oracle_bf16_decode(c->b[nn * c->r + j]);
            c->t[i * c->r + j] = at;
            c->g[i * c->r + j] = ag;
        }
}

/* dx rows [i0, i1): the sum over nn in ascending order, then the LoRA term */
static void bwd_dx_rows(void *p, int64_t i0, int64_t i1) {
    bwd_ctx *c = (bwd_ctx *)p;
    const int64_t k = c->k;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)k);
    if (!wrow) return;
    for (int64_t i = i0; i < i1; ++i)
        for (int64_t kk = 0; kk < k; ++kk) c->dx[i * k + kk] = 0.0;
    for (int64_t nn = 0; nn < c->n; ++nn) {
        for (int64_t kk = 0; kk < k; ++kk) {
            uint8_t byte = c->packed[nn * (k / 2) + kk / 2];
            int code = (kk & 1) ? (byte >> 4) : (byte & 15);
            wrow[kk] = oracle_e2m1_decode(code) * oracle_e4m3_decode(c->scales[nn * (k / 16) + kk / 16]) * c->s_t;
        }
        for (int64_t i = i0; i < i1; ++i) {
            const double d = oracle_bf16_decode(c->dy[i * c->n + nn]);
            for (int64_t kk = 0; kk < k; ++kk) c->dx[i * k + kk] += d * wrow[kk];
        }
    }
    for (int64_t i = i0; i < i1; ++i)
        for (int64_t kk = 0; kk < k; ++kk) {
            double acc = 0.0;
            for (int j = 0; j < c->r; ++j) acc += c->g[i * c->r + j] * oracle_bf16_decode(c->a[(int64_t)j * k + kk]);
            c->dx[i * k + kk] += c->lam * acc;
        }
    free(wrow);
}

/* dA columns [k0, k1) of every rank row: sums over i in ascending order */
static void bwd_da_cols(void *p, int64_t k0, int64_t k1) {
    bwd_ctx *c = (bwd_ctx *)p;
    for (int j = 0; j < c->r; ++j)
        for (int64_t kk = k0; kk < k1; ++kk) {
            double acc = 0.0;
            for (int64_t i = 0; i < c->m; ++i) acc += c->g[i * c->r + j] * oracle_bf16_decode(c->x[i * c->k + kk]);
            c->da[(int64_t)j * c->k + kk] = c->lam * acc;
        }
}

/* dB rows [n0, n1): sums over i in ascending order */
static void bwd_db_rows(void *p, int64_t n0, int64_t n1) {
    bwd_ctx *c = (bwd_ctx *)p;
    for (int64_t nn = n0; nn < n1; ++nn)
        for (int j = 0; j < c->r; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < c->m; ++i) acc += oracle_bf16_decode(c->dy[i * c->n + nn]) * c->t[i * c->r + j];
            c->db[nn * c->r + j] = c->lam * acc;
        }
}

int oracle_w4a16_lora_backward(const uint16_t *dy, const uint16_t *x, int64_t m, int64_t n, int64_t k,
                               const uint8_t *packed, const uint8_t *scales, float s_t,
                               const uint16_t *lora_a, const uint16_t *lora_b, int r, float lora_scale,
                               double *dx, double *da, double *db, int threads) {
    if (!dy || !x || !packed || !scales || m <= 0 || n <= 0 || k <= 0 || k % 16 || r < 0) return -1;
    if (r > 0 && (!lora_a || !lora_b)) return -1;
    double *t = (double *)calloc((size_t)(m * (r > 0 ? r : 1)), sizeof(double));
    double *g = (double *)calloc((size_t)(m * (r > 0 ? r : 1)), sizeof(double));
    if (!t || !g) { free(t); free(g); return -2; }
    bwd_ctx c = {dy, x, m, n, k, packed, scales, (double)s_t, lora_a, lora_b, r, (double)lora_scale,
                 t, g, dx, da, db};
    /* each stage splits its independent output rows (or columns) over the
     * threads; every sum runs in the order the definition writes it */
    if (r > 0) parallel_range(threads, m, bwd_rank_rows, &c);
    if (dx) parallel_range(threads, m, bwd_dx_rows, &c);
    if (da && r > 0) parallel_range(threads, k, bwd_da_cols, &c);
    if (db && r > 0) parallel_range(threads, n, bwd_db_rows, &c);
    free(t);
    free(g);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* AQN: schedule, Philox4x64-10 noise, noisy RMSNorm                         */
/* ------------------------------------------------------------------------ */

/* Exponential decay from sigma_start (stage 0) to sigma_end (stage S-1),
 * [README-Hint] knobs with the exponential form of [1kp-Sum]:
 * sigma_k = sigma_start * (sigma_end / sigma_start)^(k / (S - 1)).
 * Reading: one stage means sigma_start; stages outside [0, S-1] clamp.    */
double oracle_aqn_sigma(int stage, int num_stages, double sigma_start, double sigma_end) {
    if (num_stages <= 1) return sigma_start;
    if (stage < 0) stage = 0;
    if (stage > num_stages - 1) stage = num_stages - 1;
    return sigma_start * pow(sigma_end / sigma_start, (double)stage / (double)(num_stages - 1));
}

/* Philox4x64-10 [Philox]: 10 rounds of the 4x64 S-box; round multipliers and
 * key increments (Weyl constants) from the paper. */
void oracle_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Channel noise z[0..h) for one (seed, step, layer): channel c uses block
 * i = c/4 of Philox with key (seed, layer) and counter (i, step, 0, 0).
 * Box-Muller [BoxMuller] on the pairs (r0, r1) -> channels 4i, 4i+1 and
 * (r2, r3) -> 4i+2, 4i+3:  u1 = ((ra >> 40) + 1) 2^-24 in (0, 1],
 * u2 = (rb >> 40) 2^-24 in [0, 1),  z = sqrt(-2 ln u1) (cos, sin)(2 pi u2).
 * Reading: the pages give only "channel-wise Gaussian"; this stream is the
 * implementation's own definition.                                         */
void oracle_aqn_noise(uint64_t seed, uint64_t step, uint32_t layer, int64_t h, double *z) {
    const double two24 = 16777216.0;
    for (int64_t i = 0; i * 4 < h; ++i) {
        uint64_t ctr[4] = {(uint64_t)i, step, 0, 0}, key[2] = {seed, (uint64_t)layer}, r[4];
        oracle_philox4x64_10(ctr, key, r);
        for (int pair = 0; pair < 2; ++pair) {
            double u1 = ((double)(r[2 * pair] >> 40) + 1.0) / two24;
            double u2 = (double)(r[2 * pair + 1] >> 40) / two24;
            double rad = sqrt(-2.0 * log(u1));
            double ang = 2.0 * M_PI * u2;
            int64_t c = 4 * i + 2 * pair;
            if (c < h) z[c] = rad * cos(ang);
            if (c + 1 < h) z[c + 1] = rad * sin(ang);
        }
    }
}

/* y[m, c] = x[m, c] / sqrt(mean_c x[m, c]^2 + eps) * w_eff[c]  (fp64) */
int oracle_rmsnorm(const uint16_t *x, int64_t m, int64_t h, int64_t ldx,
                   const double *w_eff, double eps, double *y) {
    if (!x || !w_eff || !y || m <= 0 || h <= 0 || ldx < h) return -1;
    for (int64_t r = 0; r < m; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < h; ++c) {
            double v = oracle_bf16_decode(x[r * ldx + c]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)h + eps);
        for (int64_t c = 0; c < h; ++c)
            y[r * h + c] = oracle_bf16_decode(x[r * ldx + c]) * inv * w_eff[c];
    }
    return 0;
}

/* AQN RMSNorm [1kp-Sum], [Dfc-Test]: the noise enters additively through the
 * norm's FP32 scale vector, w_noisy = w + sigma * z, shared by all rows;
 * then y = RMSNorm(x) * w_noisy.  w_noisy_out may be NULL.               */
int oracle_aqn_rmsnorm(const uint16_t *x, int64_t m, int64_t h, int64_t ldx,
                       const float *w, double eps, double sigma,
                       uint64_t seed, uint64_t step, uint32_t layer,
                       double *y, double *w_noisy_out) {
    if (!x || !w || !y || m <= 0 || h <= 0 || ldx < h || !(eps > 0.0) || !(sigma >= 0.0))
        return -1;
    double *z = (double *)malloc(sizeof(double) * (size_t)h);
    double *we = (double *)malloc(sizeof(double) * (size_t)h);
    if (!z || !we) { free(z); free(we); return -2; }
    oracle_aqn_noise(seed, step, layer, h, z);
    for (int64_t c = 0; c < h; ++c) we[c] = (double)w[c] + sigma * z[c];
    if (w_noisy_out) memcpy(w_noisy_out, we, sizeof(double) * (size_t)h);
    int rc = oracle_rmsnorm(x, m, h, ldx, we, eps, y);
    free(z);
    free(we);
    return rc;
}
