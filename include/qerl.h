/*
 * qerl.h -- C ABI of libqerl: the rollout-phase linear layer of QeRL on
 * AMD Instinct MI355X (gfx950).
 *
 * Three operations, each backed by hand-written HIP kernels:
 *   qerl_nvfp4_quantize   BF16 weight -> NVFP4 (E2M1 codes, one E4M3 scale per
 *                         16 values along K, one FP32 tensor scale);
 *   qerl_w4a16_lora_gemm  y = x * deq(W)^T + lora_scale * (x * A^T) * B^T with
 *                         NVFP4 W, BF16 x, BF16 LoRA A/B, BF16 y;
 *   qerl_aqn_rmsnorm      RMSNorm whose FP32 scale vector carries the adaptive
 *                         quantization noise w + sigma * z (z channel-wise N(0,1)).
 *
 * Sources (page -- section):
 *   NVFP4 format and block scaling: "QeRL: NVFP4-Quantized Reinforcement
 *     Learning -- Redefining Efficiency in AI Training and Inference", section
 *     "NVFP4: NVIDIA's FP4 Format" (16-value blocks, E4M3 block scale, FP32
 *     tensor scale, scale = round_up(amax / vmax), value = round_to_even(v / scale)).
 *   NVFP4 x BF16 rollout kernel with LoRA: "NVlabs/QeRL" README,
 *     "Acknowledgement"; bitsofall page, "LoRA (Low-Rank Adaptation)" and
 *     "Implementation and Practical Details" (weight-only; NVFP4 + LoRA sum).
 *   AQN: "Paper 2510.11696 -- QeRL: Beyond Efficiency", "Summary" (channel-wise
 *     Gaussian noise through the normalization layer, exponential decay);
 *     README "Hints for QeRL training", item 3 (sigma_start, sigma_end,
 *     num_stages).
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers into caller-owned memory; the
 *     library never allocates, frees or retains them.  BF16 arrays are passed as
 *     void* to 16-bit payloads.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work: QERL_OK means "enqueued"; device faults surface at the caller's next
 *     synchronization.  Calls are stream-ordered and thread-safe.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     the call then returns a non-OK status and touches no memory.
 *   - Alignment (else QERL_ERR_ALIGN): the arrays a call streams with 16-byte
 *     vector loads -- w, packed, scales, workspace of the quantizer; x, packed,
 *     scales, lora_a, lora_b, workspace of the GEMM -- must be 16-byte aligned
 *     and their leading dimensions (ldw, ldx of the GEMM) multiples of 8
 *     elements.  Every other pointer needs only the alignment of its element
 *     type, and other leading dimensions are free.
 *   - No C++ exception crosses this interface.
 */
#ifndef QERL_H
#define QERL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qerl_status {
    QERL_OK = 0,
    QERL_ERR_NULL = 1,      /* a required pointer is NULL */
    QERL_ERR_SHAPE = 2,     /* a size is non-positive, too large, or k % 16 != 0 */
    QERL_ERR_ALIGN = 3,     /* a pointer or leading dimension breaks the alignment rule */
    QERL_ERR_ARG = 4,       /* a scalar argument is out of range (flags, rank, eps, sigma) */
    QERL_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the size query returns */
    QERL_ERR_HIP = 6        /* the HIP runtime rejected a launch; see qerl_last_error() */
} qerl_status;

/* flags of qerl_nvfp4_quantize, bit 0: how the block scale is rounded to E4M3 */
#define QERL_SCALE_ROUND_UP 0u /* least E4M3 value >= amax_b / (6 s_t) (default) */
#define QERL_SCALE_RNE 1u      /* nearest E4M3 value, ties to the even code */

#define QERL_MAX_LORA_RANK 128
#define QERL_MAX_SEGMENTS 4    /* projections of one qerl_w4a16_lora_gemm_multi call */
#define QERL_MAX_NORM_WIDTH 16384
/* bytes of the per-device static scratch behind qerl_w4a16_lora_gemm_noalloc */
#define QERL_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/* ----------------------------------------------------------------------- */
/* BF16 -> NVFP4 quantizer                                                   */
/* ----------------------------------------------------------------------- */
/* Bytes of device workspace qerl_nvfp4_quantize needs for an [n, k] weight. */
size_t qerl_nvfp4_quantize_workspace_size(int64_t n, int64_t k);

/*
 * Quantize W (BF16, [n, k] row-major, row stride ldw >= k elements) to NVFP4,
 * following the block-scaling formula of the bitsofall page ("NVFP4: NVIDIA's
 * FP4 Format"), with the two-level scale of the same section:
 *   s_t   = fl32(amax(|W|) / 2688)          (2688 = 6 * 448; s_t = 1 if W == 0)
 *   sb    = E4M3 rounding of amax_b / (6 s_t) per block of 16 along k, clamped
 *           to 448 (flags: QERL_SCALE_ROUND_UP or QERL_SCALE_RNE)
 *   code  = signbit(w) << 3 | RNE of |w| / (E4M3(sb) s_t) onto the E2M1 grid
 *           {0, .5, 1, 1.5, 2, 3, 4, 6} (saturating at 6; all 0 when sb == 0)
 * All rounding decisions are exact (the result is the unique one defined by
 * exact rational arithmetic).
 *
 * Outputs (device, caller-owned):
 *   packed       uint8 [n, k/2]: byte j of a row holds element 2j in its low
 *                nibble and element 2j+1 in its high nibble;
 *   scales       uint8 [n, k/16]: E4M3 (OCP "FN") byte of each block;
 *   tensor_scale float [1]: s_t, a decode multiplier: w ~= e2m1 * e4m3 * s_t.
 * tensor_scale_in (device, nullable): when given, that s_t is used unchanged
 *   and the tensor amax pass is skipped; it must be positive and finite.
 * Non-finite input (a NaN or Inf weight, or an invalid tensor_scale_in) is
 * reported in-band: *tensor_scale = NaN, packed and scales unspecified.
 * Requires n >= 1, k >= 16, k % 16 == 0, workspace_bytes >= the size query.
 */
qerl_status qerl_nvfp4_quantize(const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                const float *tensor_scale_in, uint32_t flags,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * qerl_nvfp4_quantize with stochastic rounding of the elements (the FP4
 * training work that the bitsofall page's "NVFP4: NVIDIA's FP4 Format"
 * section cites pairs 16-value blocks with stochastic rounding): s_t and the
 * block scales are exactly those of qerl_nvfp4_quantize with the same flags;
 * each element goes to one of the two E2M1 grid points lo <= |w|/S < hi
 * around it (S = E4M3(sb) s_t), to hi with probability (|w|/S - lo)/(hi - lo),
 * so its expected dequantized value is w (values at or above 6 S take 6, grid
 * values stay).  The uniform of element e = row * k + col is u = (r >> 40) 2^-24
 * for word e % 4 of Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0)
 * and counter (e / 4, 0, 1, 0); up <=> u (hi - lo) S < |w| - lo S, decided
 * exactly.  Same arguments, workspace and errors as qerl_nvfp4_quantize.
 */
qerl_status qerl_nvfp4_quantize_stochastic(const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                           uint8_t *packed, uint8_t *scales, float *tensor_scale,
                                           const float *tensor_scale_in, uint32_t flags, uint64_t seed,
                                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * BF16 -> MXFP4 (OCP Microscaling Formats v1.0: E2M1 elements, one E8M0 scale
 * per 32 elements along k), the coarser sibling format the bitsofall page
 * ("NVFP4: NVIDIA's FP4 Format") contrasts with NVFP4's 16-value blocks:
 *   scale byte = floor(log2 amax_b) - 2 + 127 clamped to [0, 254] (0 for an
 *                all-zero block; 0xFF, with zero codes, for a block holding
 *                Inf or NaN); X = 2^(byte - 127)
 *   code       = signbit(w) << 3 | RNE of |w| / X onto the E2M1 grid,
 *                saturating at 6
 * Outputs: packed uint8 [n, k/2] (nibble order as qerl_nvfp4_quantize), scales
 * uint8 [n, k/32].  One pass, no workspace.  Requires n >= 1, k >= 32,
 * k % 32 == 0, ldw >= k, 16-byte aligned w/packed and ldw % 8 == 0.
 */
qerl_status qerl_mxfp4_quantize(const void *w_bf16, int64_t n, int64_t k, int64_t ldw,
                                uint8_t *packed, uint8_t *scales, void *stream);

/*
 * NVFP4 -> BF16: out[n, j] = e2m1(code[n, j]) * e4m3(scales[n, j/16]) * s_t,
 * the value the bitsofall page's "NVFP4: NVIDIA's FP4 Format" gives a stored
 * weight, rounded once to the nearest BF16 (ties to even; the exact product
 * is formed first).  This is the dequantization an unfused update-phase
 * forward performs before 16-bit GEMMs (README "Hints for QeRL training",
 * item 2; bitsofall "Workflow: Rollout, Update, Quantization");
 * qerl_w4a16_lora_gemm computes the same layer without it.
 *   packed        uint8 [n, k/2] as written by qerl_nvfp4_quantize (even
 *                 element in the low nibble), 8-byte aligned
 *   scales        uint8 [n, k/16] E4M3 bytes (0x7F / 0xFF, E4M3 NaN, give NaN)
 *   tensor_scale  device pointer to the FP32 s_t
 *   out_bf16      [n, k], row stride ldo >= k, ldo % 8 == 0, 16-byte aligned;
 *                 must not overlap the inputs
 * Requires n >= 1, k >= 16, k % 16 == 0.  No workspace.
 */
qerl_status qerl_nvfp4_dequantize(const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                  int64_t n, int64_t k, void *out_bf16, int64_t ldo, void *stream);

/* ----------------------------------------------------------------------- */
/* W4A16 (NVFP4 weight x BF16 activation) linear layer with LoRA epilogue   */
/* ----------------------------------------------------------------------- */
/* Bytes of device workspace qerl_w4a16_lora_gemm needs. */
size_t qerl_w4a16_lora_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t r);

/*
 * y[m, n] = sum_k x[m,k] * e2m1(q[n,k]) * e4m3(sb[n,k/16]) * s_t
 *         + lora_scale * sum_j (sum_k x[m,k] * A[j,k]) * B[n,j]
 * i.e. the frozen NVFP4 base (README "Acknowledgement": NVFP4 x BF16 kernel)
 * plus the BF16 low-rank update (bitsofall "LoRA (Low-Rank Adaptation)";
 * lora_scale is alpha / r).  No bias.  FP32 accumulation, BF16 (RNE) output.
 *
 *   x_bf16        [m, k], row stride ldx >= k
 *   packed, scales, tensor_scale   as written by qerl_nvfp4_quantize for an
 *                 [n, k] weight (tensor_scale is a device pointer)
 *   lora_a_bf16   [r, k] contiguous; lora_b_bf16 [n, r] contiguous; both may be
 *                 NULL only when r == 0 (no LoRA)
 *   y_bf16        [m, n], row stride ldy >= n; must not overlap any input
 *   workspace     device memory of at least the size query (partial sums;
 *                 no state is kept between calls, nothing needs to be zero);
 *                 calls that overlap in time must not share a workspace
 * m <= 256 takes the decode path: a launch that streams the packed weights
 * once (E2M1/E4M3 decode in registers, BF16 MFMA) and stores partial sums,
 * and a small launch that adds them in a fixed order with the LoRA term;
 * larger m takes a BF16-MFMA path on dequantized tiles with the LoRA product
 * folded into the same accumulation.
 * Requires m, n >= 1, k >= 16, k % 16 == 0, 0 <= r <= QERL_MAX_LORA_RANK,
 * finite lora_scale, workspace_bytes >= the size query.
 */
qerl_status qerl_w4a16_lora_gemm(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                 const uint8_t *packed, const uint8_t *scales,
                                 const float *tensor_scale, int64_t n,
                                 const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                 float lora_scale, void *y_bf16, int64_t ldy,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the layer of
 * qerl_w4a16_lora_gemm (same arguments, same kernels, same results) with no
 * workspace argument.  Its partial sums go to a static device array of
 * QERL_NOALLOC_SCRATCH_BYTES (48 MiB) that the library's code object holds
 * on each device it runs on, for the life of the process; its device address
 * is looked up once per device on the first call there.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *   Returns QERL_ERR_WORKSPACE, before enqueueing anything, when
 *   qerl_w4a16_lora_gemm_workspace_size(m, n, k, r) exceeds the scratch (48
 *   MiB covers decode batches of m <= 64 at r <= 128 for weights of up to
 *   27648 x 5120 and 5120 x 27648, the largest projections of a 32B-class
 *   decoder layer).
 *   Every call on one device shares that device's scratch, which keeps the
 *   last call's partial sums (nothing in it needs to start at zero): calls
 *   that may overlap in time on one device -- on different streams, or from
 *   different threads without ordering -- race and give wrong results.
 *   Stream-ordered calls on one stream are safe.
 */
qerl_status qerl_w4a16_lora_gemm_noalloc(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                         const uint8_t *packed, const uint8_t *scales,
                                         const float *tensor_scale, int64_t n,
                                         const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                         float lora_scale, void *y_bf16, int64_t ldy, void *stream);

/*
 * One projection of qerl_w4a16_lora_gemm_multi: every field as the argument
 * of the same name of qerl_w4a16_lora_gemm (device pointers; y_bf16 [m, n]
 * with row stride ldy).
 */
typedef struct {
    const uint8_t *packed;
    const uint8_t *scales;
    const float *tensor_scale;
    int64_t n;
    const void *lora_a_bf16;
    const void *lora_b_bf16;
    int32_t r;
    float lora_scale;
    void *y_bf16;
    int64_t ldy;
} qerl_gemm_segment;

/* Bytes of device workspace qerl_w4a16_lora_gemm_multi needs (reads n and r
 * of segs[0 .. nseg)). */
size_t qerl_w4a16_lora_gemm_multi_workspace_size(int64_t m, int64_t k, const qerl_gemm_segment *segs,
                                                 int32_t nseg);

/*
 * Several projections of the same activations in one call: for each segment
 * i < nseg (1 <= nseg <= QERL_MAX_SEGMENTS), exactly what qerl_w4a16_lora_gemm
 * computes for x and segs[i] -- each with its own weight, tensor scale, LoRA
 * and output.  The operation is the layer of qerl_w4a16_lora_gemm (README
 * "Acknowledgement"; bitsofall "LoRA (Low-Rank Adaptation)"), applied to the
 * projections that read one normed input (q/k/v, gate/up).  For m <= 256 the
 * segments share the launches (so a decode step spends two launches, not two
 * per projection, on them); the K split is chosen for all segments together, so
 * the FP32 summation order, and with it the last bit of y, can differ from
 * separate calls.  Larger m runs the segments one after another.
 *   segs          host array of nseg segments, read during the call only
 *   workspace     as for qerl_w4a16_lora_gemm, of at least the size query
 * Requires the conditions of qerl_w4a16_lora_gemm for every segment, outputs
 * that overlap neither each other nor any input.
 */
qerl_status qerl_w4a16_lora_gemm_multi(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                       const qerl_gemm_segment *segs, int32_t nseg, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Bytes of device workspace qerl_rmsnorm_w4a16_lora_gemm_multi needs (reads
 * n and r of segs[0 .. nseg)). */
size_t qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size(int64_t m, int64_t k, const qerl_gemm_segment *segs,
                                                         int32_t nseg);

/*
 * An RMSNorm and the projections that read its output, in one call: with
 *   xn[i, c] = x[i, c] / sqrt(mean_c x[i, c]^2 + eps) * norm_weight[c]
 * each segment i < nseg gets what qerl_w4a16_lora_gemm computes for xn and
 * segs[i].  This is the norm of qerl_aqn_rmsnorm with its scale vector given:
 * AQN's noise lives in the norm's scale parameters (dataforcee page; 1kpapers
 * "Summary"), one vector per (seed, step, layer), so norm_weight is the
 * vector qerl_aqn_noisy_weight returns for the current noise stage (or the
 * plain weight for sigma = 0), drawn once per step rather than once per call.
 * For m <= 16 and k % 32 == 0 the norm runs inside the decode launches: each
 * row's 1 / rms is a factor of its whole output row, so the product takes
 * bf16(x * norm_weight) and the FP32 result is scaled by 1 / rms at the end
 * (the LoRA term likewise).  Otherwise the norm is a launch of its
 * own writing BF16 xn (as qerl_aqn_rmsnorm's y_bf16) into the workspace,
 * followed by qerl_w4a16_lora_gemm_multi on it.  The two roundings differ in
 * the last bits of y, within the GEMM's tolerance.
 *   x_bf16        [m, k] (row stride ldx): the norm's input
 *   norm_weight   FP32 [k], 16-byte aligned
 *   segs, workspace as for qerl_w4a16_lora_gemm_multi, workspace of at least
 *                 the size query
 * Requires the conditions of qerl_w4a16_lora_gemm_multi, k <=
 * QERL_MAX_NORM_WIDTH, eps > 0 and finite.
 */
qerl_status qerl_rmsnorm_w4a16_lora_gemm_multi(const void *x_bf16, int64_t m, int64_t k, int64_t ldx,
                                               const float *norm_weight, float eps,
                                               const qerl_gemm_segment *segs, int32_t nseg,
                                               void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------- */
/* Backward of the layer (update phase: LoRA trained, NVFP4 base frozen)    */
/* ----------------------------------------------------------------------- */
/* Bytes of device workspace qerl_w4a16_lora_backward needs. */
size_t qerl_w4a16_lora_backward_workspace_size(int64_t m, int64_t n, int64_t k, int32_t r);

/*
 * Gradients of the layer of qerl_w4a16_lora_gemm, y = x what^T +
 * lora_scale (x A^T) B^T, for an upstream gradient dy: only the low-rank
 * matrices train, the NVFP4 weight stays frozen (bitsofall page, "LoRA
 * (Low-Rank Adaptation)"; the rollout kernel's layer, README
 * "Acknowledgement").  With t = x A^T and g = dy B ([m, r], FP32):
 *   dx = dy what + lora_scale g A       BF16 [m, k] (RNE of the FP32 sum)
 *   dA = lora_scale g^T x               FP32 [r, k]
 *   dB = lora_scale dy^T t              FP32 [n, r]
 * what is dequantized exactly (e2m1 * e4m3 * s_t) inside the kernel; nothing
 * is re-laid out.
 *   dy_bf16      [m, n], row stride ldy; x_bf16 [m, k], row stride ldx (the
 *                forward input, for dA and dB)
 *   packed, scales, tensor_scale, lora_a_bf16, lora_b_bf16, r, lora_scale
 *                as for qerl_w4a16_lora_gemm
 *   dx_bf16      nullable; [m, k] with row stride lddx
 *   da_f32, db_f32  nullable; contiguous; ignored when r == 0
 *   workspace    device memory of at least the size query (t, g and partial
 *                sums; no state is kept)
 * Requires m, n >= 1, k >= 16, k % 16 == 0, 0 <= r <= QERL_MAX_LORA_RANK,
 * ldy >= n, ldx >= k, lddx >= k, finite lora_scale, 16-byte aligned dy, x,
 * packed and lora_a with ldx % 8 == 0 (ldy any), 2-byte aligned dx.
 */
qerl_status qerl_w4a16_lora_backward(const void *dy_bf16, int64_t m, int64_t n, int64_t ldy,
                                     const void *x_bf16, int64_t k, int64_t ldx,
                                     const uint8_t *packed, const uint8_t *scales, const float *tensor_scale,
                                     const void *lora_a_bf16, const void *lora_b_bf16, int32_t r,
                                     float lora_scale, void *dx_bf16, int64_t lddx, float *da_f32,
                                     float *db_f32, void *workspace, size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------------- */
/* AQN RMSNorm                                                               */
/* ----------------------------------------------------------------------- */
/*
 * sigma of noise stage `stage` out of `num_stages` (README "Hints for QeRL
 * training", item 3; exponential decay per the 1kpapers "Summary"):
 *   sigma_k = sigma_start * (sigma_end / sigma_start)^(k / (num_stages - 1)),
 * stage clamped to [0, num_stages - 1]; num_stages <= 1 gives sigma_start.
 * Host-only; returns NaN for non-positive or non-finite sigma_start/sigma_end.
 */
float qerl_aqn_sigma(int32_t stage, int32_t num_stages, float sigma_start, float sigma_end);

/*
 * y[i, c] = x[i, c] / sqrt(mean_c x[i, c]^2 + eps) * (w[c] + sigma * z[c])
 * The noise z is one channel-wise N(0, 1) vector shared by every row (the
 * 1kpapers "Summary": channel-wise Gaussian noise via the normalization layer;
 * dataforcee page: it lives in the norm's scale parameters).  z is defined by
 * counter-based Philox4x64-10 (Salmon et al., SC'11) with key (seed, layer_id)
 * and counter (c / 4, step, 0, 0); its four words r0..r3 give channels 4i..4i+3
 * by Box-Muller: u1 = ((ra >> 40) + 1) 2^-24, u2 = (rb >> 40) 2^-24,
 * z = sqrt(-2 ln u1) * (cos, sin)(2 pi u2) for (ra, rb) = (r0, r1), (r2, r3).
 *
 *   x_bf16   [m, h] with row stride ldx >= h; weight FP32 [h]
 *   y_f32    FP32 [m, h] (nullable), y_bf16 BF16 [m, h] (nullable, RNE of the
 *            FP32 value); at least one must be given; both use row stride ldy
 *   noisy_weight_out FP32 [h] (nullable): w + sigma * z
 * Requires m, h >= 1, h <= QERL_MAX_NORM_WIDTH, eps > 0 and finite,
 * sigma >= 0 and finite.
 */
qerl_status qerl_aqn_rmsnorm(const void *x_bf16, int64_t m, int64_t h, int64_t ldx,
                             const float *weight, float eps, float sigma,
                             uint64_t seed, uint64_t step, uint32_t layer_id,
                             float *y_f32, void *y_bf16, int64_t ldy,
                             float *noisy_weight_out, void *stream);

/*
 * The AQN scale vector alone: noisy_weight_out[c] = weight[c] + sigma * z[c],
 * with z exactly as qerl_aqn_rmsnorm draws it (the same seed, step and
 * layer_id give the vector that call multiplies by, bit for bit).  For
 * qerl_rmsnorm_w4a16_lora_gemm_multi, which takes the vector as its norm
 * weight.
 *   weight, noisy_weight_out  FP32 [h] device arrays (may be the same array)
 * Requires 1 <= h <= QERL_MAX_NORM_WIDTH, sigma >= 0 and finite.
 */
qerl_status qerl_aqn_noisy_weight(const float *weight, int64_t h, float sigma, uint64_t seed, uint64_t step,
                                  uint32_t layer_id, float *noisy_weight_out, void *stream);

/* ----------------------------------------------------------------------- */
/* diagnostics                                                               */
/* ----------------------------------------------------------------------- */
/* Static English text for a status code. */
const char *qerl_status_string(qerl_status status);
/* Text of the last error on the calling thread ("" if none): the argument
 * check that failed, or the HIP runtime's message for QERL_ERR_HIP; valid
 * until the next library call on that thread. */
const char *qerl_last_error(void);
/* The same text (thread-local), under the name the boundary's error
 * convention gives launch failures. */
const char *qerl_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QERL_H */
