/*
 * q4g128.h -- C ABI of the int4 group-128 weight-streaming GEMV library for
 * AMD Instinct MI355X (gfx950).
 *
 * Weight format (rumik-oss-1 int4 write-up, rtts.neoandmatrix.me, section
 * "Step 3: an int4 file and a first kernel on the laptop"): a projection
 * matrix W with N output rows and K input columns is quantised in groups of
 * 128 consecutive columns of each row; every group has one fp16 scale and
 * one fp16 minimum, and two 4-bit codes share one byte.  The dequantised
 * weight is
 *
 *     w[n][k] = code[n][k] * scale[n][k / 128] + min[n][k / 128].
 *
 * Canonical layout used by every entry point (readings of the format that
 * the pages leave open are stated here once):
 *   packed  uint8  [N][K/2]  row-major; byte j of row n holds code[n][2j] in
 *                            bits 0..3 and code[n][2j+1] in bits 4..7.
 *   scales  uint16 [N][K/128] row-major fp16 bit patterns.
 *   mins    uint16 [N][K/128] row-major fp16 bit patterns.
 *   x / X   uint16 [B][K]    row-major fp16 bit patterns, one activation
 *                            vector (request or prompt token) per row.
 *   y / Y   float  [B][N]    row-major fp32 results; Y = X * W^T.
 *
 * Ownership and execution model (all entry points):
 *   - Every pointer is DEVICE memory owned by the caller (except the
 *     grouped call's descriptor array, a host array).  The library never
 *     allocates or frees device memory, keeps no pointer after returning,
 *     and needs no workspace; only the grouped call uses host memory of its
 *     own, for checking its descriptors during the call.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work; they never synchronise the host.  Buffers must stay alive until
 *     the enqueued work completes.
 *   - Outputs are fully overwritten and must not overlap any input.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call enqueues nothing.
 *   - Results are deterministic: no atomics, fixed reduction orders.
 *
 * Limits: 1 <= N <= 2^31 - 256; K a multiple of 128 with 128 <= K <= 32768;
 * batch / prompt rows at most 2^31 - 256.
 */
#ifndef Q4G128_H
#define Q4G128_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t q4_status;

/* Only the entry points below are exported from libq4g128.so. */
#define Q4_API __attribute__((visibility("default")))

#define Q4_OK 0
/* NULL pointer, N <= 0, B outside [1, 16], M <= 0, or an output that
   overlaps an input. */
#define Q4_EINVAL (-1)
/* K not a positive multiple of 128, K above 32768, or N / M above
   Q4G128_MAX_N. */
#define Q4_ESHAPE (-2)
/* codes / packed / x / X / W not 16-byte aligned; scales / mins not 2-byte
   aligned; y / Y not 4-byte aligned. */
#define Q4_EALIGN (-3)
/* The HIP runtime reported an error while querying the device or launching;
   q4g128_last_hip_error() returns the hipError_t of the calling thread. */
#define Q4_EDEVICE (-4)

#define Q4G128_GROUP 128
#define Q4G128_MAX_K 32768
#define Q4G128_MAX_BATCH 16
#define Q4G128_MAX_N 0x7FFFFF00LL
#define Q4G128_INT8_MAX_K 8192

/*
 * q4g128_pack -- two codes per byte.
 *   codes  [N][K] uint8, only the low 4 bits of each code are used.
 *   packed [N][K/2] uint8, written.
 * The export step of the rumik write-up ("Step 3": a short CPU job wrote the
 * int4 file) in device form; untimed set-up, not part of the decode step.
 */
Q4_API q4_status q4g128_pack(const uint8_t* codes, uint8_t* packed,
                      int64_t n, int64_t k, void* stream);

/*
 * q4g128_gemm_prefill_epilogue -- the same Y[m][n] = sum_k w[n][k] * X[m][k]
 * in the form of the rumik write-up's prefill ("Step 8: a prefill that
 * stays int4"): each 128-column group is unpacked on chip to exact integer
 * codes and contracted with the activations on the matrix cores (fp32
 * accumulation), and the group's scale and minimum are applied to that
 * result: Y += scale * sum(code*x) + min * sum(x).  No weight is rounded to
 * fp16, so results carry only fp32 summation error (within 512 * 2^-24 *
 * sum_k |w*x| of the exact product).  Same arguments, limits, errors and
 * execution model as q4g128_gemm_prefill; any M >= 1.
 */
Q4_API q4_status q4g128_gemm_prefill_epilogue(const uint8_t* packed, const uint16_t* scales,
                                       const uint16_t* mins, const uint16_t* X, float* Y,
                                       int64_t n, int64_t k, int64_t m, void* stream);

/*
 * q4g128_quantize -- export float32 weights to the format above.
 * The rumik write-up ("Step 3") exports every projection with a short CPU
 * job: groups of 128 columns, one fp16 scale and one fp16 minimum per group.
 * The pages give no formula; the reading implemented is the min/max affine
 * quantiser that the dequantisation w = code*scale + min implies.  For each
 * group, with every step one IEEE fp32 operation rounded to nearest even:
 *     lo = min, hi = max of the group's 128 values
 *     min   = fp16(lo + 0)            (a zero minimum is stored as +0)
 *     scale = fp16((hi - lo) / 15)
 *     code  = clamp(round_half_even((w - min) / scale), 0, 15) against the
 *             stored fp16 min and scale; code 0 everywhere if scale == 0.
 *   W      [N][K] float32, row-major, finite with |w| <= 65504 (other values
 *          give unspecified codes, never a fault).
 *   packed [N][K/2], scales [N][K/128], mins [N][K/128]: written in full.
 * Errors: Q4_EINVAL for a NULL pointer, N <= 0 or outputs that overlap W or
 * each other; Q4_ESHAPE for K outside the limits or more than 2^36 groups;
 * Q4_EALIGN unless W and packed are 16-byte and scales / mins 2-byte
 * aligned.  Untimed set-up work, not part of the decode step.
 */
Q4_API q4_status q4g128_quantize(const float* W, uint8_t* packed, uint16_t* scales,
                          uint16_t* mins, int64_t n, int64_t k, void* stream);

/*
 * q4g128_gemv -- y[n] = sum_k w[n][k] * x[k]   (batch-1 decode product).
 * The operation that dominates batch-1 decoding in the rumik write-up
 * ("Step 3" and "Step 7: why the GEMV was stuck, and a CUDA kernel"): the
 * packed weights are streamed once, dequantised in registers and multiplied
 * by the fp16 activation vector with fp32 accumulation.
 *   packed [N][K/2], scales [N][K/128], mins [N][K/128], x [K] -> y [N] fp32.
 */
Q4_API q4_status q4g128_gemv(const uint8_t* packed, const uint16_t* scales,
                      const uint16_t* mins, const uint16_t* x, float* y,
                      int64_t n, int64_t k, void* stream);

/*
 * q4g128_gemv_grouped -- many independent batch-1 products in few launches:
 *   for every i < count:  descs[i].y = W_i * descs[i].x   (as q4g128_gemv).
 * The rumik write-up ("A detour: the laptop engine on an H100") measures a
 * small projection at about one launch latency on a fast GPU and a decode
 * step as launch-bound, and advises counting launches and issuing far fewer
 * kernels per layer ("What I would tell someone starting this").  Here all
 * projections whose K has the same pass mapping are streamed by one
 * persistent launch of up to 64 projections; the projections are read from
 * `descs` (a HOST array, read during the call and not kept).
 *   descs[i]: packed, scales, mins, x, y, n, k with the layout, alignment and
 *   limits of q4g128_gemv.
 * Every y_i is bit-identical to q4g128_gemv on projection i (same lanes,
 * chunk order and reductions per row).  The projections must be
 * independent: no y_i may overlap any input of any projection or any other
 * output (x and weights may be shared between projections).  The order in
 * which projections execute is unspecified.
 * Errors: Q4_EINVAL for descs == NULL, count < 1 or count above
 * Q4G128_MAX_GROUPED, or any overlap above; every descriptor is checked as
 * q4g128_gemv checks its arguments (first failing status returned), all
 * before any HIP call.  Q4_EDEVICE: a launch failed; projections enqueued
 * before it stay enqueued.
 */
typedef struct q4g128_gemv_desc {
    const uint8_t* packed;   /* [n][k/2] */
    const uint16_t* scales;  /* [n][k/128] fp16 */
    const uint16_t* mins;    /* [n][k/128] fp16 */
    const uint16_t* x;       /* [k] fp16 */
    float* y;                /* [n] fp32, written in full */
    int64_t n;
    int64_t k;
} q4g128_gemv_desc;

#define Q4G128_MAX_GROUPED 65536

Q4_API q4_status q4g128_gemv_grouped(const q4g128_gemv_desc* descs, int64_t count, void* stream);

/*
 * q4g128_gemm_small_batch -- Y[b][n] = sum_k w[n][k] * X[b][k], 1 <= B <= 16.
 * Continuous request batching ("Adding GPU backends to a pure-C TTS engine:
 * Metal, CUDA, and the rented-Mac trick", batching passage): each weight row
 * is read once and used for all B requests.  Row b of Y is bit-identical to
 * q4g128_gemv(X[b]) on the same weights (the same page's lesson on matching
 * the single-stream accumulation order): the arithmetic per output depends
 * on (N, K) only, never on B.
 *   X [B][K] fp16 -> Y [B][N] fp32.
 */
Q4_API q4_status q4g128_gemm_small_batch(const uint8_t* packed, const uint16_t* scales,
                                  const uint16_t* mins, const uint16_t* X, float* Y,
                                  int64_t n, int64_t k, int64_t b, void* stream);

/*
 * q4g128_gemm_prefill -- Y[m][n] = sum_k w[n][k] * X[m][k] for M prompt
 * tokens (rumik write-up, "Step 8: a prefill that stays int4": the weights
 * stay int4 in memory and are unpacked on chip for a matrix-core product).
 * Each weight is dequantised on chip to fp16, fp16(code*scale + min) with
 * one rounding, and contracted with the fp16 activations on the gfx950
 * matrix cores with fp32 accumulation.  M is a runtime argument (any
 * M >= 1, no re-specialisation per M).
 * Accuracy contract: |Y - Y16| <= 256 * 2^-24 * sum_k |fp16(w) * x| where Y16
 * is the exact product of the fp16-rounded weights; against the exact
 * weights the error adds the rounding of each weight, up to 2^-11 * |w|.
 * That term does not shrink with K: at short K (K = 128, one group per row)
 * and millions of outputs a few outputs exceed a 2e-3 relative bound of the
 * exact product (a few per 8 M outputs in tests).  Callers that need the
 * exact-weight accuracy at every output use q4g128_gemm_prefill_epilogue,
 * which keeps exact codes.  Results are not bit-identical to q4g128_gemv.
 *   X [M][K] fp16 -> Y [M][N] fp32.
 */
Q4_API q4_status q4g128_gemm_prefill(const uint8_t* packed, const uint16_t* scales,
                              const uint16_t* mins, const uint16_t* X, float* Y,
                              int64_t n, int64_t k, int64_t m, void* stream);

/*
 * q4g128_gemv_int8 -- y[n] = scale[n] * sum_k q[n][k] * x[k]  (int8 output head).
 * The rumik write-up moved the audio output head to int8 with a kernel of its
 * own: int4 group-128 was measurably too lossy there (the passage on the
 * remaining per-token time after the 36 layers, and "What I would tell
 * someone starting this").  The pages give no int8 layout; the reading
 * implemented is per-row symmetric int8:
 *   q      [N][K] int8, row-major, every value -128..127 accepted;
 *   scales [N] fp16 bit patterns, one per output row;
 *   x      [K] fp16;  y [N] fp32, written in full.
 * Products q*x are exact; sums are fp32 in a fixed order (deterministic).
 * Errors: Q4_EINVAL for a NULL pointer, N <= 0 or y overlapping an input;
 * Q4_ESHAPE unless K is a multiple of 128 with 128 <= K <= 8192 and
 * N <= Q4G128_MAX_N; Q4_EALIGN unless q and x are 16-byte, scales 2-byte
 * and y 4-byte aligned; Q4_EDEVICE as for the other entry points.
 */
Q4_API q4_status q4g128_gemv_int8(const int8_t* q, const uint16_t* scales, const uint16_t* x,
                           float* y, int64_t n, int64_t k, void* stream);

/* Static, NUL-terminated description of a status code. */
Q4_API const char* q4g128_status_string(q4_status status);

/* hipError_t recorded by the last Q4_EDEVICE return on the calling thread
   (0 if none). */
Q4_API int32_t q4g128_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4G128_H */
