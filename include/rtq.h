/*
 * rtq.h - C ABI of the quantized-resident projection GEMM for AMD MI355X (gfx950).
 *
 * The operation: y = x . W^T, with fp32 activations x [M, K] (row-major), fp32
 * output y [M, N] (row-major) and weights W [N, K] that stay in their packed,
 * weight-only quantized form in device memory and are dequantized inside the
 * GEMM ("RT-J - int4 (Q4-style, mixed-precision) quantized checkpoints",
 * opening paragraph): only the packed bytes cross the memory bus.
 *
 * Storage formats (the checkpoints' tensors, one payload plus one companion):
 *
 *   int4 ("RT-J - int4 ... quantized checkpoints", section "Quantization
 *   format"): uint4 codes in groups of 32 along the input dimension K.
 *     payload  uint8   [N][K/2]     byte j of row o holds code W[o][2j] in its
 *                                   low nibble and W[o][2j+1] in its high nibble
 *     pairs    float16 [N][K/32][2] per group: [0] = scale, [1] = min,
 *                                   passed as uint16_t bit patterns
 *     W[o][i] = code * scale + min   (evaluated in fp32; exact product, one rounding)
 *
 *   int8 ("RT-J - int8 (Q8_0-style) quantized checkpoints", section
 *   "Quantization format"): symmetric, one fp32 scale per output row.
 *     payload  int8    [N][K]
 *     scale    float32 [N]          scale[o] = max|W[o][:]| / 127
 *     W[o][i] = q[o][i] * scale[o]
 *
 *   FP8 E4M3 ("RT-J - FP8 E4M3 checkpoints", section "FP8 Format"): one
 *   float8_e4m3fn code per weight, no scale.
 *     codes    uint8   [N][K]       W[o][i] = the E4M3 value of codes[o][i]
 *
 * Conventions for every call below:
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never retains a caller's pointer past the call's work on its stream.
 *   - Memory and state of the library itself: a GEMM call on the split path
 *     with M above 32 (or a K other than 256, 512, 1024, 2048) takes one
 *     stream-ordered workspace (limb images of x, K-chunk partials) from a
 *     memory pool of the library's own (one per device, created on first
 *     use, kept for the process, releasing nothing back to the device), with
 *     hipMallocFromPoolAsync / hipFreeAsync on the caller's stream, so
 *     steady-state calls reuse pool memory without a driver allocation;
 *     smaller calls split x inside the GEMM kernel and allocate nothing. The
 *     device's default pool is not touched. The arithmetic is an argument of
 *     each call. Process-wide state: those pools and the timing events
 *     (rtq_timing_enable, a profiling aid); per thread: the last error message.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     selects the null stream). Nothing is synchronized. Faults during
 *     execution surface at the caller's next synchronization.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns its status and launches nothing. rtq_last_error() then holds a
 *     message naming the argument.
 *   - M == 0 is a no-op returning RTQ_OK. N >= 1 and K >= 1 are required;
 *     M, N, K must each be below 2^30 and M*N, M*K, N*K at most 2^38.
 *   - Base pointers must be 16-byte aligned (4-byte for scale / pair arrays).
 *   - The output must not overlap any input. Inputs may alias each other.
 *   - Launch failures return RTQ_ERR_HIP with the runtime's message copied
 *     into rtq_last_error().
 */
#ifndef RTQ_H_
#define RTQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rtq_status {
    RTQ_OK = 0,
    RTQ_ERR_NULL = 1,     /* a required pointer is NULL */
    RTQ_ERR_SHAPE = 2,    /* M/N/K (or n_blocks) out of range, K not a multiple of 32 for int4 */
    RTQ_ERR_ALIGN = 3,    /* a pointer is not aligned as required */
    RTQ_ERR_FORMAT = 4,   /* unknown format code in a block descriptor */
    RTQ_ERR_HIP = 5,      /* the HIP runtime reported an error */
    RTQ_ERR_OVERLAP = 6   /* the output range overlaps an input range */
} rtq_status;

#define RTQ_Q4_GROUP 32
#define RTQ_MAX_BLOCKS 64

enum { RTQ_FMT_NONE = 0, RTQ_FMT_Q4 = 1, RTQ_FMT_Q8 = 2, RTQ_FMT_F8 = 3 };

/* int4 projection: y[M][N] = x[M][K] . dequant(payload, pairs)^T.
 * K must be a multiple of 32 (the group size). */
rtq_status rtq_gemm_q4(const float* x, const uint8_t* payload, const uint16_t* pairs,
                       float* y, int64_t M, int64_t N, int64_t K, void* stream);

/* int8 projection: y[M][N] = x[M][K] . dequant(q, scale)^T. Any K >= 1. */
rtq_status rtq_gemm_q8(const float* x, const int8_t* q, const float* scale,
                       float* y, int64_t M, int64_t N, int64_t K, void* stream);

/* FP8 E4M3 projection: y[M][N] = x[M][K] . W^T with W[o][i] the E4M3 ("fn":
 * bias 7, subnormals, no infinities, S.1111.111 = NaN) value of the byte
 * codes[o][i], row-major [N][K], no scale ("RT-J - FP8 E4M3 checkpoints",
 * section "FP8 Format": 2-D weights kept in the float8_e4m3fn type, no scale).
 * Any K >= 1; codes must be 16-byte aligned. A NaN code makes its outputs NaN. */
rtq_status rtq_gemm_f8(const float* x, const uint8_t* codes, float* y,
                       int64_t M, int64_t N, int64_t K, void* stream);

/* One RT-J block's projections (names of the int4 card, section "Quantization
 * format"; the block count and widths of the "Backends" page, section "Meta").
 * fmt is RTQ_FMT_Q4, RTQ_FMT_Q8 or RTQ_FMT_F8 (so the mixed int4/int8 recipe,
 * the all-int8 recipe and the FP8 checkpoint are expressible); payload == NULL
 * skips the projection (for example a checkpoint without the attention gate
 * wg). `scale` is the pairs array for int4, the per-row scale for int8 and is
 * ignored (may be NULL) for FP8. Each projection reads its own
 * x [M][K] and writes its own y [M][N]; projections may share x.
 * `bias`, when not NULL, is an fp32 [N] vector (4-byte aligned) and the
 * projection computes y = x . W^T + bias, bias[o] added to column o of every
 * row: the checkpoints keep biases in fp32 beside the quantized matrices
 * ("RT-J - int4 (Q4-style, mixed-precision) quantized checkpoints", section
 * "Quantization format"). A bias is an input: no y may overlap it. */
typedef struct rtq_proj {
    int32_t fmt;
    int32_t N;
    int32_t K;
    int32_t reserved;          /* must be 0 */
    const void* payload;
    const void* scale;
    const float* x;
    float* y;
    const float* bias;         /* fp32 [N] added to every row of y, or NULL */
} rtq_proj;

typedef struct rtq_block {
    rtq_proj wq, wk, wv, wg, wo, w1, w3, w2;
} rtq_block;

/* Runs every projection of n_blocks blocks (1..RTQ_MAX_BLOCKS) at batch M in
 * as few grouped launches as the kernel-argument limit allows, on one stream.
 * `blocks` is a HOST array; it may be freed as soon as the call returns. The y
 * of one projection must not overlap any input or any other projection's y. */
rtq_status rtq_block_project(const rtq_block* blocks, int32_t n_blocks, int64_t M, void* stream);

/* Dequantize to a dense fp32 W [N][K], element by element, with the same
 * arithmetic the GEMM uses (bit-exact check of unpacking and dequantization). */
rtq_status rtq_dequant_q4(const uint8_t* payload, const uint16_t* pairs, float* w,
                          int64_t N, int64_t K, void* stream);
rtq_status rtq_dequant_q8(const int8_t* q, const float* scale, float* w,
                          int64_t N, int64_t K, void* stream);
rtq_status rtq_dequant_f8(const uint8_t* codes, float* w, int64_t N, int64_t K, void* stream);

/* Quantize a dense fp32 W [N][K] into the int4 format: per 32-group min-MSE
 * clip search over the shrink factors {1.00, 0.95, 0.90, 0.85, 0.80} applied
 * to both ends of the group range ("RT-J - int4 ... quantized checkpoints",
 * section "Quantization format"). Arithmetic in fp64, fp16 pair rounded to
 * nearest even, codes rounded half to even and clamped to 0..15; ties keep the
 * larger factor. Inputs must be finite with |W| <= 65504. */
rtq_status rtq_quantize_q4(const float* w, uint8_t* payload, uint16_t* pairs,
                           int64_t N, int64_t K, void* stream);

/* Quantize a dense fp32 W [N][K] into the int8 format: scale[o] =
 * max|W[o][:]| / 127 rounded to fp32, q = clamp(rint(W / scale), -127, 127)
 * (fp64 quotient, half to even); an all-zero row gets scale 0 and q 0
 * ("RT-J - int8 ... quantized checkpoints", section "Quantization format"). */
rtq_status rtq_quantize_q8(const float* w, int8_t* q, float* scale,
                           int64_t N, int64_t K, void* stream);

/* Encode a dense fp32 W [N][K] as FP8 E4M3 codes the way a cast to PyTorch's
 * float8_e4m3fn does ("RT-J - FP8 E4M3 checkpoints", section "FP8 Format"):
 * nearest E4M3 value, ties to the even code; magnitudes that round past 448,
 * infinities and NaN become NaN (0x7F with the input's sign). */
rtq_status rtq_quantize_f8(const float* w, uint8_t* codes, int64_t N, int64_t K, void* stream);

/* Host quantizers, for writing quantized checkpoints on a machine without a
 * GPU (the RT-J cards' offline quantizing tool, "rt_quantize --type q4 / q8"):
 * the same formats and the same arithmetic as rtq_quantize_q4 / _q8 / _f8
 * above, which they match bit for bit. Every pointer is a HOST pointer owned
 * by the caller; the call runs synchronously on the calling thread plus up to
 * threads - 1 worker threads (threads <= 0: one per hardware thread, at most
 * 1024), makes no HIP call and needs no GPU. Layouts, validation and
 * alignment as for the GPU quantizers; the arrays must not overlap. */
rtq_status rtq_quantize_q4_host(const float* w, uint8_t* payload, uint16_t* pairs,
                                int64_t N, int64_t K, int32_t threads);
rtq_status rtq_quantize_q8_host(const float* w, int8_t* q, float* scale,
                                int64_t N, int64_t K, int32_t threads);
rtq_status rtq_quantize_f8_host(const float* w, uint8_t* codes, int64_t N, int64_t K, int32_t threads);

/* Arithmetic of a GEMM call, chosen per call (the `math` argument of
 * rtq_gemm_ex and rtq_block_project_ex; rtq_gemm_q4 / _q8 / _f8 and
 * rtq_block_project run RTQ_MATH_SPLIT_BF16). No arithmetic state is kept
 * between calls.
 *
 * Range. The three split arithmetics form code sums (sum of code*x) before
 * the scale. Calls that take the pre-pass (M > 32, or any K other than 256,
 * 512, 1024, 2048) first scale each row of x by the power of two 2^e that puts
 * its largest magnitude in [2^14, 2^15) (exact, as is the scaling back of each
 * output row by 2^-e), so rows of any finite magnitude stay far inside fp32.
 * Calls that take the small-M direct kernel (M <= 32, every K one of 256, 512,
 * 1024, 2048, int4 pair arrays 16-byte aligned) split x unscaled: results meet
 * the parity bar for rows whose elements lie in [2^-100, 2^100] in magnitude;
 * far above that a row's code sums can overflow, and its outputs are then not
 * finite (never finite and wrong; other rows are unaffected). The fp32-MFMA
 * arithmetic multiplies the dequantized fp32 weights by x: an fp32 GEMM's
 * range on every route.
 *
 * RTQ_MATH_SPLIT_BF16: each activation (row-scaled where the route scales)
 *   is split exactly into three
 *   bf16 limbs (v = v1 + v2 + v3, no rounding); the int4/int8 codes and the
 *   E4M3 values are exact in bf16, so every code*limb product is exact in fp32
 *   and the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) accumulate them in
 *   fp32. Per 32-group: y += scale*sum(code*x) + min*sum(x) (int4),
 *   y = scale[o]*sum(q*x) (int8). Same accuracy class as an fp32 GEMM (fp32
 *   accumulation of exact products). Where rows are scaled, the scale is
 *   exact for every element whose scaled value stays a normal fp32 number
 *   (above 2^-126, i.e. more than 2^-140 of the row's largest magnitude);
 *   smaller ones lose low bits, far below the fp32 accumulation error.
 * RTQ_MATH_FP32_MFMA: the weights are dequantized to fp32 while staging and the
 *   fp32 matrix cores (v_mfma_f32_16x16x4_f32) run the contraction on the
 *   unscaled x.
 * Both satisfy the same parity bar against the fp64 reference.
 * RTQ_MATH_BF16: bf16 activations. Each x (row-scaled where the route
 *   scales) is rounded once to the
 *   nearest bf16 (ties to even) and takes the place of the three limbs:
 *   y = bf16(x) . W^T with the exact weight side and fp32 accumulation of the
 *   first mode, a third of its matrix work (the power-of-two scale does not
 *   change the rounding of a normal-range x). The result carries the rounding
 *   of x (about 2^-9 relative per element), so it is a lower-precision mode.
 * RTQ_MATH_SPLIT_F16: fp32 activations in two fp16 limbs: every row-scaled
 *   value v is split into h = fp16(v) and l = fp16(v - h), both rounded to nearest:
 *   h + l carries 22 significant bits of v (relative error at most 2^-22 per
 *   element, plus 2^-25 * 2^-e absolute for elements far below the row's
 *   largest). The fp16 matrix cores (v_mfma_f32_16x16x32_f16) run two limb
 *   products per code instead of three. Meets the same parity bar as
 *   RTQ_MATH_SPLIT_BF16 (relative Frobenius error 1e-5). Calls that take the
 *   small-M direct kernel (M <= 32, every K one of 256, 512, 1024, 2048, int4
 *   pair arrays 16-byte aligned) run the exact three-limb split there.
 * Shapes the split path does not take (int8/FP8 K not a multiple of 32, x or
 * payload not 16-byte aligned, N*K >= 2^32) run on the fp32 kernels in every
 * mode: correct, but several times slower than the split path (no error is
 * returned; keep shapes inside these conditions for the fast route). An
 * unknown mode returns RTQ_ERR_FORMAT. */
enum { RTQ_MATH_SPLIT_BF16 = 0, RTQ_MATH_FP32_MFMA = 1, RTQ_MATH_BF16 = 2, RTQ_MATH_SPLIT_F16 = 3 };

/* rtq_gemm_q4 / _q8 / _f8 with the format as an argument (fmt = RTQ_FMT_Q4,
 * RTQ_FMT_Q8 or RTQ_FMT_F8; `scale` is the int4 pairs, the int8 row scales,
 * ignored for FP8) and the arithmetic chosen by `math`. */
rtq_status rtq_gemm_ex(int32_t fmt, const float* x, const void* payload, const void* scale, float* y,
                       int64_t M, int64_t N, int64_t K, int32_t math, void* stream);

/* rtq_block_project with the arithmetic chosen by `math`. */
rtq_status rtq_block_project_ex(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math,
                                void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * rtq_block_project_ex that allocates nothing. Where the split path needs a
 * workspace (limb images of x and K-chunk partials: M above 32, or a K other
 * than 256, 512, 1024, 2048) it uses a fixed 32 MiB device array of the
 * library instead of its memory pool; each GPU the library runs on holds its
 * own copy of that array until the process ends. The call makes no
 * hipMalloc / hipFree or other allocating call. A call whose workspace would
 * exceed 32 MiB returns RTQ_ERR_SHAPE and launches nothing (the 12-block RT-J
 * projection set at M = 80 needs 22.1 MB with two fp16 limbs, 29.0 MB with
 * the exact split, 15.2 MB with bf16 activations). Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (each call writes all of what it reads): calls that
 * overlap in time on one GPU (different streams, or different host threads)
 * race on it and must be ordered by the caller. Results are those of
 * rtq_block_project_ex, bit for bit. */
rtq_status rtq_block_project_noalloc(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math,
                                     void* stream);

/* rtq_block_project_ex with a workspace the caller provides and keeps (the
 * usual pattern of BLAS libraries), for callers that run the same projection
 * set again and again: the library's own per-call workspace costs a
 * stream-ordered allocation and free (about 2 us per call on MI355X).
 *
 * rtq_block_workspace_bytes validates the call exactly as rtq_block_project_ex
 * would (same arguments, no stream) and stores in *bytes the workspace it
 * needs in arithmetic `math`: 0 when it runs no split-path launch that needs
 * one (M <= 32 with every K one of 256, 512, 1024, 2048 takes the direct
 * kernel; the fp32-MFMA arithmetic needs none). It launches nothing and makes
 * no HIP call.
 *
 * rtq_block_project_ws: `workspace` is a device buffer of `workspace_bytes`
 * bytes, 256-byte aligned, at least the size the query returns for the same
 * call (it may be NULL when that is 0), not overlapping any input or output
 * of the call; otherwise the call returns RTQ_ERR_SHAPE, RTQ_ERR_NULL,
 * RTQ_ERR_ALIGN or RTQ_ERR_OVERLAP and launches nothing. The library
 * allocates nothing and keeps no pointer to the workspace past the call's
 * work on `stream`. Calls that share one workspace must be ordered by the
 * caller (the same stream, or events between streams). Results are those of
 * rtq_block_project_ex, bit for bit. */
rtq_status rtq_block_workspace_bytes(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math,
                                     int64_t* bytes);
rtq_status rtq_block_project_ws(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* Kernel timing (profiling aid). While enabled, every main GEMM kernel launch
 * of the entry points above is bracketed by a pair of HIP events recorded on
 * its stream (events are created on first use and kept for reuse). Enabling
 * (or disabling) clears the record. rtq_timing_read waits for the recorded
 * events, returns the summed elapsed time in ms and the number of timed
 * launches, and clears the record. At most 16384 launches are recorded per
 * window; later ones are not timed. */
rtq_status rtq_timing_enable(int32_t on);
rtq_status rtq_timing_read(double* total_ms, int64_t* launches);

/* Diagnostics: the measured ceilings the kernels are compared with, beside
 * the published peaks. Both launch on `stream` and are timed by the caller
 * (events around the call). Neither writes anything the caller reads.
 *
 * rtq_diag_stream_read: reads `bytes` (a positive multiple of 16) of the
 * device buffer `buf` (16-byte aligned) with coalesced 16-byte loads, `unroll`
 * (4, 8 or 16) loads in flight per lane, over `blocks` workgroups of 256
 * threads striding over the buffer. `sink` is a device word the kernel writes
 * only in a case that does not arise (it keeps the loads live).
 *
 * rtq_diag_mfma_loop: `blocks` workgroups of four waves, each wave issuing
 * iters x 8 independent matrix instructions back to back: kind 0
 * v_mfma_f32_16x16x32_f16, 1 v_mfma_f32_16x16x32_bf16, 2
 * v_mfma_f32_16x16x4_f32. *flops (if not NULL) receives the floating-point
 * operations of the launch (2*16*16*32 or 2*16*16*4 per instruction). `sink`
 * as above. */
rtq_status rtq_diag_stream_read(const void* buf, int64_t bytes, int32_t unroll, int32_t blocks, uint32_t* sink,
                                void* stream);
rtq_status rtq_diag_mfma_loop(int32_t kind, int64_t iters, int32_t blocks, float* sink, double* flops,
                              void* stream);

const char* rtq_status_string(rtq_status status);
const char* rtq_last_error(void);   /* thread-local; valid until the next call on this thread */
const char* rtq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RTQ_H_ */
