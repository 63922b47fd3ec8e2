/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA NF4 linear-layer library.
 *
 * One QLoRA linear layer: a frozen base weight W0 [d x k] stored as blockwise
 * 4-bit NormalFloat (NF4) with double-quantized block constants, plus a
 * trainable low-rank adapter:
 *
 *     h = W0 x + (alpha / r) B (A x)          x in R^k, A [r x k], B [d x r]
 *
 * (fromzero2ai.dev "LoRA and QLoRA", sections "Linear Layer Deconstruction"
 * and "Low-Rank Matrix Factorization"; chkda.github.io "Why do we need LoRA
 * and QLoRA?", "How does it work?".)  Rows of X [M x k] are the inputs, so
 * the batched form is Y = X What^T + s (X A^T) B^T with s = alpha / r and What
 * the bf16 weights recovered by doubleDequant (chkda, "Double quantization
 * and double dequantization").  No bias term.
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers, allocated, owned and freed by
 *     the caller; the library never allocates, frees or keeps a pointer past
 *     the call (the one exception is the measurement-only
 *     qlora_time_next_kernel, which holds its span buffer until the next
 *     launch of the kernel it names).  Matrices are dense and row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; the library never synchronises.
 *   - Outputs are overwritten, never accumulated; outputs must not alias
 *     inputs or each other.
 *   - bf16 values are passed as their raw 16-bit patterns (qlora_bf16).
 *   - Every argument is validated before anything is launched: a call that
 *     returns an error other than QLORA_EHIP has no device side effects.
 *   - Inputs are assumed finite; NaN or Inf in W0, x, A, B or dY gives
 *     undefined (but memory-safe) results.
 *   - Calls are reentrant: the library holds no mutable global state (the
 *     NF4 table is computed once, on first use, behind a thread-safe
 *     initialiser; qlora_linear_fwd_noalloc keeps the device address of its
 *     static scratch per device; a pending qlora_time_next_kernel request is
 *     process-wide, behind a mutex).  Calls that share a workspace must be
 *     ordered on one stream.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QLORA_OK          0  /* success                                                  */
#define QLORA_EINVAL      1  /* null pointer, size <= 0, k % block != 0, non-finite alpha */
#define QLORA_ENOTSUP     2  /* block not 64/128/256, dq_block not 256 or 0, c2_format,
                                r > 128, d k > 2^30 weights, a linear call's sizes beyond
                                those listed at qlora_linear_workspace                 */
#define QLORA_EALIGN      3  /* a pointer read/written with 128-bit accesses is not 16-byte aligned */
#define QLORA_EWORKSPACE  4  /* workspace NULL or smaller than the *_workspace() size     */
#define QLORA_EHIP        5  /* a HIP launch or runtime error (hipGetLastError)          */
#define QLORA_ESCRATCH    6  /* qlora_linear_fwd_noalloc: M > 16, or the call's scratch
                                exceeds the library's static maximum (8 MiB)           */

#define QLORA_NF4_BLOCK     64   /* weights per NF4 block (chkda, "Quantizing and dequantizing with the codebook") */
#define QLORA_NF4_DQ_BLOCK  256  /* block constants per second-level group (chkda, "Double quantization ...")   */
#define QLORA_NF4_NO_DQ     0    /* dq_block value of the format without double quantization: one fp32
                                    absmax per block (chkda, the bits-per-weight accounting after
                                    "Double quantization and double dequantization": 4.5 bits/weight) */
#define QLORA_C2_INT8       0    /* c2_format: c2 as int8, Int8 absmax rule (127)                        */
#define QLORA_C2_FP8_E4M3   1    /* c2_format: c2 as OCP FP8 e4m3 bytes (the "c2_FP8" of chkda's
                                    doubleDequant(c1_FP32, c2_FP8, W_NF4)), absmax rule with 448    */
#define QLORA_MAX_RANK      128

typedef uint16_t qlora_bf16; /* raw bfloat16 bits */

/*
 * The stored form of W0 (chkda, "Double quantization and double
 * dequantization": W_NF4 codes in blocks of 64, the quantized block
 * constants c2 in groups of 256, one fp32 second-level scale c1 per group,
 * and the mean subtracted before quantizing the constants).  All pointers
 * are device memory owned by the caller.  With N = d*k, nb = N/64 and
 * G = ceil(nb/256):
 *   codes        uint8 [N/2]  byte t = code[2t] | code[2t+1] << 4, codes in
 *                             row-major order of W0 (16-byte aligned)
 *   absmax_q     int8  [nb]   c2, in [-127, 127]
 *   absmax_scale float [G]    c1 (4-byte aligned)
 *   absmax_mean  float [1]    the mean of the nb block absmax values
 *   d, k                      W0 shape, d >= 1, k >= 1, k % block == 0
 *   block, dq_block           block: 64 (the pages' size), 128 or 256 weights,
 *                             nb = N / block, k % block == 0; dq_block: 256
 *                             (or QLORA_NF4_NO_DQ, below).  The kernels work
 *                             on 64-weight sub-blocks; sub-block j takes the
 *                             constants of block j / (block / 64)
 *   c2_format                 QLORA_C2_INT8 (0) or QLORA_C2_FP8_E4M3: how the
 *                             c2 bytes encode their values (ignored without
 *                             double quantization)
 * With QLORA_C2_FP8_E4M3 each c2 byte is an OCP FP8 e4m3 value (sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest finite 448) read
 * exactly as fp32, and c1 = 448 / max|s - mean| per group.
 * With dq_block == QLORA_NF4_NO_DQ the block constants are not double
 * quantized (the "before" format of the same page's bits-per-weight
 * accounting): absmax_scale holds the fp32 absmax of each block, [nb]
 * entries, the block's own scale; absmax_q and absmax_mean are neither read
 * nor written and may be NULL.  Every call below takes either format.
 */
typedef struct {
    uint8_t *codes;
    int8_t  *absmax_q;
    float   *absmax_scale;
    float   *absmax_mean;
    int64_t  d, k;
    int32_t  block, dq_block;
    int32_t  c2_format;
} qlora_nf4_weight;

/* Bytes of device workspace qlora_nf4_quantize needs for this shape
 * (0 for invalid arguments). */
size_t qlora_nf4_quantize_workspace(int64_t d, int64_t k, int32_t block, int32_t dq_block);

/*
 * qlora_nf4_quantize -- NF4 + double quantization of W0.
 * chkda, "Quantizing and dequantizing with the codebook": per block of 64
 * (row-major flattening) scale = max|w|, each w/scale goes to the nearest of
 * the 16 NF4 levels (ties to the smaller index; an all-zero block gets the
 * exact-zero level); "Double quantization and double dequantization" with the
 * Int8 absmax rule of "First, how does k-bit quantization work?": the block
 * scales minus their mean are quantized to int8 per group of 256 with
 * c1 = 127 / max|s - mean| (a zero group stores zeros and c1 = 127).  With
 * c2_format == QLORA_C2_FP8_E4M3: c1 = 448 / max|s - mean| (448 for a zero
 * group) and c2 = e4m3(fp32(c1 (s - mean))), round to nearest, ties to the
 * even code.
 *   W0  device fp32 [d x k], 16-byte aligned, read only.
 *   w   host struct: shape fields and the four output arrays (all written;
 *       without double quantization only codes and the per-block absmax).
 *   ws  device workspace of >= qlora_nf4_quantize_workspace(...) bytes,
 *       16-byte aligned; its contents on entry are ignored.
 * The result is bit-identical on every run (fixed-order fp64 mean).
 */
int qlora_nf4_quantize(const float *W0, const qlora_nf4_weight *w,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_nf4_dequantize -- doubleDequant into a dense bf16 matrix.
 * chkda, "Double quantization and double dequantization":
 *   scale[j] = fp32(c2[j] / c1[j/256]) + mean          (IEEE fp32 ops; c2[j]
 *                                                       its int8 or e4m3 value)
 *   W[i]     = BF16(C[code[i]] * scale[i/64])          (one RNE rounding)
 * (without double quantization scale[j] is the stored fp32 absmax of block j).
 *   W_out  device bf16 [d x k], 16-byte aligned, written.
 */
int qlora_nf4_dequantize(const qlora_nf4_weight *w, qlora_bf16 *W_out, void *stream);

/* Bytes of device workspace qlora_linear_fwd / qlora_linear_bwd need for
 * these sizes (the same figure serves both calls; 0 for invalid arguments).
 * Sizes every linear call (fwd, bwd, their dropout forms, gemm_only)
 * supports, else QLORA_ENOTSUP (0 here): d % 8 == 0 (each bf16 row of Y and
 * dY [M x d] starts 16-byte aligned; k % 64 == 0 already holds for X and
 * dX); d, k <= 2^20; M k, M d and d k at most 2^30 elements; M r16 <= 2^29
 * with r16 = r rounded up to 16.  Each operand is addressed with 32-bit byte
 * offsets inside the kernels. */
size_t qlora_linear_workspace(int64_t M, int64_t d, int64_t k, int32_t r);

/*
 * qlora_linear_fwd -- Y = X What^T + (alpha/r) (X A^T) B^T.
 * chkda, "Double quantization and double dequantization" (the full QLoRA
 * expression, Y = X doubleDequant(c1, c2, W_NF4) + X L1 L2 with L1 = A^T,
 * L2 = B^T and the scale alpha/r of "How does alpha/r control adapter
 * strength?").  Products accumulate in fp32.  For 16 < M <= 512 the GEMM
 * expands What from the NF4 codes tile by tile; for M > 512 the call first
 * writes a bf16 copy of What (2 d k bytes of the workspace) and the GEMM
 * streams it (faster there than expanding every weight tile once per 512
 * rows of X); both bit-identical to qlora_nf4_dequantize.  Where the
 * output tiles alone would leave most of the GPU idle (e.g. M <= 512 against
 * a few thousand columns), the GEMM's k-steps run in up to 8 slices whose
 * fp32 partial sums (up to 64 MiB of the workspace) are added in slice order
 * before the one rounding to bf16: the sum is associated differently from an
 * unsplit call, deterministically.  For M <= 16 (decode; M <= 32 as
 * consecutive 16-row chunks of X, one decode launch each, the same bits as
 * separate calls on the chunks) the 64-weight block scale is applied once to
 * the fp32 sum over the block (over each half block with M <= 2, r <= 16,
 * k <= 4096 and d >= 8192, which take a vector dot-product kernel), with the
 * NF4 levels in bf16: the same product, rounded differently (within the
 * library's fwd tolerance of the bf16 What product).
 * A call with M <= 16 and r <= 16 is one kernel (U = X A^T included); it
 * keeps counters in the first 32 KiB of the workspace between calls, which
 * it tags and resets itself: the caller need not clear them, but must not
 * write into that region between calls.
 *   x      device bf16 [M x k], 16-byte aligned
 *   A      device bf16 [r x k], 16-byte aligned;  B device bf16 [d x r]
 *   r      1..128; alpha finite
 *   Y      device bf16 [M x d], written
 *   U_save device fp32 [M x r] or NULL: if given, receives U = X A^T (the
 *          adapter's inner activation, needed by the backward)
 *   ws     device workspace of >= qlora_linear_workspace(M, d, k, r) bytes.
 */
int qlora_linear_fwd(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M,
                     const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha,
                     qlora_bf16 *Y, float *U_save, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_fwd_noalloc -- qlora_linear_fwd for decode-shaped calls
 * (M <= 16) that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It runs the kernels of
 * qlora_linear_fwd's M <= 16 path and gives the same bits.  Their device
 * memory (the decode kernel's counters and partial sums and, for r > 16, U)
 * is a static array of 8 MiB that the library holds on every GPU it runs on
 * until the process ends; a call whose needs exceed it returns
 * QLORA_ESCRATCH, as does M > 16.  Arguments as for qlora_linear_fwd, without
 * ws and ws_bytes; the current device must be the device of `stream`.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race and
 * may return wrong results.  The array keeps the last call's counters, which
 * the kernel tags on first use and leaves ready for the next call (nothing
 * needs clearing between calls).
 */
int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M,
                             const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha,
                             qlora_bf16 *Y, float *U_save, void *stream);

/*
 * qlora_linear_bwd -- gradients of the layer for an upstream gradient dY.
 * chkda, "Double quantization and double dequantization": backpropagation
 * runs through the reconstructed base weights into the adapters only; the
 * 4-bit weights get no gradient.  With s = alpha/r, U = X A^T, G = dY B:
 *   dX = dY What + s G A        dA = s G^T X        dB = s dY^T U
 *   x   device bf16 [M x k];  dY device bf16 [M x d] (16-byte aligned)
 *   A, B, r, alpha as in qlora_linear_fwd
 *   U   device fp32 [M x r] from qlora_linear_fwd's U_save, or NULL to
 *       recompute it
 *   dX  device bf16 [M x k], written; or NULL to skip the input gradient
 *   dA  device fp32 [r x k], written;  dB device fp32 [d x r], written
 *   ws  device workspace of >= qlora_linear_workspace(M, d, k, r) bytes.
 * Reductions over M run in a fixed order: results are bit-identical on
 * every run.  With r <= 16 and B 16-byte aligned, G is formed from B as
 * stored in one launch (otherwise B is first copied transposed into the
 * workspace); both give the same bits.
 */
int qlora_linear_bwd(const qlora_nf4_weight *w, const qlora_bf16 *x, const qlora_bf16 *dY,
                     const qlora_bf16 *A, const qlora_bf16 *B, const float *U,
                     int64_t M, int32_t r, float alpha,
                     qlora_bf16 *dX, float *dA, float *dB,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Adapter dropout (fromzero2ai "LoRA and QLoRA", "Python Implementation:
 * Fine-Tuning with PEFT and BitsAndBytes": training with a LoRA dropout rate;
 * chkda "Merging LoRA weights for inference": the two-path layer equals the
 * merged one only with dropout disabled).  Dropout acts on the adapter's input
 * only:  Xd = drop(X),  U = Xd A^T,  Y = X What^T + s U B^T,
 *        dA = s G^T Xd,  dB = s dY^T U,  dX = dY What + c (Mask o (s G A)),
 * with c = fp32(1 / fp32(1 - p)).  The keep mask is Philox4x32-10 (Salmon et
 * al., "Parallel random numbers: as easy as 1, 2, 3", SC 2011): element
 * i = m k + col of X [M x k] uses word i mod 4 of the block for counter
 * (i div 4 low word, i div 4 high word, 0, 0) and key (seed low, seed high),
 * and is dropped iff that word < floor(p 2^32) (p is its fp32 value; the
 * realised rate is floor(p 2^32) / 2^32).  The same (p, seed) in the
 * forward and the backward gives the same mask; nothing is stored.
 *   p     dropout probability, 0 <= p < 1 (p = 0: the calls without dropout
 *         give the same results); seed any 64-bit value.
 */

/*
 * qlora_lora_dropout -- Xd = drop(X) alone:  Xd[m][c] = BF16(fp32(x c))
 * (round to nearest even) where kept, +0 where dropped.
 *   x, xd  device bf16 [M x k], 16-byte aligned, k % 8 == 0; may not overlap.
 */
int qlora_lora_dropout(const qlora_bf16 *x, int64_t M, int64_t k, float p, uint64_t seed,
                       qlora_bf16 *xd, void *stream);

/* Bytes of device workspace the two dropout calls need (a linear workspace
 * plus room for Xd [M x k] bf16 and the backward's fp32 dX sums [M x k]); 0
 * for invalid arguments. */
size_t qlora_linear_dropout_workspace(int64_t M, int64_t d, int64_t k, int32_t r);

/*
 * qlora_linear_fwd_dropout -- qlora_linear_fwd with dropout on the adapter
 * input.  Arguments as qlora_linear_fwd plus p and seed; U_save receives
 * U = Xd A^T, the value qlora_linear_bwd_dropout takes as U.
 *   ws  >= qlora_linear_dropout_workspace(M, d, k, r) bytes.
 */
int qlora_linear_fwd_dropout(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M,
                             const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha,
                             float p, uint64_t seed, qlora_bf16 *Y, float *U_save,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_bwd_dropout -- qlora_linear_bwd with dropout on the adapter
 * input, for the forward with the same p and seed.  Arguments as
 * qlora_linear_bwd plus p and seed (U: that forward's U_save, or NULL to
 * recompute it).  dX: the base term dY What and the masked adapter term are
 * added in fp32 and the sum is rounded once to bf16.
 *   ws  >= qlora_linear_dropout_workspace(M, d, k, r) bytes.
 */
int qlora_linear_bwd_dropout(const qlora_nf4_weight *w, const qlora_bf16 *x, const qlora_bf16 *dY,
                             const qlora_bf16 *A, const qlora_bf16 *B, const float *U,
                             int64_t M, int32_t r, float alpha, float p, uint64_t seed,
                             qlora_bf16 *dX, float *dA, float *dB,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_linear_gemm_only -- measurement only (benchmarks; not part of the
 * layer's computation): the dequant-GEMM kernel of the preceding
 * qlora_linear_fwd (backward = 0) or qlora_linear_bwd (backward = 1) call,
 * launched alone, so that its duration can be measured in isolation.  Those
 * calls first run small preparation kernels (U = X A^T or G = dY B, the
 * dequantized block scales, the adapter operands laid out as extra k-columns,
 * a bf16 copy of What when M > 512) into the workspace and then one GEMM
 * kernel; this call re-runs only the GEMM on that prepared workspace.
 *   expand  0: the kernel the call ran.  1: the block scales and the GEMM
 *           kernel that expands What from the NF4 codes tile by tile (the one
 *           the calls use for M <= 512), at any M, on the adapter operands the
 *           call prepared -- the two ways of feeding the weights, side by side.
 *   a    the call's x (forward) or dY (backward); M, r, ws as in that call
 *   out  rewritten with the values the call wrote to Y (forward) or dX
 *        (backward): both kernels give the same bits
 * The workspace must not have been used by another call in between.  A
 * forward with M <= 16 has no separate GEMM (one kernel): QLORA_EINVAL.
 */
int qlora_linear_gemm_only(const qlora_nf4_weight *w, int32_t backward, int32_t expand, const qlora_bf16 *a,
                           int64_t M, int32_t r, qlora_bf16 *out, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_time_next_kernel -- measurement only (benchmarks): the next launch of
 * the named kernel records its own execution span, so that the kernel's
 * duration can be read while it runs inside ordinary calls.  kernel: 0 the
 * forward dequant-GEMM (qlora_linear_fwd with M > 16), 1 the dX dequant-GEMM
 * (qlora_linear_bwd), 2 the decode kernel (qlora_linear_fwd with M <= 16).
 * span: device memory, two uint64 holding {UINT64_MAX, 0} beforehand; each
 * workgroup of that launch folds the constant-rate clock (s_memrealtime) at
 * its start into span[0] (atomic min) and after its last store into span[1]
 * (atomic max), so span[1] - span[0] ticks is the launch's duration
 * (qlora_wall_clock_khz gives the tick rate).  The request is used once;
 * NULL cancels a pending one.  It is process-wide: no other thread may launch
 * that kernel meanwhile.
 * Errors: QLORA_EINVAL (unknown kernel), QLORA_EALIGN (span not 8-byte
 * aligned).
 */
int qlora_time_next_kernel(int32_t kernel, uint64_t *span);

/* Measurement only: the rate of the clock qlora_time_next_kernel reads, in
 * kHz, on the current device (hipDeviceAttributeWallClockRate).  QLORA_EHIP
 * without a device. */
int qlora_wall_clock_khz(int32_t *khz);


/*
 * qlora_adapter_merge -- fold the adapter into a dense bf16 weight.
 * chkda, "Merging LoRA weights for inference": W_merged = W0 + (alpha/r) B A,
 * with W0 the double-dequantized What of the NF4 weight ("Double quantization
 * and double dequantization").  The arithmetic is fixed so that the result is
 * reproducible bit for bit:
 *   S[n][k]      = sum over j = 0 .. r-1, ascending, of B[n][j] * A[j][k], in
 *                  fp64 (each product of two bf16 values is exact in fp64)
 *   W_out[n][k]  = BF16( What[n][k] + s * S[n][k] ),  s = fp32(alpha / r)
 * where s * S and the sum are separate fp64 roundings and the fp64 result is
 * rounded once to the nearest bf16 (ties to even).  To requantize the merged
 * weight, widen W_out to fp32 and call qlora_nf4_quantize.
 *   w      the NF4 weight (as for qlora_nf4_dequantize).
 *   A      device bf16 [r x k], 16-byte aligned;  B  device bf16 [d x r].
 *   W_out  device bf16 [d x k], 16-byte aligned, written.  No workspace.
 * Errors: QLORA_EINVAL (null pointer, r <= 0, non-finite alpha), QLORA_ENOTSUP
 * (r > 128, weight format), QLORA_EALIGN.
 */
int qlora_adapter_merge(const qlora_nf4_weight *w, const qlora_bf16 *A, const qlora_bf16 *B, int32_t r,
                        float alpha, qlora_bf16 *W_out, void *stream);

/*
 * qlora_adapter_unmerge -- take an adapter back out of a merged bf16 weight
 * (chkda, "Merging LoRA weights for inference": keeping base and adapters apart
 * lets one switch adapters):
 *   W_out[n][k] = BF16( W_in[n][k] - s * S[n][k] )   (one rounding, as for the merge)
 * with S and s as in qlora_adapter_merge.  unmerge(merge(What)) recovers What
 * up to the two bf16 roundings: half an ulp of the merged value plus half an
 * ulp of the result, per element.
 *   W_in   device bf16 [d x k], 16-byte aligned; may equal W_out (in place).
 *   k % 8 == 0.  Errors as for qlora_adapter_merge.
 */
int qlora_adapter_unmerge(const qlora_bf16 *W_in, int64_t d, int64_t k, const qlora_bf16 *A, const qlora_bf16 *B,
                          int32_t r, float alpha, qlora_bf16 *W_out, void *stream);

/*
 * qlora_nf4_codebook -- host-only: copies the library's 16 fp32 NF4 levels
 * (chkda, "NF4: Choose the codebook to fit the distribution"; built as in
 * "Building the NF4 codebook" from standard-normal quantiles) into out[16].
 * Needs no GPU.
 */
int qlora_nf4_codebook(float out[16]);

/*
 * qlora_nf4_thresholds -- host-only: the 15 fp32 decision thresholds T_j used
 * by the quantizer; x goes to level j+1 or above iff fp32 x >= T_j, where
 * T_j is the smallest fp32 strictly above the exact midpoint of levels j and
 * j+1 (chkda: nearest level, ties to the smaller index).  Needs no GPU.
 */
int qlora_nf4_thresholds(float out[15]);

/* Static description of a status code (never NULL). */
const char *qlora_status_str(int status);

/* ABI version of this header/library pair. */
int qlora_abi_version(void);
#define QLORA_ABI_VERSION 6

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
