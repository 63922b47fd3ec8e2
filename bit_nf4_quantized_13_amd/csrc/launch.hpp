// Host-side launchers of the HIP kernels (internal; the public surface is
// include/qlora_nf4.h).  All launchers enqueue on `stream` and return the
// hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.hpp"

namespace qnf4 {

const Nf4Consts &nf4_consts();  // built once on the host (nf4_table.cpp)

// ---- quantize (three kernels) --------------------------------------------
// fmt = kNoDq: the fp32 block absmax goes to c1 (one per block); c2 and mean are unused.
// block: 64, 128 or 256 weights (the blocks of 128 and 256 take a plain per-block kernel)
hipError_t launch_quantize(const float *W0, int64_t n, int block, uint8_t *codes, int8_t *c2, float *c1,
                           float *mean, float *absmax_ws, double *group_sum_ws, int fmt, hipStream_t s);

// ---- standalone double dequant --------------------------------------------
hipError_t launch_dequantize(const uint8_t *codes, const int8_t *c2, const float *c1,
                             const float *mean, int fmt, int bshift, int64_t n, uint16_t *out, hipStream_t s);

// ---- adapter dropout (dropout.hip) ----------------------------------------
// xd[M x k] = bf16(x c) where the Philox keep mask (threshold thr, 64-bit seed)
// keeps the element, +0 where it drops it; M k % 8 == 0, 16-byte aligned rows.
hipError_t launch_lora_dropout(const uint16_t *x, int64_t M, int64_t k, uint32_t thr, float c, uint64_t seed,
                               uint16_t *xd, hipStream_t st);
// dx[M x k] = bf16( base[m][n] + (kept ? sc (G A)[m][n] : 0) ), one rounding, with base [M x k]
// fp32, G [M x r] fp32 and A [r x k] bf16.
hipError_t launch_dropout_dx_add(const float *base, uint16_t *dx, int64_t M, int64_t k, const float *G, int r,
                                 const uint16_t *A, float sc, uint32_t thr, uint64_t seed, hipStream_t st);

// ---- skinny GEMMs ----------------------------------------------------------
// out[M x R] (fp32) = In[M x K] (bf16) * W[R x K]^T (bf16), R <= 128.  vt: null,
// or [2][Rp][M] bf16 receiving the transposed hi and lo planes of out (rows
// R..Rp-1 zero), Rp = cols_rank_pad(R).
int64_t cols_rank_pad(int r);
// part: rows_split_part_bytes(M, K, R) bytes of scratch for the partial sums
// of the wide-rank path (null when that is 0).
size_t rows_split_part_bytes(int64_t M, int64_t K, int R);
hipError_t launch_rows_skinny(const uint16_t *in, const uint16_t *w, int64_t M, int64_t K, int R,
                              float *out, uint16_t *vt, float *part, hipStream_t s);
// Backward preparation: Bt[r x d] = B[d x r]^T and, when U is given, the
// transposed hi / lo planes of U [M x r] into vt [2][Rp][M].
// G = dY B (r <= 16, M r > 4096, B 16-byte aligned) from B as stored, with U's
// planes when U is given: the backward preparation and rows_skinny in one launch
bool rows_bt_supported(int64_t M, int R, const void *B);
hipError_t launch_rows_bt(const uint16_t *dY, const uint16_t *B, int64_t M, int64_t d, int R, float *G, uint16_t *vt_g,
                          const float *U, uint16_t *vt_u, hipStream_t s);
// The wide-rank row products of launch_rows_skinny (r > 16, M >= 256) without
// their reduction: S partials [S][R][M] for launch_gemm_fwd to add.
bool rows_split_partials_used(int64_t M, int R);
hipError_t launch_rows_split_partials(const uint16_t *in, const uint16_t *w, int64_t M, int64_t K, int R, float *part,
                                      int *S, hipStream_t s);
hipError_t launch_bwd_prep(const uint16_t *B, int64_t d, int r, uint16_t *Bt, const float *U, int64_t M,
                           uint16_t *vt, hipStream_t s);
// Two column reductions in one launch (job 1 skipped when in1 is null):
// part_i[S][R][N_i] = split-M partial sums of V_i^T In_i (V_i given as vt_i),
// S = cols_splits(M).  The reduction out_i = scale_i * sum over splits, stored
// out_i[N_i x R] (trans_i = 0) or out_i[R x N_i] (trans_i = 1), is described by
// a ColsReduceJob and run by the next launch that takes one (the dX GEMM's
// preparation, or launch_cols_reduce).
int cols_splits(int64_t M);
struct ColsReduceJob {
    const float *part;
    int64_t N;
    int R, splits, trans;
    float scale;
    float *out;
};
hipError_t launch_cols_pair(const uint16_t *in0, const uint16_t *vt0, int64_t N0, float scale0, float *part0,
                            float *out0, int trans0, const uint16_t *in1, const uint16_t *vt1, int64_t N1,
                            float scale1, float *part1, float *out1, int trans1, int64_t M, int R,
                            ColsReduceJob *jobs, hipStream_t s);

// ---- measurement hook (qlora_time_next_kernel) -----------------------------
// The span buffer a benchmark asked the next launch of `kernel` to fill (null
// if none; the request is used once).  A kernel given one folds each
// workgroup's first and last s_memrealtime reading into span[0] (atomic min)
// and span[1] (atomic max).
enum TimedKernel : int { kTimeFwdGemm = 0, kTimeDxGemm = 1, kTimeDecode = 2, kTimedKernels = 3 };
unsigned long long *timing_take(int kernel);
__device__ __forceinline__ void span_start(unsigned long long *span) {
    if (span) __hip_atomic_fetch_min(span, (unsigned long long)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void span_end(unsigned long long *span) {
    if (span) __hip_atomic_fetch_max(span + 1, (unsigned long long)__builtin_amdgcn_s_memrealtime(),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- fused NF4 dequant GEMMs ----------------------------------------------
struct Nf4Weights {
    const uint8_t *codes;
    const int8_t *c2;
    const float *c1;    // double-quantized: c1 per group of 256 blocks; else the fp32 absmax per block
    const float *mean;  // double-quantized only
    int64_t d, k;
    int fmt;            // ScaleFormat (common.hpp): kNoDq, kDqInt8 or kDqFp8
    int bshift;         // blocks of 64 << bshift weights (0, 1, 2: 64, 128, 256)
};
// Workspace of one dequant-GEMM call: the dequantized block scales
// (d*k/64 floats) and the adapter operands laid out as extra k-columns,
// ext_a [M x Ke] and ext_b [N x Ke] bf16 with Ke = gemm_ext_cols(r).
// wbf: dequantized bf16 copy of the weight operand, used when the output has
// more than one 512-row tile row (gemm_wbf_elems(M, d, k) elements, else 0).
struct GemmWs {
    float *shat;
    uint16_t *ext_a;
    uint16_t *ext_b;
    uint16_t *wbf;
    float *kpart;          // split-K partial sums (gemm_ksplit_bytes)
    size_t kpart_bytes;
};
int64_t gemm_ext_cols(int r);
// Bytes of fp32 partial sums the GEMMs of an M-row call split over K need (the
// larger of the forward's and dX's; 0 when neither splits): grids that leave
// most CUs idle (M <= 512 expands the weight tiles in 512 x 128 tiles, one tile
// row) take their k-steps in up to 8 slices.  At most 64 MiB.
size_t gemm_ksplit_bytes(int64_t M, int64_t d, int64_t k);
int64_t gemm_wbf_elems(int64_t M, int64_t d, int64_t k);
// Y[M x d] = bf16( X[M x k] What^T + [hi(sU) | lo(sU)] [B | B]^T ),  U [M x r] fp32.
// Upart (U null): U's S partial sums [S][r][M] of rows_split, added in slice
// order by the preparation launch (the additions of rows_reduce), which also
// stores U into Uout [M x r].
hipError_t launch_gemm_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const float *U,
                           const uint16_t *B, int r, float s, uint16_t *Y, const GemmWs &ws,
                           hipStream_t st, const float *Upart = nullptr, int Us = 0, float *Uout = nullptr);
// dX[M x k] = bf16( dY[M x d] What + [hi(sG) | lo(sG)] [A ; A] ),  G [M x r] fp32
// red: null, or two column reductions (ColsReduceJob) to run in the same
// preparation launch; launch_cols_reduce runs them alone.  dX_f32: null, or
// [M x k] fp32 receiving the unrounded sums instead of dX.
hipError_t launch_cols_reduce(const ColsReduceJob *red, hipStream_t st);
hipError_t launch_gemm_dx(const Nf4Weights &w, const uint16_t *dy, int64_t M, const float *G,
                          const uint16_t *A, int r, float s, uint16_t *dX, const GemmWs &ws,
                          const ColsReduceJob *red, hipStream_t st, float *dX_f32 = nullptr);

// The GEMM kernel of launch_gemm_fwd (dx = false) or launch_gemm_dx (dx = true)
// alone, on a workspace that a full launch with the same arguments prepared;
// force_expand: the block scales and the expanding kernel instead, at any M
// (measurement of the expanding path against the bf16 copy).
hipError_t launch_gemm_core(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, int r, uint16_t *out,
                            const GemmWs &ws, hipStream_t st, bool force_expand = false);

// Adapter merge / unmerge: w_out[d x k] = bf16(fp32(base + s * (B A))) with the
// sum over ranks in fp64, j ascending; base = doubleDequant(w) when w is not
// null (merge), else w_in (unmerge, s negated by the caller; w_in may be w_out).
// k % 8 == 0; no workspace.
hipError_t launch_adapter_merge(const Nf4Weights *w, const uint16_t *w_in, int64_t d, int64_t k, const uint16_t *A,
                                const uint16_t *B, int r, double s, uint16_t *w_out, hipStream_t st);

// Decode-shaped forward, M <= 16: Y = X What^T + s U B^T.  U [M x r] fp32 is
// either given (U != null) or computed in the same kernel from A [r x k]
// (U == null, r <= 16; written to U_save when that is not null).  part holds
// decode_part_bytes(M, d, k) bytes of partial sums; ctr points at
// decode_counter_bytes() bytes of counters that no other kernel writes (the
// kernel tags them on first use and leaves them ready for the next call).
// Forwards of up to kDecodeChunkRows rows run it on consecutive 16-row chunks
// of X (one launch each, sharing part and ctr in stream order): the weight is
// streamed once per chunk, which beats the GEMM (64-row tiles, split K) for
// two chunks (4096 x 4096: 17.8-18.5 us against 22.7-22.9 for 17-32 rows;
// 14336 x 4096: 29-31 against 42.5) but not for three.
constexpr int64_t kDecodeChunkRows = 32;
size_t decode_counter_bytes();
size_t decode_part_bytes(int64_t M, int64_t d, int64_t k);
hipError_t launch_decode_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const uint16_t *A, const float *U,
                             const uint16_t *B, int r, float s, uint16_t *Y, float *U_save, float *part,
                             unsigned long long *ctr, hipStream_t st);
// The same for M <= 2, r <= 16, k <= 4096, d >= 8192, U computed from A, on
// packed dot products (decode_dot.hip); launch_decode_fwd takes this path
// whenever decode_dot_supported holds.  span: the measurement span or null.
bool decode_dot_supported(int64_t M, int64_t d, int64_t k, int r);
hipError_t launch_decode_dot(const Nf4Weights &w, const uint16_t *x, int64_t M, const uint16_t *A, const uint16_t *B,
                             int r, float s, uint16_t *Y, float *U_save, unsigned long long *span, hipStream_t st);

}  // namespace qnf4
