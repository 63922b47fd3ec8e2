// Merging the trained adapter into the weight, and taking it out again:
//   merge:    W_out = bf16( What + s S )      What = doubleDequant(W_NF4)
//   unmerge:  W_out = bf16( W_in - s S )      W_in bf16, may be W_out
// with S[n][k] = sum_j B[n][j] A[j][k] and s = alpha / r.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Merging LoRA weights for
// inference": once training is done, W_merged = W0 + (alpha/r) B A has the
// shape of W0 and replaces the two-path forward; with the NF4 base, W0 is the
// double-dequantized What of "Double quantization and double dequantization".
// The page leaves the merge's arithmetic open (it notes that floating point
// can introduce small differences); here it is fixed so that a merge is
// reproducible bit for bit: S in fp64 with j ascending -- a bf16 x bf16
// product is exact in fp64, so each step is one fp64 FMA, i.e. one rounding
// of the exact product added to S -- then s S and the add as two fp64
// roundings, then one rounding of that fp64 value to the nearest bf16 (ties
// to even).  The narrowing goes through fp32 rounded to odd (truncate, then set
// the last bit if anything was dropped): with 24 >= 8 + 2 significant bits the
// following fp32 -> bf16 round to nearest even then rounds the fp64 value
// itself, where a plain fp64 -> fp32 -> bf16 chain could round twice.
//
// Bound: r fp64 FMAs per weight against 2.5 bytes of HBM traffic (merge:
// 0.5 + 1/64 code and constant bytes read, 2 written), so fp64 ALU for large
// r and HBM for small.  A workgroup takes a 64-row x 256-column tile; the A
// and B entries of 32 ranks at a time sit in LDS (bf16), and each thread
// accumulates an 8 x 8 block of S in 64 fp64 registers.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int kMRows = 64, kMCols = 256, kMRanks = 32;

template <bool NF4>  // NF4: merge from the packed weight; else unmerge from bf16 W_in
__global__ __launch_bounds__(256) void adapter_merge_kernel(const uint8_t *__restrict__ codes,
                                                            const int8_t *__restrict__ c2,
                                                            const float *__restrict__ c1,
                                                            const float *__restrict__ mean_p, int fmt, int bshift,
                                                            const uint16_t *__restrict__ w_in,
                                                            const uint16_t *__restrict__ A,
                                                            const uint16_t *__restrict__ B, int64_t d,
                                                            int64_t k, int r, double s, Nf4Consts tab,
                                                            uint16_t *w_out) {
    __shared__ __attribute__((aligned(16))) uint16_t a_s[kMRanks][kMCols];  // A[j0 + jj][c0 ..]
    __shared__ __attribute__((aligned(16))) uint16_t b_s[kMRanks][kMRows];  // B[r0 ..][j0 + jj], transposed
    __shared__ float lut[16];
    const int tid = threadIdx.x;
    const int64_t tiles_c = (k + kMCols - 1) / kMCols;
    const int64_t r0 = ((int64_t)blockIdx.x / tiles_c) * kMRows, c0 = ((int64_t)blockIdx.x % tiles_c) * kMCols;
    const int ng = tid & 7, kg = tid >> 3;
    const int64_t n0 = r0 + 8 * ng;  // this thread's rows n0 .. n0 + 7
    const __amdgpu_buffer_rsrc_t rout = out_rsrc(w_out, d * k * 2);
    const int64_t k0 = c0 + 8 * kg;  // and columns k0 .. k0 + 7 (k % 8 == 0: all in or all out)
    if (tid < 16) lut[tid] = tab.level[tid];

    double acc[8][8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[e][c] = 0.0;

    for (int j0 = 0; j0 < r; j0 += kMRanks) {
        __syncthreads();  // the previous chunk is consumed
        // A rows j0 .. j0 + 31 over the tile's columns: 16 bytes per thread and row
#pragma unroll
        for (int u = 0; u < kMRanks * kMCols / 8 / 256; ++u) {
            const int e = tid + 256 * u;  // (jj, 8-column group)
            const int jj = e / (kMCols / 8), cg = e % (kMCols / 8);
            const int64_t col = c0 + 8 * cg;
            uint4 v{0, 0, 0, 0};
            if (j0 + jj < r && col < k) v = *reinterpret_cast<const uint4 *>(A + (int64_t)(j0 + jj) * k + col);
            *reinterpret_cast<uint4 *>(&a_s[jj][8 * cg]) = v;
        }
        // B rows of the tile over ranks j0 .. j0 + 31, stored transposed
#pragma unroll
        for (int u = 0; u < kMRanks * kMRows / 256; ++u) {
            const int e = tid + 256 * u;  // (row, jj), jj fastest
            const int row = e / kMRanks, jj = e % kMRanks;
            const int64_t n = r0 + row;
            b_s[jj][row] = (n < d && j0 + jj < r) ? B[n * r + j0 + jj] : (uint16_t)0;
        }
        __syncthreads();
        // ranks in ascending order, this chunk's only (the zero-filled entries past r
        // are not visited)
        const int nj = r - j0 < kMRanks ? r - j0 : kMRanks;
        for (int jj = 0; jj < nj; ++jj) {
            const uint4 av = *reinterpret_cast<const uint4 *>(&a_s[jj][8 * kg]);
            const uint4 bv = *reinterpret_cast<const uint4 *>(&b_s[jj][8 * ng]);
            const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
            double ad[8], bd[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                ad[2 * h] = (double)bf16_bits_to_f32(aw[h] & 0xFFFFu);
                ad[2 * h + 1] = (double)bf16_bits_to_f32(aw[h] >> 16);
                bd[2 * h] = (double)bf16_bits_to_f32(bw[h] & 0xFFFFu);
                bd[2 * h + 1] = (double)bf16_bits_to_f32(bw[h] >> 16);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[e][c] = __builtin_fma(bd[e], ad[c], acc[e][c]);
        }
    }
    if (k0 >= k) return;
    const float mean = NF4 && fmt != kNoDq ? *mean_p : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t n = n0 + e;
        if (n >= d) break;
        float base[8];
        if constexpr (NF4) {  // What: doubleDequant, bit-identical to qlora_nf4_dequantize
            const uint32_t cw = *reinterpret_cast<const uint32_t *>(codes + (n * k + k0) / 2);
            const int64_t blk = (n * k + k0) / 64;
            const float sh = block_scale(fmt, c2, c1, mean, blk, bshift);
#pragma unroll
            for (int c = 0; c < 8; ++c) base[c] = bf16_round(lut[(cw >> (4 * c)) & 15u] * sh);
        } else {
            const uint4 wv = *reinterpret_cast<const uint4 *>(w_in + n * k + k0);
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                base[2 * h] = bf16_bits_to_f32(ww[h] & 0xFFFFu);
                base[2 * h + 1] = bf16_bits_to_f32(ww[h] >> 16);
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float f[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const double t = s * acc[e][2 * h + q];     // one rounding
                const double m = (double)base[2 * h + q] + t;  // one rounding
                const float tz = __double2float_rz(m);       // fp64 -> fp32 rounded to odd
                f[q] = (double)tz == m ? tz : __uint_as_float(__float_as_uint(tz) | 1u);
            }
            o[h] = pack_bf16x2(f[0], f[1]);                  // -> bf16, nearest even: one rounding of m
        }
        store16_dev(rout, (uint32_t)((n * k + k0) * 2), uint4{o[0], o[1], o[2], o[3]});
    }
}

}  // namespace

hipError_t launch_adapter_merge(const Nf4Weights *w, const uint16_t *w_in, int64_t d, int64_t k, const uint16_t *A,
                                const uint16_t *B, int r, double s, uint16_t *w_out, hipStream_t st) {
    const int64_t tiles = ((d + kMRows - 1) / kMRows) * ((k + kMCols - 1) / kMCols);
    if (w)
        hipLaunchKernelGGL(adapter_merge_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, st, w->codes, w->c2, w->c1,
                           w->mean, w->fmt, w->bshift, nullptr, A, B, d, k, r, s, nf4_consts(), w_out);
    else
        hipLaunchKernelGGL(adapter_merge_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, st, nullptr, nullptr,
                           nullptr, nullptr, 0, 0, w_in, A, B, d, k, r, s, nf4_consts(), w_out);
    return hipGetLastError();
}

}  // namespace qnf4
