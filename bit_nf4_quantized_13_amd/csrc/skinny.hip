// Rank-r ("skinny") GEMMs of the adapter path, on bf16 MFMA with fp32
// accumulation.
//
// The adapter of chkda.github.io "Why do we need LoRA and QLoRA?", "How does
// it work?" (h = W0 x + (alpha/r) B(A x), A acting first) needs, for rows X of
// the batch and upstream gradients dY:
//   U  = X A^T          rows_skinny  (reduction over k)
//   G  = dY B           rows_skinny on B^T (reduction over d)
//   dB = s dY^T U       cols_skinny  (reduction over the M tokens)
//   dA = s G^T X        cols_skinny
// and "How does alpha/r control adapter strength?" notes that alpha/r scales
// the adapter gradients too.  These kernels stream one activation matrix from
// HBM; the rank-r operand stays in L2.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64):
//   A (16 x 32): lane l holds A[l % 16][8 (l / 16) .. +7]
//   B (32 x 16): lane l holds B[8 (l / 16) .. +7][l % 16]
//   D (16 x 16): lane l, register v holds D[4 (l / 16) + v][l % 16]
// Since the k-order of a reduction is free, a lane may take 32 contiguous k
// values (64 bytes) and feed them to four consecutive MFMAs, provided both
// operands use the same k-assignment.
#include "launch.hpp"

namespace qnf4 {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// out[M x R] = In[M x K] W[R x K]^T.  One workgroup per 16 rows; the four
// waves split K in chunks of 128 (round robin) and are summed in LDS in a
// fixed order.
// ---------------------------------------------------------------------------
constexpr int kRowsMaxTiles = 8;  // R <= 128

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

template <int NT, int W>  // W waves split K
__global__ __launch_bounds__(64 * W) void rows_skinny_kernel(const uint16_t *__restrict__ in,
                                                             const uint16_t *__restrict__ w,
                                                             int64_t M, int64_t K, int R,
                                                             float *__restrict__ out) {
    __shared__ f32x4 s_acc[W][NT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t rows = (M - m0) < 16 ? (M - m0) : 16;
    // rows past M and W rows past R read as zero (outside the buffers); the
    // pieces past K of a row are zeroed by the selects below
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + m0 * K, rows * K * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (int64_t)R * K * 2);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Two chunks of 128 k per iteration, all loads issued before the MFMAs
    // (enough bytes in flight per CU to stream the activations from HBM).
    const int64_t chunks = (K + 127) / 128;
    for (int64_t c = wave; c < chunks; c += 2 * W) {
        uint4 a[2][4], b[2][NT][4];
        bool ok[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t k0 = (c + W * u) * 128 + 32 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ok[u][e] = k0 + 8 * e < K;  // K % 8 == 0: pieces are entirely inside or outside
                a[u][e] = load16(rin, (uint32_t)((i * K + k0 + 8 * e) * 2));
#pragma unroll
                for (int t = 0; t < NT; ++t) b[u][t][e] = load16(rw, (uint32_t)(((t * 16 + i) * K + k0 + 8 * e) * 2));
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint4 av = ok[u][e] ? a[u][e] : uint4{0, 0, 0, 0};
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] = mfma16(av, b[u][t][e], acc[t]);
            }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) s_acc[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 v = s_acc[0][t][lane];
            for (int q = 1; q < W; ++q) v += s_acc[q][t][lane];
            const int j = t * 16 + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = (int64_t)blockIdx.x * 16 + 4 * g + r;
                if (row < M && j < R) out[row * R + j] = v[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dst[C x R] = src[R x C]^T (bf16), 64 x 64 tiles through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ src,
                                                             int64_t R, int64_t C,
                                                             uint16_t *__restrict__ dst) {
    __shared__ uint16_t tile[64][65];
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int rr = e / 64, cc = e % 64;
        const int64_t r = r0 + rr, c = c0 + cc;
        tile[rr][cc] = (r < R && c < C) ? src[r * C + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int cc = e / 64, rr = e % 64;
        const int64_t r = r0 + rr, c = c0 + cc;
        if (r < R && c < C) dst[c * R + r] = tile[rr][cc];
    }
}

// ---------------------------------------------------------------------------
// Split-M partial sums of In^T [hi(V) | lo(V)]:
//   part[sp][n][j]     = sum_{m in split sp} In[m][n] hi(V[m][j])
//   part[sp][n][R + j] = sum_{m in split sp} In[m][n] lo(V[m][j])
// hi(v) = bf16(v), lo(v) = bf16(v - hi(v)), so hi + lo carries V to about 16
// significant bits through bf16 MFMA.  A workgroup owns 64 columns n and one
// split; per round it stages 64 rows of In (transposed, m contiguous) and of
// V (split, transposed) in LDS and runs two MFMA k-steps.
// ---------------------------------------------------------------------------
constexpr int kColsTileN = 64;
constexpr int kColsRows = 64;
constexpr int kPitch = kColsRows + 8;  // bf16 elements per LDS row (16-byte multiple)

template <int NT2>  // 16-wide tiles covering 2R
__global__ __launch_bounds__(256) void cols_skinny_partial_kernel(
    const uint16_t *__restrict__ in, const float *__restrict__ v, int64_t M, int64_t N, int R,
    int64_t rows_per_split, float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint16_t s_in[kColsTileN][kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[NT2 * 16][kPitch];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * kColsTileN;
    const int sp = blockIdx.y;
    const int64_t mbeg = (int64_t)sp * rows_per_split;
    const int64_t mend = (mbeg + rows_per_split < M) ? mbeg + rows_per_split : M;
    const int R2 = 2 * R;

    f32x4 acc[NT2];
#pragma unroll
    for (int t = 0; t < NT2; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t m0 = mbeg; m0 < mend; m0 += kColsRows) {
        // In[m0 .. m0+63][n0 .. n0+63]: each thread loads 2 x 8 columns of one row
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = tid + 256 * h;     // 512 pieces of 8 columns
            const int rr = e >> 3, cc = (e & 7) * 8;
            const int64_t mm = m0 + rr, nn = n0 + cc;
            uint4 val = uint4{0, 0, 0, 0};
            if (mm < mend && nn < N) val = *reinterpret_cast<const uint4 *>(in + mm * N + nn);
            const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s_in[cc + 2 * q][rr] = (uint16_t)(wv[q] & 0xFFFF);
                s_in[cc + 2 * q + 1][rr] = (uint16_t)(wv[q] >> 16);
            }
        }
        // V[m0 .. m0+63][0 .. R) split into hi / lo, stored s_v[j'][m]
        for (int e = tid; e < kColsRows * NT2 * 16 / 2; e += 256) {
            const int rr = e % kColsRows, j = e / kColsRows;  // j < NT2*8
            uint16_t hi = 0, lo = 0;
            const int64_t mm = m0 + rr;
            if (j < R && mm < mend) {
                const float x = v[mm * R + j];
                const uint32_t hb = pack_bf16x2(x, 0.0f) & 0xFFFFu;
                hi = (uint16_t)hb;
                lo = (uint16_t)(pack_bf16x2(x - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
            }
            if (j < R) {
                s_v[j][rr] = hi;
                s_v[R + j][rr] = lo;
            }
        }
        // zero the pad columns j' in [2R, NT2*16)
        for (int e = tid; e < kColsRows * (NT2 * 16 - R2); e += 256) {
            const int rr = e % kColsRows, j = R2 + e / kColsRows;
            s_v[j][rr] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kColsRows / 32; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4 *>(&s_in[16 * wave + i][32 * ks + 8 * g]);
#pragma unroll
            for (int t = 0; t < NT2; ++t) {
                const uint4 b = *reinterpret_cast<const uint4 *>(&s_v[16 * t + i][32 * ks + 8 * g]);
                acc[t] = mfma16(a, b, acc[t]);
            }
        }
        __syncthreads();
    }
    // D[4g + r][i]: row = column n of In, col = j'
#pragma unroll
    for (int t = 0; t < NT2; ++t) {
        const int j = 16 * t + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t nn = n0 + 16 * wave + 4 * g + r;
            if (nn < N && j < R2) part[((int64_t)sp * N + nn) * R2 + j] = acc[t][r];
        }
    }
}

__global__ __launch_bounds__(256) void cols_skinny_reduce_kernel(const float *__restrict__ part,
                                                                 int64_t N, int R, int splits,
                                                                 float scale, float *__restrict__ out,
                                                                 int transpose_out) {
    const int64_t total = N * R;
    const int R2 = 2 * R;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int64_t n = e / R;
        const int j = (int)(e % R);
        float hi = 0.0f, lo = 0.0f;
        for (int sp = 0; sp < splits; ++sp) {
            const float *p = part + ((int64_t)sp * N + n) * R2;
            hi += p[j];
            lo += p[R + j];
        }
        const float val = scale * (hi + lo);
        if (transpose_out) out[(int64_t)j * N + n] = val;
        else out[n * R + j] = val;
    }
}

// ---------------------------------------------------------------------------
// Small-rank column reductions on the vector ALU (R <= 16):
//   part[sp][n][j] = sum over rows m of split sp of In[m][n] V[m][j]   (fp32)
// A workgroup owns 512 columns and one row split; lane l of every wave owns
// columns 8 l .. 8 l + 7 (one 16-byte load per row) and the 4 waves take every
// 4th row.  V of the split is staged in LDS (each row's R values are read as a
// broadcast); the 4 wave partials are summed in LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kVColsN = 512;
constexpr int kVRowsMax = 128;  // rows per split

struct ColsJob {
    const uint16_t *in;
    const float *v;
    int64_t N;
    float *part;
};

template <int R>
__global__ __launch_bounds__(256) void cols_valu_kernel(ColsJob j0, ColsJob j1, int64_t M, int64_t rows_per_split) {
    __shared__ float sv[kVRowsMax * R];
    __shared__ float red[4][kVColsN * R];
    const ColsJob &jb = blockIdx.z ? j1 : j0;
    const int64_t N = jb.N;
    if ((int64_t)blockIdx.x * kVColsN >= N) return;  // the other job is wider
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * kVColsN + 8 * lane;
    const int sp = blockIdx.y;
    const int64_t mbeg = (int64_t)sp * rows_per_split;
    const int64_t mend = (mbeg + rows_per_split < M) ? mbeg + rows_per_split : M;
    const int rows = (int)(mend > mbeg ? mend - mbeg : 0);
    for (int e = tid; e < rows * R; e += 256) sv[e] = jb.v[mbeg * R + e];
    __syncthreads();
    // N % 8 == 0: a lane's 8 columns are all inside or all outside
    const bool col_ok = n0 < N;
    const int64_t nrows_buf = (M - mbeg) > 0 ? (M - mbeg) : 0;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(jb.in + mbeg * N, nrows_buf * N * 2);
    float acc[8][R];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[c][j] = 0.0f;
    for (int r0 = wave; r0 < rows; r0 += 16) {
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = load16(rin, (uint32_t)(((int64_t)(r0 + 4 * u) * N + n0) * 2));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rr = r0 + 4 * u;
            if (rr >= rows || !col_ok) continue;
            const uint32_t xw[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
            float xf[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xf[2 * q] = __uint_as_float(xw[q] << 16);
                xf[2 * q + 1] = __uint_as_float(xw[q] & 0xFFFF0000u);
            }
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float vj = sv[rr * R + j];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c][j] = __builtin_fmaf(xf[c], vj, acc[c][j]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < R; ++j) red[wave][(8 * lane + c) * R + j] = acc[c][j];
    __syncthreads();
    for (int e = tid; e < kVColsN * R; e += 256) {
        const int64_t n = (int64_t)blockIdx.x * kVColsN + e / R;
        if (n < N) jb.part[((int64_t)sp * N) * R + (int64_t)blockIdx.x * kVColsN * R + e] =
            (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
    }
}

// ---------------------------------------------------------------------------
// out[M x R] = In W^T for few rows (M * R <= 4096): one wave per output element,
// a dot product of two K-vectors (16-byte loads, all in flight, then a
// cross-lane sum in a fixed order).  Spreads the decode-shaped down-projection
// over the whole chip instead of one workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dot_rows_kernel(const uint16_t *__restrict__ in, const uint16_t *__restrict__ w,
                                                       int64_t M, int64_t K, int R, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // output element
    if (e >= M * R) return;
    const int64_t m = e / R;
    const int j = (int)(e - m * R);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(in + m * K, K * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(w + (int64_t)j * K, K * 2);
    float acc = 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += 64 * 8 * 8) {
        uint4 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t off = (uint32_t)((k0 + (u * 64 + lane) * 8) * 2);
            a[u] = load16(ra, off);  // past K: zero
            b[u] = load16(rb, off);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w}, bv[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = __builtin_fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc);
                acc = __builtin_fmaf(__uint_as_float(av[q] & 0xFFFF0000u), __uint_as_float(bv[q] & 0xFFFF0000u), acc);
            }
        }
    }
    // fixed-order butterfly over the 64 lanes
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) out[e] = acc;
}

}  // namespace

hipError_t launch_rows_skinny(const uint16_t *in, const uint16_t *w, int64_t M, int64_t K, int R,
                              float *out, hipStream_t s) {
    const dim3 grid((unsigned)((M + 15) / 16));
    const int nt = (R + 15) / 16;
    // decode-sized M: one wave per output element, spread over the chip
    if (M * R <= 4096) {
        hipLaunchKernelGGL(dot_rows_kernel, dim3((unsigned)((M * R + 3) / 4)), dim3(256), 0, s, in, w, M, K, R, out);
        return hipGetLastError();
    }
    switch (nt) {
#define QNF4_ROWS(NTV) \
    case NTV: hipLaunchKernelGGL((rows_skinny_kernel<NTV, 4>), grid, dim3(256), 0, s, in, w, M, K, R, out); break;
        QNF4_ROWS(1) QNF4_ROWS(2) QNF4_ROWS(3) QNF4_ROWS(4)
        QNF4_ROWS(5) QNF4_ROWS(6) QNF4_ROWS(7) QNF4_ROWS(8)
#undef QNF4_ROWS
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t *src, int64_t R, int64_t C, uint16_t *dst,
                                 hipStream_t s) {
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, src, R, C, dst);
    return hipGetLastError();
}

int cols_valu_splits(int64_t M) {
    int64_t splits = (M + kVRowsMax - 1) / kVRowsMax;
    return (int)(splits < 1 ? 1 : splits);
}

hipError_t launch_cols_valu_pair(const uint16_t *in0, const float *v0, int64_t N0, float scale0, float *part0,
                                 float *out0, int trans0, const uint16_t *in1, const float *v1, int64_t N1,
                                 float scale1, float *part1, float *out1, int trans1, int64_t M, int R,
                                 ColsReduceJob *jobs, hipStream_t s) {
    const int splits = cols_valu_splits(M);
    const int64_t rps = kVRowsMax;
    const int64_t nmax = in1 && N1 > N0 ? N1 : N0;
    const dim3 grid((unsigned)((nmax + kVColsN - 1) / kVColsN), (unsigned)splits, in1 ? 2u : 1u);
    const ColsJob j0{in0, v0, N0, part0}, j1{in1, v1, N1, part1};
    switch (R) {
#define QNF4_CV(RV)                                                                     \
    case RV:                                                                            \
        hipLaunchKernelGGL(cols_valu_kernel<RV>, grid, dim3(256), 0, s, j0, j1, M, rps); \
        break;
        QNF4_CV(1) QNF4_CV(2) QNF4_CV(3) QNF4_CV(4) QNF4_CV(5) QNF4_CV(6) QNF4_CV(7) QNF4_CV(8)
        QNF4_CV(9) QNF4_CV(10) QNF4_CV(11) QNF4_CV(12) QNF4_CV(13) QNF4_CV(14) QNF4_CV(15) QNF4_CV(16)
#undef QNF4_CV
        default: return hipErrorInvalidValue;
    }
    jobs[0] = ColsReduceJob{part0, N0, R, splits, trans0, scale0, out0};
    jobs[1] = ColsReduceJob{part1, in1 ? N1 : 0, R, splits, trans1, scale1, out1};
    return hipGetLastError();
}

int cols_skinny_splits(int64_t M, int64_t N) {
    const int64_t tiles = (N + kColsTileN - 1) / kColsTileN;
    int64_t splits = (1024 + tiles - 1) / tiles;  // aim for >= 1024 workgroups
    const int64_t max_splits = (M + kColsRows - 1) / kColsRows;
    if (splits > max_splits) splits = max_splits;
    if (splits > 64) splits = 64;
    if (splits < 1) splits = 1;
    return (int)splits;
}

hipError_t launch_cols_skinny(const uint16_t *in, const float *v, int64_t M, int64_t N, int R,
                              float scale, float *part, int splits, float *out, int transpose_out,
                              hipStream_t s) {
    int64_t rows = (M + splits - 1) / splits;
    rows = (rows + kColsRows - 1) / kColsRows * kColsRows;
    const dim3 grid((unsigned)((N + kColsTileN - 1) / kColsTileN), (unsigned)splits);
    const int nt2 = (2 * R + 15) / 16;
    switch (nt2) {
#define QNF4_COLS(NTV)                                                                         \
    case NTV:                                                                                  \
        hipLaunchKernelGGL(cols_skinny_partial_kernel<NTV>, grid, dim3(256), 0, s, in, v, M, N, \
                           R, rows, part);                                                     \
        break;
        QNF4_COLS(1) QNF4_COLS(2) QNF4_COLS(3) QNF4_COLS(4) QNF4_COLS(5) QNF4_COLS(6)
        QNF4_COLS(7) QNF4_COLS(8) QNF4_COLS(9) QNF4_COLS(10) QNF4_COLS(11) QNF4_COLS(12)
        QNF4_COLS(13) QNF4_COLS(14) QNF4_COLS(15) QNF4_COLS(16)
#undef QNF4_COLS
        default: return hipErrorInvalidValue;
    }
    int64_t rgrid = (N * R + 255) / 256;
    if (rgrid > 4096) rgrid = 4096;
    hipLaunchKernelGGL(cols_skinny_reduce_kernel, dim3((unsigned)rgrid), dim3(256), 0, s, part, N,
                       R, splits, scale, out, transpose_out);
    return hipGetLastError();
}

}  // namespace qnf4
