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
// Since the k-order of a reduction is free, any assignment of k to the MFMAs
// of a chunk works if both operands use it; rows_skinny gives MFMA e of a
// 128-wide chunk the standard 32-wide slab 32 e .., so that the four lane
// groups of a row load 64 contiguous bytes per instruction (16-byte pieces 64
// bytes apart ran the activation stream at about half the rate).
#include "launch.hpp"

namespace qnf4 {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// out[M x R] = In[M x K] W[R x K]^T.  One workgroup per 16 rows; its W waves
// (eight as launched) split K in chunks of 128 (round robin) and are summed
// in LDS in a fixed order.
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

template <int NT, int W, int CPI>  // W waves split K; CPI chunks of 128 k in flight per wave
__global__ __launch_bounds__(64 * W) void rows_skinny_kernel(const uint16_t *__restrict__ in,
                                                             const uint16_t *__restrict__ w,
                                                             int64_t M, int64_t K, int R,
                                                             float *__restrict__ out, uint16_t *__restrict__ vt,
                                                             int64_t Rp) {
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

    // CPI chunks of 128 k per iteration, all loads issued before the MFMAs
    // (enough bytes in flight per CU to stream the activations from HBM).
    const int64_t chunks = (K + 127) / 128;
    for (int64_t c = wave; c < chunks; c += CPI * W) {
        uint4 a[CPI][4], b[CPI][NT][4];
        bool ok[CPI][4];
#pragma unroll
        for (int u = 0; u < CPI; ++u) {
            // MFMA e of the chunk takes k = 32 e .. 32 e + 31, lane group g its 8 k at 32 e + 8 g:
            // the four lanes of a row read 64 contiguous bytes per load
            const int64_t k0 = (c + W * u) * 128 + 8 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ok[u][e] = k0 + 32 * e < K;  // K % 8 == 0: pieces are entirely inside or outside
                a[u][e] = load16(rin, (uint32_t)((i * K + k0 + 32 * e) * 2));
#pragma unroll
                for (int t = 0; t < NT; ++t) b[u][t][e] = load16(rw, (uint32_t)(((t * 16 + i) * K + k0 + 32 * e) * 2));
            }
        }
#pragma unroll
        for (int u = 0; u < CPI; ++u)
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
                if (vt && row < M && j < Rp) {  // transposed bf16 hi + lo planes (zero rows past R)
                    const float f = j < R ? v[r] : 0.0f;
                    const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
                    vt[(int64_t)j * M + row] = (uint16_t)hb;
                    vt[(Rp + j) * M + row] = (uint16_t)(pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// G = dY B for ranks r <= 16 with B in its stored layout [d x r], and, when a
// U is given, U's transposed bf16 hi + lo planes: one launch in place of the
// backward preparation (B^T, U's planes) followed by rows_skinny_kernel.
// The same chunks of 128 k, waves and MFMA order as rows_skinny_kernel<1, W,
// CPI>, so G and its planes come out bit for bit the same.  The second MFMA
// operand (lane (j, g): B[k .. k + 7][j]) has its k strided in memory, so each
// wave loads the B rows of its chunk whole (16-byte pieces of the contiguous
// 128 r values, B 16-byte aligned) and writes them transposed into its own
// LDS buffer B^T [16][128] (rows 272 bytes apart: the 16 fragment rows fall on
// distinct banks), from which it reads the fragments; LDS operations of one
// wave run in order, so the buffer needs no barrier between chunks.  A
// workgroup's 16 rows of U become their planes exactly as the preparation
// launch formed them.
// ---------------------------------------------------------------------------
template <int W, int CPI>
__global__ __launch_bounds__(64 * W) void rows_bt_kernel(const uint16_t *__restrict__ in,
                                                         const uint16_t *__restrict__ bmat, int64_t M, int64_t K,
                                                         int R, uint32_t rinv, float *__restrict__ out,
                                                         uint16_t *__restrict__ vt, int64_t Rp,
                                                         const float *__restrict__ u_in, uint16_t *__restrict__ vt_u) {
    constexpr int PITCH = 136;  // bf16 per row of the B^T buffer: 128 + 8
    __shared__ f32x4 s_acc[W][64];
    __shared__ __attribute__((aligned(16))) uint16_t s_bt[W][16 * PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t rows = (M - m0) < 16 ? (M - m0) : 16;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + m0 * K, rows * K * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bmat, K * R * 2);  // rows past K read as zero
    uint16_t *const bt = &s_bt[wave][0];
    // rows R .. 15 of the buffer stay zero (their columns of G are never stored)
    for (int q = lane; q < 16 * PITCH / 8; q += 64) reinterpret_cast<uint4 *>(bt)[q] = uint4{0, 0, 0, 0};
    if (u_in) {  // U's planes for this workgroup's rows: vt_u[j][m] = hi(U[m][j]), vt_u[Rp + j][m] = lo(U[m][j])
        for (int idx = tid; idx < 16 * Rp; idx += 64 * W) {
            const int64_t j = idx / 16, m = m0 + idx % 16;
            if (m < M) {
                const float f = j < R ? u_in[m * R + j] : 0.0f;
                const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
                vt_u[j * M + m] = (uint16_t)hb;
                vt_u[(Rp + j) * M + m] = (uint16_t)(pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
            }
        }
    }
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int npc = 16 * R;  // 16-byte pieces of B per chunk (128 rows x R values)
    const int64_t chunks = (K + 127) / 128;
    for (int64_t c = wave; c < chunks; c += CPI * W) {
        uint4 a[CPI][4], bp[CPI][4];
        bool ok[CPI][4];
#pragma unroll
        for (int u = 0; u < CPI; ++u) {
            const int64_t ch = c + W * u;
            const int64_t k0 = ch * 128 + 8 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ok[u][e] = k0 + 32 * e < K;  // K % 8 == 0: pieces are entirely inside or outside
                a[u][e] = load16(rin, (uint32_t)((i * K + k0 + 32 * e) * 2));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // piece lane + 64 q of the chunk (at most 4 x 64 = 16 x 16)
                const int pc = lane + 64 * q;
                bp[u][q] = load16(rb, pc < npc && ch < chunks ? (uint32_t)(ch * 256 * R + 16 * pc) : 0x80000000u);
            }
        }
#pragma unroll
        for (int u = 0; u < CPI; ++u) {
            // this chunk's B rows into the buffer as B^T: value e of the chunk is B[e / R][e % R]
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int pc = lane + 64 * q;
                if (pc < npc) {
                    const uint32_t wv[4] = {bp[u][q].x, bp[u][q].y, bp[u][q].z, bp[u][q].w};
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const uint32_t e = 8u * (uint32_t)pc + (uint32_t)h;
                        const uint32_t kk = (e * rinv) >> 16, j = e - kk * (uint32_t)R;
                        bt[j * PITCH + kk] = (uint16_t)((h & 1) ? (wv[h >> 1] >> 16) : (wv[h >> 1] & 0xFFFFu));
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint4 bf = *reinterpret_cast<const uint4 *>(bt + i * PITCH + 32 * e + 8 * g);
                const uint4 av = ok[u][e] ? a[u][e] : uint4{0, 0, 0, 0};
                acc = mfma16(av, bf, acc);
            }
        }
    }
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 v = s_acc[0][lane];
        for (int q = 1; q < W; ++q) v += s_acc[q][lane];
        const int j = i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + 4 * g + r;
            if (row < M && j < R) out[row * R + j] = v[r];
            if (vt && row < M && j < Rp) {  // transposed bf16 hi + lo planes (zero rows past R)
                const float f = j < R ? v[r] : 0.0f;
                const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
                vt[(int64_t)j * M + row] = (uint16_t)hb;
                vt[(Rp + j) * M + row] = (uint16_t)(pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward preparation, one launch, one thread per element: threads [0, R C)
// transpose src = B [R = d rows x C = r columns] into dst = B^T [r x d]
// (thread i: column i / R, row i % R); the next M Rp write the transposed bf16
// planes of a given U [M x r] fp32 (thread: j = i / M, m = i % M):
// vt[j][m] = hi(U[m][j]), vt[Rp + j][m] = lo(U[m][j]) (zero for r <= j < Rp).
// Stores of consecutive threads are consecutive; enough threads to cover the
// latency of the strided loads (B and U are small).  No LDS, no barrier.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t *__restrict__ src, int64_t R, int C,
                                                       uint16_t *__restrict__ dst, const float *__restrict__ U,
                                                       int64_t M, int Rp, uint16_t *__restrict__ vt) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nt = R * C;
    if (i < nt) {
        const int64_t c = i / R, row = i - c * R;
        dst[c * R + row] = src[row * C + c];
        return;
    }
    const int64_t iu = i - nt;
    if (!U || iu >= M * Rp) return;
    const int64_t j = iu / M, m = iu - j * M;
    const float f = j < C ? U[m * C + j] : 0.0f;
    const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
    vt[j * M + m] = (uint16_t)hb;
    vt[(Rp + j) * M + m] = (uint16_t)(pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// Split-M column reductions on MFMA, two jobs in one launch (blockIdx.z):
//   part[sp][j][n] = sum_{m in split sp} V[m][j] In[m][n]     (j < R)
// with V supplied as transposed bf16 hi + lo planes vt [2][Rp][M] (hi + lo
// carry V to about 16 significant bits).  A workgroup owns 128 columns and
// one split; its four waves take 32-row steps in turn.  Lane (n, g) loads rows
// m0 + 8 g .. + 7 of columns 8 n .. 8 n + 7 (16 lanes read a 256-byte row
// segment), transposes the 8 x 8 block in registers (v_perm) and so holds, for
// each q = 0..7, column 8 n + q over those 8 rows: the second MFMA operand of
// tile q, whose column index is n.  The first operand is vt (rows j, k = m),
// contiguous.  Result lane (n, g) register v of tile q: j = 16 t + 4 g + v,
// column 8 n + q.
// ---------------------------------------------------------------------------
constexpr int kCColsN = 128;
constexpr int kCRows = 512;  // rows per split

struct ColsMJob {
    const uint16_t *in;   // [M x N] bf16
    const uint16_t *vt;   // [2][Rp][M] bf16
    int64_t N;
    float *part;          // [splits][R][N]
};

template <int RT>  // 16-row tiles of Rp
__global__ __launch_bounds__(256) void cols_mfma_kernel(ColsMJob j0, ColsMJob j1, int64_t M, int R) {
    __shared__ __attribute__((aligned(16))) float red[4][16 * kCColsN];
    const ColsMJob &jb = blockIdx.z ? j1 : j0;
    const int64_t N = jb.N;
    const int64_t cb = (int64_t)blockIdx.x * kCColsN;
    if (cb >= N) return;  // the other job is wider
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t Rp = 16 * RT;
    const int sp = blockIdx.y;
    const int64_t mbeg = (int64_t)sp * kCRows;
    const int64_t mend = mbeg + kCRows < M ? mbeg + kCRows : M;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(jb.in, M * N * 2);
    const __amdgpu_buffer_rsrc_t rvt = make_rsrc(jb.vt, 2 * Rp * M * 2);
    const bool col_ok = cb + 8 * n16 < N;  // N % 8 == 0
    f32x4 acc[RT][8];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t m0 = mbeg + 32 * wave; m0 < mend; m0 += 128) {
        uint4 rv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t row = m0 + 8 * g + e;
            rv[e] = load16(rin, row < mend && col_ok ? (uint32_t)((row * N + cb + 8 * n16) * 2) : 0x80000000u);
        }
        uint4 ph[RT], pl[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int64_t off = ((16 * t + n16) * M + m0 + 8 * g) * 2;
            ph[t] = load16(rvt, (uint32_t)off);
            pl[t] = load16(rvt, (uint32_t)(off + Rp * M * 2));
        }
        // 8 x 8 transpose: word h of column q pairs rows 2 h (low half) and 2 h + 1 (high half)
        uint4 fr[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint4 a = rv[2 * h], b = rv[2 * h + 1];
                const uint32_t lo = q < 2 ? a.x : q < 4 ? a.y : q < 6 ? a.z : a.w;
                const uint32_t hi = q < 2 ? b.x : q < 4 ? b.y : q < 6 ? b.z : b.w;
                w[h] = __builtin_amdgcn_perm(hi, lo, sel);
            }
            fr[q] = uint4{w[0], w[1], w[2], w[3]};
        }
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                acc[t][q] = mfma16(ph[t], fr[q], acc[t][q]);
                acc[t][q] = mfma16(pl[t], fr[q], acc[t][q]);
            }
    }
    // the four waves in a fixed order, one 16-row tile of j at a time
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float *dst = &red[wave][(4 * g + v) * kCColsN + 8 * n16];
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[t][0][v], acc[t][1][v], acc[t][2][v], acc[t][3][v]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{acc[t][4][v], acc[t][5][v], acc[t][6][v], acc[t][7][v]};
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;  // (j, column), column fastest
            const int jl = e / kCColsN, c = e % kCColsN;
            const int j = 16 * t + jl;
            const int64_t n = cb + c;
            if (j < R && n < N)
                jb.part[((int64_t)sp * R + j) * N + n] = (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// out[M x R] = In W^T for few rows (M * R <= 4096): one wave per output element,
// a dot product of two K-vectors (16-byte loads, all in flight, then a
// cross-lane sum in a fixed order).  Spreads the decode-shaped down-projection
// over the whole chip instead of one workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dot_rows_kernel(const uint16_t *__restrict__ in, const uint16_t *__restrict__ w,
                                                       int64_t M, int64_t K, int R, float *__restrict__ out,
                                                       uint16_t *__restrict__ vt, int64_t Rp) {
    const int lane = threadIdx.x & 63;
    const int64_t Rc = vt ? Rp : R;  // columns computed: Rp when the zero-padded planes are wanted
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // output element (m, j)
    if (e >= M * Rc) return;
    const int64_t m = e / Rc;
    const int j = (int)(e - m * Rc);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(in + m * K, K * 2);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(w + (int64_t)(j < R ? j : 0) * K, j < R ? K * 2 : 0);
    float acc = 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += 64 * 8 * 8) {
        uint4 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t off = (uint32_t)((k0 + (u * 64 + lane) * 8) * 2);
            a[u] = load16(ra, off);  // past K (and W rows past R): zero
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
    if (lane == 0) {
        if (j < R) out[m * R + j] = acc;
        if (vt) {  // transposed bf16 hi + lo planes
            const uint32_t hb = pack_bf16x2(acc, 0.0f) & 0xFFFFu;
            vt[(int64_t)j * M + m] = (uint16_t)hb;
            vt[(Rp + j) * M + m] = (uint16_t)(pack_bf16x2(acc - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
        }
    }
}

// ---------------------------------------------------------------------------
// The same product for wide ranks (R > 16) with many rows: every workgroup of
// rows_skinny_kernel reads all of W (R x K; 512 KiB at R = 64, K = 4096) for
// its 16 rows, so W dominated the traffic.  Here a workgroup owns MT 16-row
// tiles and one of S slices of K (whole 128-wide chunks), so W is read once per
// 16 MT rows; its four waves take the slice's chunks in turn, every MFMA on a
// W fragment serving the MT row tiles.  The workgroup's sum over its waves (in
// wave order) is a partial [S][R][M] fp32; rows_reduce_kernel adds the S
// partials in slice order into out (and its planes).
// ---------------------------------------------------------------------------
template <int NT, int MT>
__global__ __launch_bounds__(256) void rows_split_kernel(const uint16_t *__restrict__ in,
                                                         const uint16_t *__restrict__ w, int64_t M, int64_t K,
                                                         int R, int64_t kslice, float *__restrict__ part) {
    __shared__ f32x4 s_acc[4][NT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16 * MT;
    const int sl = blockIdx.y;
    const int64_t rows = (M - m0) < 16 * MT ? (M - m0) : 16 * MT;
    // rows past M and W rows past R read as zero (outside the buffers); pieces
    // past the slice or past K are zeroed by the selects below
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + m0 * K, rows * K * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (int64_t)R * K * 2);
    const int64_t kb = sl * kslice;
    const int64_t ke = (kb + kslice) < K ? (kb + kslice) : K;
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t chunks = (ke - kb + 127) / 128;
    for (int64_t c = wave; c < chunks; c += 4) {
        // MFMA e of the chunk takes k = 32 e .. 32 e + 31, lane group g its 8 k at 32 e + 8 g
        const int64_t k0 = kb + c * 128 + 8 * g;
        uint4 a[MT][4], b[NT][4];
        bool ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = k0 + 32 * e < ke;  // K % 8 == 0 and kslice % 128 == 0: pieces wholly in or out
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt][e] = load16(rin, (uint32_t)(((16 * mt + i) * K + k0 + 32 * e) * 2));
#pragma unroll
            for (int t = 0; t < NT; ++t) b[t][e] = load16(rw, (uint32_t)(((t * 16 + i) * K + k0 + 32 * e) * 2));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 av = ok[e] ? a[mt][e] : uint4{0, 0, 0, 0};
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[mt][t] = mfma16(av, b[t][e], acc[mt][t]);
            }
    }
    // wave sums, one row tile at a time: wave w adds column tiles w, w + 4 over
    // the four waves in order; lane (i, g) register r is row 4 g + r, column 16 t + i
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int t = 0; t < NT; ++t) s_acc[wave][t][lane] = acc[mt][t];
        __syncthreads();
        for (int t = wave; t < NT; t += 4) {
            f32x4 v = s_acc[0][t][lane];
            for (int q = 1; q < 4; ++q) v += s_acc[q][t][lane];
            const int j = 16 * t + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * mt + 4 * g + r;
                if (row < M && j < R) part[((int64_t)sl * R + j) * M + row] = v[r];
            }
        }
        __syncthreads();
    }
}

// out[m][j] = the S partials of rows_split_kernel added in slice order; vt: the
// transposed hi / lo planes as in rows_skinny_kernel (zero for R <= j < Rp).
// Thread (j, m), m fastest: partial reads and plane stores are contiguous.
__global__ __launch_bounds__(256) void rows_reduce_kernel(const float *__restrict__ part, int S, int64_t M, int R,
                                                          float *__restrict__ out, uint16_t *__restrict__ vt,
                                                          int64_t Rp) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rc = vt ? Rp : R;
    if (e >= M * rc) return;
    const int64_t j = e / M, m = e - j * M;
    float v = 0.0f;
    if (j < R) {
        for (int q = 0; q < S; ++q) v += part[((int64_t)q * R + j) * M + m];
        out[m * R + j] = v;
    }
    if (vt) {
        const uint32_t hb = pack_bf16x2(v, 0.0f) & 0xFFFFu;
        vt[j * M + m] = (uint16_t)hb;
        vt[(Rp + j) * M + m] = (uint16_t)(pack_bf16x2(v - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
    }
}

// The split of a wide-rank product over workgroups: MT row tiles per workgroup
// and S slices of K such that about 256 workgroups of four waves cover it
// (measured: eight waves, or twice the slices, left waves idle and doubled the
// partials).
struct RowsSplit {
    int mt, S;
    int64_t groups, kslice;
};
RowsSplit rows_split_plan(int64_t M, int64_t K, int R) {
    RowsSplit p;
    p.mt = R <= 64 ? 4 : 2;
    p.groups = (M + 16 * p.mt - 1) / (16 * p.mt);
    int64_t S = 256 / p.groups;
    S = S < 1 ? 1 : (S > 16 ? 16 : S);
    const int64_t chunks = (K + 127) / 128;
    if (S > chunks) S = chunks;
    p.kslice = (chunks + S - 1) / S * 128;
    p.S = (int)((K + p.kslice - 1) / p.kslice);
    return p;
}
bool rows_split_used(int64_t M, int R) { return R > 16 && M >= 256; }

}  // namespace

size_t rows_split_part_bytes(int64_t M, int64_t K, int R) {
    if (!rows_split_used(M, R)) return 0;
    return sizeof(float) * (size_t)rows_split_plan(M, K, R).S * (size_t)R * (size_t)M;
}

bool rows_split_partials_used(int64_t M, int R) { return rows_split_used(M, R); }

hipError_t launch_rows_split_partials(const uint16_t *in, const uint16_t *w, int64_t M, int64_t K, int R, float *part,
                                      int *S, hipStream_t s) {
    if (!rows_split_used(M, R) || !part) return hipErrorInvalidValue;
    const RowsSplit pl = rows_split_plan(M, K, R);
    const dim3 sgrid((unsigned)pl.groups, (unsigned)pl.S);
    switch ((R + 15) / 16) {
#define QNF4_SPLIT(NTV, MTV)                                                                                       \
    case NTV:                                                                                                      \
        hipLaunchKernelGGL((rows_split_kernel<NTV, MTV>), sgrid, dim3(256), 0, s, in, w, M, K, R, pl.kslice, part); \
        break;
        QNF4_SPLIT(2, 4) QNF4_SPLIT(3, 4) QNF4_SPLIT(4, 4)
        QNF4_SPLIT(5, 2) QNF4_SPLIT(6, 2) QNF4_SPLIT(7, 2) QNF4_SPLIT(8, 2)
#undef QNF4_SPLIT
        default: return hipErrorInvalidValue;
    }
    *S = pl.S;
    return hipGetLastError();
}

hipError_t launch_rows_skinny(const uint16_t *in, const uint16_t *w, int64_t M, int64_t K, int R,
                              float *out, uint16_t *vt, float *part, hipStream_t s) {
    const int64_t Rp = cols_rank_pad(R);
    const dim3 grid((unsigned)((M + 15) / 16));
    const int nt = (R + 15) / 16;
    // decode-sized M: one wave per output element, spread over the chip
    // (the choice of kernel must not depend on vt: U and its recomputation agree bit for bit)
    if (M * R <= 4096) {
        const int64_t rc = vt ? Rp : R;
        hipLaunchKernelGGL(dot_rows_kernel, dim3((unsigned)((M * rc + 3) / 4)), dim3(256), 0, s, in, w, M, K, R, out,
                           vt, Rp);
        return hipGetLastError();
    }
    if (rows_split_used(M, R)) {
        if (!part) return hipErrorInvalidValue;
        const RowsSplit pl = rows_split_plan(M, K, R);
        const dim3 sgrid((unsigned)pl.groups, (unsigned)pl.S);
        switch (nt) {
#define QNF4_SPLIT(NTV, MTV)                                                                                       \
    case NTV:                                                                                                      \
        hipLaunchKernelGGL((rows_split_kernel<NTV, MTV>), sgrid, dim3(256), 0, s, in, w, M, K, R, pl.kslice, part); \
        break;
            QNF4_SPLIT(2, 4) QNF4_SPLIT(3, 4) QNF4_SPLIT(4, 4)
            QNF4_SPLIT(5, 2) QNF4_SPLIT(6, 2) QNF4_SPLIT(7, 2) QNF4_SPLIT(8, 2)
#undef QNF4_SPLIT
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t rc = vt ? Rp : R;
        hipLaunchKernelGGL(rows_reduce_kernel, dim3((unsigned)((M * rc + 255) / 256)), dim3(256), 0, s, part, pl.S, M,
                           R, out, vt, Rp);
        return hipGetLastError();
    }
    switch (nt) {
#define QNF4_ROWS(NTV) \
    case NTV:                                                                                          \
        hipLaunchKernelGGL((rows_skinny_kernel<NTV, 8, (NTV == 1 ? 4 : 2)>), grid, dim3(512), 0, s, in, w, M, K, R, \
                           out, vt, Rp);                                                                       \
        break;
        QNF4_ROWS(1) QNF4_ROWS(2) QNF4_ROWS(3) QNF4_ROWS(4)
        QNF4_ROWS(5) QNF4_ROWS(6) QNF4_ROWS(7) QNF4_ROWS(8)
#undef QNF4_ROWS
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t cols_rank_pad(int r) { return (r + 15) / 16 * 16; }

bool rows_bt_supported(int64_t M, int R, const void *B) {
    return R <= 16 && M * R > 4096 && reinterpret_cast<uintptr_t>(B) % 16 == 0;
}

hipError_t launch_rows_bt(const uint16_t *dY, const uint16_t *B, int64_t M, int64_t d, int R, float *G, uint16_t *vt_g,
                          const float *U, uint16_t *vt_u, hipStream_t s) {
    if (!rows_bt_supported(M, R, B)) return hipErrorInvalidValue;
    const int64_t Rp = cols_rank_pad(R);
    const uint32_t rinv = (65536u + (uint32_t)R - 1) / (uint32_t)R;  // e / R = (e rinv) >> 16 for e < 2048
    hipLaunchKernelGGL((rows_bt_kernel<8, 4>), dim3((unsigned)((M + 15) / 16)), dim3(512), 0, s, dY, B, M, d, R, rinv,
                       G, vt_g, Rp, U, vt_u);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const uint16_t *B, int64_t d, int r, uint16_t *Bt, const float *U, int64_t M,
                           uint16_t *vt, hipStream_t s) {
    const int Rp = (int)cols_rank_pad(r);
    const int64_t n = d * r + (U ? M * Rp : 0);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, B, d, r, Bt, U, M, Rp, vt);
    return hipGetLastError();
}

int cols_splits(int64_t M) {
    const int64_t sp = (M + kCRows - 1) / kCRows;
    return (int)(sp < 1 ? 1 : sp);
}

hipError_t launch_cols_pair(const uint16_t *in0, const uint16_t *vt0, int64_t N0, float scale0, float *part0,
                            float *out0, int trans0, const uint16_t *in1, const uint16_t *vt1, int64_t N1,
                            float scale1, float *part1, float *out1, int trans1, int64_t M, int R,
                            ColsReduceJob *jobs, hipStream_t s) {
    const int splits = cols_splits(M);
    const int64_t nmax = in1 && N1 > N0 ? N1 : N0;
    const dim3 grid((unsigned)((nmax + kCColsN - 1) / kCColsN), (unsigned)splits, in1 ? 2u : 1u);
    const ColsMJob j0{in0, vt0, N0, part0}, j1{in1, vt1, N1, part1};
    switch ((R + 15) / 16) {
#define QNF4_CM(RT)                                                                  \
    case RT:                                                                         \
        hipLaunchKernelGGL(cols_mfma_kernel<RT>, grid, dim3(256), 0, s, j0, j1, M, R); \
        break;
        QNF4_CM(1) QNF4_CM(2) QNF4_CM(3) QNF4_CM(4) QNF4_CM(5) QNF4_CM(6) QNF4_CM(7) QNF4_CM(8)
#undef QNF4_CM
        default: return hipErrorInvalidValue;
    }
    jobs[0] = ColsReduceJob{part0, N0, R, splits, trans0, scale0, out0};
    jobs[1] = ColsReduceJob{part1, in1 ? N1 : 0, R, splits, trans1, scale1, out1};
    return hipGetLastError();
}

}  // namespace qnf4
