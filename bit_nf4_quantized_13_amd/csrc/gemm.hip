// Fused NF4-dequant GEMMs on bf16 MFMA (gfx950), forward and input-gradient.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Double quantization and
// double dequantization": the frozen weights are reconstructed in BF16 by
// doubleDequant for the matrix multiplication, and the full layer is
// Y = X doubleDequant(c1, c2, W_NF4) + X L1 L2 (adapter scale alpha/r from
// "How does alpha/r control adapter strength?"); gradients flow through the
// reconstructed weights into the adapters only.  Here:
//   forward:  Y  = X What^T + s U B^T        (U = X A^T, from rows_skinny)
//   dX:       dX = dY What  + s G A          (G = dY B)
// What never exists in memory: each 64-deep k-step expands the packed nibbles
// of one weight tile into LDS as bf16 (bit-identical to the standalone
// dequantize), and the adapter term rides on the same MFMAs as extra k-steps
// with operands [hi(sV) | lo(sV)] and [W | W], so it needs no VALU epilogue.
//
// Tiling: 256 x 256 output tile per 256-thread workgroup, 4 waves each owning a
// 128 x 128 sub-tile (4 x 4 MFMA 32x32x16 tiles, fp32 accumulators), k-step 64,
// double-buffered LDS (2 x 64 KiB) with register prefetch of the next step.
// LDS rows are 64 bf16 = 8 chunks of 16 bytes, chunk index XOR (row & 7).
//
// MFMA v_mfma_f32_32x32x16_bf16 layout (wave64):
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) .. +7]
//   B (16 x 32): lane l holds B[8 (l / 32) .. +7][l % 32]
//   D (32 x 32): lane l, register v: D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;

struct GemmParams {
    const uint16_t *a;     // X (fwd) or dY (dx): [M x Kd] row-major
    int64_t M, N, Kd;      // output [M x N]; reduction length Kd
    const uint8_t *codes;  // packed NF4 codes of W0 [d x k]
    const float *shat;     // dequantized block scales [d*k/64]
    int64_t wk;            // k (row length of W0)
    const float *ext_v;    // U (fwd) or G (dx): [M x r] fp32
    const uint16_t *ext_w; // B [d x r] (fwd) or A [r x k] (dx)
    int r;
    float s;
    uint16_t *out;         // Y or dX [M x N]
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool DX>
__global__ __launch_bounds__(256) void nf4_gemm_kernel(GemmParams p, Nf4Consts tab) {
    __shared__ uint4 sA[2][BM * 8];
    __shared__ uint4 sB[2][BN * 8];
    __shared__ float lut[16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t ntiles_n = (p.N + BN - 1) / BN;
    const int64_t mt = blockIdx.x / ntiles_n, nt = blockIdx.x % ntiles_n;
    const int64_t m_base = mt * BM, n_base = nt * BN;
    const int64_t nK = (p.Kd + BK - 1) / BK;
    const int64_t kblocks = p.wk / 64;  // NF4 blocks per row of W0

    if (tid < 16) lut[tid] = tab.level[tid];

    // ---- global -> register prefetch --------------------------------------
    uint4 ra[8];
    uint4 rb_fwd[2];
    float rs_fwd = 0.0f;
    uint32_t rb_dx[8];
    float rs_dx[8];

    auto load_a = [&](int64_t kt) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = (tid >> 3) + 32 * i, ch = tid & 7;
            const int64_t m = m_base + row, kk = kt * BK + ch * 8;
            ra[i] = uint4{0, 0, 0, 0};
            if (m < p.M && kk < p.Kd) ra[i] = *reinterpret_cast<const uint4 *>(p.a + m * p.Kd + kk);
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = (tid >> 3) + 32 * i, ch = tid & 7;
            sA[buf][swz(row, ch)] = ra[i];
        }
    };
    auto load_b = [&](int64_t kt) {
        if constexpr (!DX) {
            // row n of W0, the 64 weights of block (n, kt)
            const int64_t n = n_base + tid;
            rb_fwd[0] = rb_fwd[1] = uint4{0, 0, 0, 0};
            rs_fwd = 0.0f;
            if (n < p.N) {
                const uint4 *c = reinterpret_cast<const uint4 *>(p.codes + (n * p.wk + kt * BK) / 2);
                rb_fwd[0] = c[0];
                rb_fwd[1] = c[1];
                rs_fwd = p.shat[n * kblocks + kt];
            }
        } else {
            // rows kr = kt*64 + 8*rg + e of W0, columns n_base + 8*cg .. +7
            const int rg = tid >> 5, cg = tid & 31;
            const int64_t col = n_base + 8 * cg;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t kr = kt * BK + 8 * rg + e;
                rb_dx[e] = 0;
                rs_dx[e] = 0.0f;
                if (kr < p.Kd && col < p.N) {
                    rb_dx[e] = *reinterpret_cast<const uint32_t *>(p.codes + (kr * p.wk + col) / 2);
                    rs_dx[e] = p.shat[kr * kblocks + col / 64];
                }
            }
        }
    };
    auto store_b = [&](int buf) {
        if constexpr (!DX) {
            const uint32_t w[8] = {rb_fwd[0].x, rb_fwd[0].y, rb_fwd[0].z, rb_fwd[0].w,
                                   rb_fwd[1].x, rb_fwd[1].y, rb_fwd[1].z, rb_fwd[1].w};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t q = w[c];
                uint4 o;
                o.x = pack_bf16x2(lut[q & 15] * rs_fwd, lut[(q >> 4) & 15] * rs_fwd);
                o.y = pack_bf16x2(lut[(q >> 8) & 15] * rs_fwd, lut[(q >> 12) & 15] * rs_fwd);
                o.z = pack_bf16x2(lut[(q >> 16) & 15] * rs_fwd, lut[(q >> 20) & 15] * rs_fwd);
                o.w = pack_bf16x2(lut[(q >> 24) & 15] * rs_fwd, lut[q >> 28] * rs_fwd);
                sB[buf][swz(tid, c)] = o;
            }
        } else {
            const int rg = tid >> 5, cg = tid & 31;
            float v[8][8];  // [row e][col f]
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int f = 0; f < 8; ++f) v[e][f] = lut[(rb_dx[e] >> (4 * f)) & 15] * rs_dx[e];
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                uint4 o;
                o.x = pack_bf16x2(v[0][f], v[1][f]);
                o.y = pack_bf16x2(v[2][f], v[3][f]);
                o.z = pack_bf16x2(v[4][f], v[5][f]);
                o.w = pack_bf16x2(v[6][f], v[7][f]);
                sB[buf][swz(8 * cg + f, rg)] = o;
            }
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = 2 * ks + (lane >> 5);
            uint4 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = sA[buf][swz(wm * 128 + 32 * i + (lane & 31), ch)];
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = sB[buf][swz(wn * 128 + 32 * j + (lane & 31), ch)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    };

    // ---- main k-loop ---------------------------------------------------------
    load_a(0);
    load_b(0);
    __syncthreads();  // lut ready
    store_a(0);
    store_b(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nK; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < nK;
        if (more) {
            load_a(kt + 1);
            load_b(kt + 1);
        }
        compute(cur);
        if (more) {
            store_a(cur ^ 1);
            store_b(cur ^ 1);
        }
        __syncthreads();
    }

    // ---- adapter term as extra k-steps: [hi(sV) | lo(sV)] x [W | W] ---------
    const int r = p.r, r2 = 2 * p.r;
    uint16_t *sA16 = reinterpret_cast<uint16_t *>(&sA[0][0]);
    uint16_t *sB16 = reinterpret_cast<uint16_t *>(&sB[0][0]);
    for (int e0 = 0; e0 < r2; e0 += BK) {
        for (int idx = tid; idx < BM * BK; idx += 256) {
            const int row = idx >> 6, c = idx & 63;
            const int kk = e0 + c;
            const int64_t m = m_base + row;
            uint16_t val = 0;
            if (kk < r2 && m < p.M) {
                const int j = kk < r ? kk : kk - r;
                const float x = p.s * p.ext_v[m * r + j];
                const uint32_t hb = pack_bf16x2(x, 0.0f) & 0xFFFFu;
                val = kk < r ? (uint16_t)hb
                             : (uint16_t)(pack_bf16x2(x - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
            }
            sA16[swz(row, c >> 3) * 8 + (c & 7)] = val;
        }
        for (int idx = tid; idx < BN * BK; idx += 256) {
            const int row = idx >> 6, c = idx & 63;
            const int kk = e0 + c;
            const int64_t n = n_base + row;
            uint16_t val = 0;
            if (kk < r2 && n < p.N) {
                const int j = kk < r ? kk : kk - r;
                val = DX ? p.ext_w[(int64_t)j * p.wk + n] : p.ext_w[n * r + j];
            }
            sB16[swz(row, c >> 3) * 8 + (c & 7)] = val;
        }
        __syncthreads();
        compute(0);
        __syncthreads();
    }

    // ---- epilogue: fp32 -> bf16 ----------------------------------------------
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n_base + wn * 128 + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m_base + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < p.M && n < p.N)
                    p.out[m * p.N + n] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu);
            }
        }
}

// dequantized block scales: shat[j] = c2[j] / c1[j / 256] + mean
__global__ __launch_bounds__(256) void dq_scales_kernel(const int8_t *__restrict__ c2,
                                                        const float *__restrict__ c1,
                                                        const float *__restrict__ mean_p, int64_t nb,
                                                        float *__restrict__ shat) {
    const float mean = *mean_p;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nb; j += (int64_t)gridDim.x * 256)
        shat[j] = dq_scale(c2[j], c1[j >> 8], mean);
}

hipError_t launch_gemm(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, const float *V,
                       const uint16_t *ext_w, int r, float s, uint16_t *out, float *shat,
                       hipStream_t st) {
    const int64_t nb = w.d * w.k / 64;
    int64_t g = (nb + 255) / 256;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(dq_scales_kernel, dim3((unsigned)g), dim3(256), 0, st, w.c2, w.c1, w.mean, nb,
                       shat);
    GemmParams p;
    p.a = a;
    p.M = M;
    p.N = dx ? w.k : w.d;
    p.Kd = dx ? w.d : w.k;
    p.codes = w.codes;
    p.shat = shat;
    p.wk = w.k;
    p.ext_v = V;
    p.ext_w = ext_w;
    p.r = r;
    p.s = s;
    p.out = out;
    const int64_t tiles = ((M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    if (dx)
        hipLaunchKernelGGL(nf4_gemm_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, st, p, nf4_consts());
    else
        hipLaunchKernelGGL(nf4_gemm_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, st, p, nf4_consts());
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const float *U,
                           const uint16_t *B, int r, float s, uint16_t *Y, float *shat_ws,
                           hipStream_t st) {
    return launch_gemm(false, w, x, M, U, B, r, s, Y, shat_ws, st);
}

hipError_t launch_gemm_dx(const Nf4Weights &w, const uint16_t *dy, int64_t M, const float *G,
                          const uint16_t *A, int r, float s, uint16_t *dX, float *shat_ws,
                          hipStream_t st) {
    return launch_gemm(true, w, dy, M, G, A, r, s, dX, shat_ws, st);
}

}  // namespace qnf4
