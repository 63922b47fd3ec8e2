// Dropout on the adapter's input, for training with a LoRA dropout rate.
//
// fromzero2ai.dev "LoRA and QLoRA", "Python Implementation: Fine-Tuning with
// PEFT and BitsAndBytes", trains with a LoRA dropout rate (0.05); chkda.github.io
// "Why do we need LoRA and QLoRA?", "Merging LoRA weights for inference", notes
// that the two-path layer equals the merged one only with dropout disabled.
// Dropout acts on the adapter path alone:
//   Xd = drop(X): x c where kept, +0 where dropped, rounded once to bf16,
//        c = fl32(1 / fl32(1 - p))
//   U = Xd A^T (forward), dA = s G^T Xd, and the adapter's share of dX is
//   c (M o (s G A)) with M the keep mask.
// The mask comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011), so the backward regenerates
// the forward's mask from the seed instead of storing it: element i = m k + col
// uses word i mod 4 of the block for counter (i div 4 low and high words, 0, 0)
// and key (seed low, seed high), and is dropped iff that word < floor(p 2^32).
//
// Both kernels stream: 16 bytes (8 elements, two Philox blocks) per thread.
#include "launch.hpp"

namespace qnf4 {
namespace {

struct Philox4 {
    uint32_t w[4];
};

// Ten rounds; the key gains the Weyl increments between rounds.
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        if (rnd) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32 x 32 -> 64-bit product each (v_mad_u64_u32: high and low words at once)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// keep bits of elements 8 t .. 8 t + 7 (bit q: element 8 t + q kept): words of
// the blocks for counters 2 t (elements 8 t .. + 3) and 2 t + 1 (the next four)
__device__ __forceinline__ uint32_t keep8(uint64_t t, uint32_t thr, uint32_t s0, uint32_t s1) {
    const uint64_t c = 2 * t;
    const Philox4 a = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u, s0, s1);
    const Philox4 b = philox4x32_10((uint32_t)(c + 1), (uint32_t)((c + 1) >> 32), 0u, 0u, s0, s1);
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        bits |= (a.w[q] >= thr ? 1u : 0u) << q;
        bits |= (b.w[q] >= thr ? 1u : 0u) << (4 + q);
    }
    return bits;
}

__global__ __launch_bounds__(256) void lora_dropout_kernel(const uint4 *__restrict__ x, int64_t items, uint32_t thr,
                                                           float c, uint32_t s0, uint32_t s1,
                                                           uint4 *__restrict__ xd) {
    const __amdgpu_buffer_rsrc_t rout = out_rsrc(xd, items * 16);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < items; t += stride) {
        const uint4 v = x[t];
        const uint32_t keep = keep8((uint64_t)t, thr, s0, s1);
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float lo = bf16_bits_to_f32(in[h] & 0xFFFFu) * c;  // one fp32 rounding
            const float hi = bf16_bits_to_f32(in[h] >> 16) * c;
            const uint32_t p = pack_bf16x2(lo, hi);
            const uint32_t m = ((keep >> (2 * h)) & 1u ? 0x0000FFFFu : 0u) | ((keep >> (2 * h + 1)) & 1u ? 0xFFFF0000u : 0u);
            o[h] = p & m;  // dropped: +0
        }
        store16_dev(rout, (uint32_t)(t * 16), uint4{o[0], o[1], o[2], o[3]});
    }
}

// dX[m][n] = bf16( base[m][n] + (kept ? sc sum_j G[m][j] A[j][n] : 0) ), j ascending,
// sc = fl32(s c): the fp32 sum of the GEMM's unrounded base term and the masked
// adapter term, rounded once.  A workgroup covers 4 rows (blockIdx.x) and 2048 columns
// (blockIdx.y); a thread takes 8 consecutive columns of the 4 rows, so each A
// load serves 4 rows, and the G values, the same for the whole workgroup, come
// through scalar loads.
constexpr int kAddRows = 4;

__global__ __launch_bounds__(256) void dropout_dx_add_kernel(const f32x4 *__restrict__ base,
                                                             uint4 *__restrict__ dx, int64_t M, int64_t k,
                                                             const float *__restrict__ G, int r,
                                                             const uint16_t *__restrict__ A, float sc, uint32_t thr,
                                                             uint32_t s0, uint32_t s1) {
    const int64_t n = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
    const int64_t m0 = (int64_t)blockIdx.x * kAddRows;
    if (n >= k) return;
    const int rows = M - m0 < kAddRows ? (int)(M - m0) : kAddRows;
    const __amdgpu_buffer_rsrc_t rout = out_rsrc(dx, M * k * 2);
    float acc[kAddRows][8];
#pragma unroll
    for (int i = 0; i < kAddRows; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
    const float *g = G + m0 * r;
#pragma unroll 4
    for (int j = 0; j < r; ++j) {
        const uint4 av = *reinterpret_cast<const uint4 *>(A + (int64_t)j * k + n);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
        float af[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            af[2 * h] = bf16_bits_to_f32(aw[h] & 0xFFFFu);
            af[2 * h + 1] = bf16_bits_to_f32(aw[h] >> 16);
        }
#pragma unroll
        for (int i = 0; i < kAddRows; ++i) {
            const float gj = i < rows ? g[(int64_t)i * r + j] : 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[i][q] = __builtin_fmaf(gj, af[q], acc[i][q]);
        }
    }
#pragma unroll
    for (int i = 0; i < kAddRows; ++i) {
        if (i >= rows) break;
        const int64_t t = ((m0 + i) * k + n) / 8;  // the 8-element item: k % 8 == 0
        const uint32_t keep = keep8((uint64_t)t, thr, s0, s1);
        const f32x4 v0 = base[2 * t], v1 = base[2 * t + 1];
        const float in[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float tlo = (keep >> (2 * h)) & 1u ? sc * acc[i][2 * h] : 0.0f;
            const float thi = (keep >> (2 * h + 1)) & 1u ? sc * acc[i][2 * h + 1] : 0.0f;
            o[h] = pack_bf16x2(in[2 * h] + tlo, in[2 * h + 1] + thi);
        }
        store16_dev(rout, (uint32_t)(t * 16), uint4{o[0], o[1], o[2], o[3]});
    }
}

int64_t stream_grid(int64_t items) {
    int64_t g = (items + 255) / 256;
    return g > 256 * 32 ? 256 * 32 : (g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_lora_dropout(const uint16_t *x, int64_t M, int64_t k, uint32_t thr, float c, uint64_t seed,
                               uint16_t *xd, hipStream_t st) {
    const int64_t items = M * k / 8;
    hipLaunchKernelGGL(lora_dropout_kernel, dim3((unsigned)stream_grid(items)), dim3(256), 0, st,
                       reinterpret_cast<const uint4 *>(x), items, thr, c, (uint32_t)seed, (uint32_t)(seed >> 32),
                       reinterpret_cast<uint4 *>(xd));
    return hipGetLastError();
}

hipError_t launch_dropout_dx_add(const float *base, uint16_t *dx, int64_t M, int64_t k, const float *G, int r,
                                 const uint16_t *A, float sc, uint32_t thr, uint64_t seed, hipStream_t st) {
    const dim3 grid((unsigned)((M + kAddRows - 1) / kAddRows), (unsigned)((k / 8 + 255) / 256));
    hipLaunchKernelGGL(dropout_dx_add_kernel, grid, dim3(256), 0, st, reinterpret_cast<const f32x4 *>(base),
                       reinterpret_cast<uint4 *>(dx), M, k, G, r, A, sc, thr, (uint32_t)seed, (uint32_t)(seed >> 32));
    return hipGetLastError();
}

}  // namespace qnf4
