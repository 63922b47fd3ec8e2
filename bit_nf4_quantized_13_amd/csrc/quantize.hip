// NF4 quantization with double-quantized block constants.
//
// chkda.github.io "Why do we need LoRA and QLoRA?":
//   "Quantizing and dequantizing with the codebook" -- per block of 64 weights
//     (row-major flattening of W0), scale = max|w|, code = nearest NF4 level
//     of w / scale, ties to the smaller index, all-zero block -> exact zero.
//   "Double quantization and double dequantization" -- the block scales minus
//     their mean are quantized to 8 bits per group of 256 with one fp32 scale
//     per group, using the Int8 absmax rule of "First, how does k-bit
//     quantization work?" (c = 127 / absmax, q = round(c x)).
//
// Three launches:
//   1. nf4_quantize_groups: one workgroup per group of 256 blocks.  Streams W0
//      once with coalesced 16-byte loads, writes the packed codes, the exact
//      fp32 block absmax (workspace) and the group's fp64 partial sum (a
//      stride-halving tree over the 256 absmax values).
//   2. dq_mean: one workgroup; the same stride-halving tree over the group
//      sums, then mean = fp32(sum / nb).
//   3. dq_encode: one workgroup per group; a_g = max|s - mean|, c1 = 127/a_g,
//      c2 = clamp(rint(c1 (s - mean)), +-127).
// The fixed tree order makes the mean, and so every output, bit-reproducible.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int kBlock = 64;
constexpr int kGroup = 256;

__device__ __forceinline__ uint32_t nearest_level(float x, const Nf4Consts &t) {
    uint32_t q = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) q += (x >= t.thresh[j]) ? 1u : 0u;
    return q;
}

// Each wave owns 64 consecutive blocks of the group: 8 rounds of 8 blocks.
// In a round lane l reads float4 #l of blocks 0-3 and float4 #l of blocks
// 4-7 (16 lanes per block), so every load instruction covers 1 KiB
// contiguously.
__global__ __launch_bounds__(256) void nf4_quantize_groups(
    const float *__restrict__ w, int64_t nb, Nf4Consts tab, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, double *__restrict__ group_sum) {
    __shared__ float s_abs[kGroup];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t blk0 = (int64_t)blockIdx.x * kGroup;
    s_abs[tid] = 0.0f;  // missing blocks of a ragged last group count as +0.0

    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t blk = blk0 + wave * 64 + (i >> 1) * 8 + (i & 1) * 4 + (lane >> 4);
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (blk < nb) v[i] = *reinterpret_cast<const float4 *>(w + blk * kBlock + (lane & 15) * 4);
    }
    __syncthreads();  // s_abs cleared before any lane records a block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int local = wave * 64 + (i >> 1) * 8 + (i & 1) * 4 + (lane >> 4);
        const int64_t blk = blk0 + local;
        float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
        m = fmaxf(m, __shfl_xor(m, 8, 16));
        m = fmaxf(m, __shfl_xor(m, 4, 16));
        m = fmaxf(m, __shfl_xor(m, 2, 16));
        m = fmaxf(m, __shfl_xor(m, 1, 16));
        uint32_t q0 = 7, q1 = 7, q2 = 7, q3 = 7;  // exact-zero level for an all-zero block
        if (m != 0.0f) {
            q0 = nearest_level(v[i].x / m, tab);
            q1 = nearest_level(v[i].y / m, tab);
            q2 = nearest_level(v[i].z / m, tab);
            q3 = nearest_level(v[i].w / m, tab);
        }
        if (blk < nb) {
            const uint16_t packed = (uint16_t)(q0 | (q1 << 4) | (q2 << 8) | (q3 << 12));
            *reinterpret_cast<uint16_t *>(codes + blk * (kBlock / 2) + (lane & 15) * 2) = packed;
            if ((lane & 15) == 0) {
                absmax[blk] = m;
                s_abs[local] = m;
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        // stride-halving tree: h = 128 and 64 in registers, then 32..1 across lanes
        double a0 = (double)s_abs[lane] + (double)s_abs[lane + 128];
        double a1 = (double)s_abs[lane + 64] + (double)s_abs[lane + 192];
        double t = a0 + a1;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {
            const double o = __shfl_down(t, h, 64);
            if (lane < h) t = t + o;
        }
        if (lane == 0) group_sum[blockIdx.x] = t;
    }
}

constexpr int kMeanThreads = 1024;
constexpr int kMeanPerThread = 64;  // supports up to 65536 groups

// Stride-halving tree over the group sums padded with +0.0 to P = 2^e entries:
// thread t first folds its entries t, t+T, t+2T, ... (T = min(P, 1024)),
// which are exactly the pairs (i, i+h) of the levels h >= T, then the levels
// h < T run across threads in LDS.
__global__ __launch_bounds__(kMeanThreads) void dq_mean(const double *__restrict__ group_sum,
                                                       int64_t groups, int64_t padded, int64_t nb,
                                                       float *__restrict__ mean) {
    __shared__ double s[kMeanThreads];
    const int t = threadIdx.x;
    const int64_t T = padded < kMeanThreads ? padded : kMeanThreads;
    const int per = (int)(padded / T);
    double v[kMeanPerThread];
#pragma unroll
    for (int u = 0; u < kMeanPerThread; ++u) {
        const int64_t i = t + T * u;
        v[u] = (t < T && u < per && i < groups) ? group_sum[i] : 0.0;
    }
#pragma unroll
    for (int h = kMeanPerThread / 2; h >= 1; h >>= 1) {
        if (2 * h <= per) {
#pragma unroll
            for (int u = 0; u < h; ++u) v[u] = v[u] + v[u + h];
        }
    }
    s[t] = v[0];
    __syncthreads();
    for (int64_t h = T / 2; h >= 1; h >>= 1) {
        if (t < h) s[t] = s[t] + s[t + h];
        __syncthreads();
    }
    if (t == 0) *mean = (float)(s[0] / (double)nb);
}

__global__ __launch_bounds__(256) void dq_encode(const float *__restrict__ absmax, int64_t nb,
                                                 const float *__restrict__ mean_p,
                                                 int8_t *__restrict__ c2, float *__restrict__ c1) {
    __shared__ float s_red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t j = (int64_t)blockIdx.x * kGroup + tid;
    const bool valid = j < nb;
    const float mean = *mean_p;
    const float centred = valid ? absmax[j] - mean : 0.0f;
    float a = fabsf(centred);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    if (lane == 0) s_red[wave] = a;
    __syncthreads();
    const float ag = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    float c = 127.0f / ag;
    const bool zero = (ag == 0.0f) || !__builtin_isfinite(c);
    if (zero) c = 127.0f;  // an all-zero group stores zeros and a nonzero scale
    if (valid) {
        float q = rintf(c * centred);  // round half to even
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        c2[j] = zero ? (int8_t)0 : (int8_t)(int)q;
    }
    if (tid == 0) c1[blockIdx.x] = c;
}

}  // namespace

hipError_t launch_quantize(const float *W0, int64_t n, uint8_t *codes, int8_t *c2, float *c1,
                           float *mean, float *absmax_ws, double *group_sum_ws, hipStream_t s) {
    const int64_t nb = n / kBlock;
    const int64_t groups = (nb + kGroup - 1) / kGroup;
    int64_t padded = 1;
    while (padded < groups) padded *= 2;
    if (padded > (int64_t)kMeanThreads * kMeanPerThread) return hipErrorInvalidValue;
    hipLaunchKernelGGL(nf4_quantize_groups, dim3((unsigned)groups), dim3(256), 0, s, W0, nb,
                       nf4_consts(), codes, absmax_ws, group_sum_ws);
    hipLaunchKernelGGL(dq_mean, dim3(1), dim3(kMeanThreads), 0, s, group_sum_ws, groups, padded, nb,
                       mean);
    hipLaunchKernelGGL(dq_encode, dim3((unsigned)groups), dim3(256), 0, s, absmax_ws, nb, mean, c2,
                       c1);
    return hipGetLastError();
}

}  // namespace qnf4
