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
//      c2 = clamp(rint(c1 (s - mean)), +-127).  With c2 in FP8 (the pages
//      label c2 as FP8; the OCP e4m3 format) the same rule maps a_g to the
//      largest finite e4m3 value: c1 = 448/a_g, c2 = e4m3(c1 (s - mean)),
//      round to nearest even.
// Without double quantization only launch 1 runs, writing the block absmax
// as the stored scale.
// With at most 1024 groups (up to 16.7M weights) every dq_encode workgroup
// runs the mean's tree itself (the same additions in the same order) and
// launch 2 is skipped; workgroup 0 stores the mean.
// The fixed tree order makes the mean, and so every output, bit-reproducible.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int kBlock = 64;
constexpr int kGroup = 256;

// Nearest level through a bucket table.  The exact rule is code = #{j : x >=
// T_j} for x = fl32(w / absmax) in [-1, 1] and the 15 thresholds T_j (the
// smallest fp32 above each midpoint).  Fast path: y = fma(w, 64 rcp(absmax),
// 64) approximates 64 x + 64 in [0, 128] to within 2.5e-5 (rcp and the two
// roundings), so bucket i = (uint) y covers x in about [(i - 64)/64, (i -
// 63)/64): 129 buckets of width 1/64, and the thresholds (at least 0.08 apart)
// put at most one in each.  Entry i is one fp32 word t'_i: the threshold
// inside the bucket in y units (ty = T_j 64 + 64, rounded once; 2^100 if there
// is none) with its four lowest mantissa bits replaced by the count of
// thresholds below the bucket, so code = (bits(t'_i) & 15) + (y >= t'_i).
// The replaced bits move t'_i by less than 16 ulp(ty) <= 1.2e-4 (ty < 128),
// so the fast decision can differ from the exact one only when |y - t'_i| is
// at most 2^-13 (five times the error of y) + 1.2e-4 < kBandY = 2^-12; such a
// y, or one that is not a number (an absmax below 2^-100 or zero
// reciprocal), takes the exact path: the IEEE quotient compared with all 15
// thresholds.  This needs every ty more than kBandY away from the edges of its
// bucket (else the neighbouring bucket would have to check it too): the NF4
// thresholds are 0.015 or more away, which the host verifies once
// (Nf4Consts::bucket_ok); were it not so, every weight would take the exact
// path.  One-dword entries keep the table's LDS reads nearly free of bank
// conflicts, and a lookup costs the wave four VALU operations besides it.
// a lane's value after a DPP lane permutation within its row of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

constexpr int kLutEntries = 129;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
constexpr float kBandY = 0x1p-12f;

// Entry i (bucket [i, i + 1) of y), as fp32 bits.
__device__ uint32_t lut_entry(int i, const Nf4Consts &t) {
    const float lo = (float)i, hi = (float)(i + 1);
    uint32_t base = 0, inside = 0x71800000u;  // 2^100: no threshold in the bucket
    for (int j = 0; j < 15; ++j) {
        const float ty = t.thresh[j] * 64.0f + 64.0f;  // one rounding (< 2^-17)
        if (ty < lo) ++base;
        else if (ty < hi) inside = __float_as_uint(ty);
    }
    return (inside & ~15u) | base;
}

// Each wave owns 64 consecutive blocks of the group: 8 rounds of 8 blocks.
// In a round lane l reads float4 #l of blocks 0-3 and float4 #l of blocks
// 4-7 (16 lanes per block), so every load instruction covers 1 KiB
// contiguously.
__global__ __launch_bounds__(256) void nf4_quantize_groups(
    const float *__restrict__ w, int64_t nb, Nf4Consts tab, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, double *__restrict__ group_sum) {
    __shared__ float s_abs[kGroup];
    __shared__ uint32_t lut[kLutEntries];  // fp32 bits, see lut_entry
    __shared__ __attribute__((aligned(16))) uint16_t s_codes[kGroup * kBlock / 4];  // the group's packed codes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t blk0 = (int64_t)blockIdx.x * kGroup;
    s_abs[tid] = 0.0f;  // missing blocks of a ragged last group count as +0.0

    // Unconditional loads through a buffer resource over this group's blocks
    // (past the last block they read zero): no branch between them, so each
    // block's codes are computed as soon as its own data is in.
    const int64_t nloc = nb - blk0 < kGroup ? nb - blk0 : kGroup;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + blk0 * kBlock, nloc * kBlock * 4);
    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int local = wave * 64 + (i >> 1) * 8 + (i & 1) * 4 + (lane >> 4);
        v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rw, (uint32_t)(local * kBlock * 4 + (lane & 15) * 16), 0, 0));
    }
    if (tid < kLutEntries) lut[tid] = lut_entry(tid, tab);
    // s_abs cleared and the table built before any lane uses them; an LDS-only
    // fence, so the barrier does not wait for the loads above
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    // codes of four weights of one block: the four table reads in flight
    // together, one branch for the (rare) exact path
    auto code4 = [&](const float4 &wv, float m, float r64) {
        const float w4[4] = {wv.x, wv.y, wv.z, wv.w};
        float y[4], t[4];
        uint32_t q[4];
        bool slow = false;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            y[c] = __builtin_fmaf(w4[c], r64, 64.0f);
            t[c] = __uint_as_float(lut[(uint32_t)fminf(fmaxf(y[c], 0.0f), 128.0f)]);  // NaN -> entry 0
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            q[c] = (__float_as_uint(t[c]) & 15u) + (y[c] >= t[c] ? 1u : 0u);
            // near a threshold (or y not a number): decide with the exact quotient
            slow |= !(fabsf(y[c] - t[c]) > kBandY);
        }
        if (__builtin_expect(slow, 0)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = w4[c] / m;
                uint32_t n = 0;
#pragma unroll
                for (int j = 0; j < 15; ++j) n += x >= tab.thresh[j] ? 1u : 0u;
                q[c] = n;
            }
        }
        return q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12);
    };
    // Codes and absmax go to LDS until every block is coded: a global store
    // issued between the waits for the loads above would be counted with them
    // (one in-order counter), and each later wait would then hold the wave
    // until loads it does not need yet have landed.  From LDS the group's codes
    // and absmax leave in whole 16-byte pieces per lane.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int local = wave * 64 + (i >> 1) * 8 + (i & 1) * 4 + (lane >> 4);
        // |w| of finite values orders like its bit pattern read as an unsigned integer
        const uint32_t a0 = __float_as_uint(v[i].x) & 0x7FFFFFFFu, a1 = __float_as_uint(v[i].y) & 0x7FFFFFFFu;
        const uint32_t a2 = __float_as_uint(v[i].z) & 0x7FFFFFFFu, a3 = __float_as_uint(v[i].w) & 0x7FFFFFFFu;
        uint32_t mb = max(max(a0, a1), max(a2, a3));
        mb = max(mb, dpp_u32<0xB1>(mb));   // quad_perm [1,0,3,2]
        mb = max(mb, dpp_u32<0x4E>(mb));   // quad_perm [2,3,0,1]
        mb = max(mb, dpp_u32<0x141>(mb));  // row_half_mirror
        mb = max(mb, dpp_u32<0x140>(mb));  // row_mirror: the max of the 16 lanes of the block
        const float m = __uint_as_float(mb);
        uint32_t packed4 = 0x7777u;  // exact-zero level for an all-zero block
        if (m != 0.0f) {
            // an absmax below 2^-100 (reciprocal near overflow, subnormal
            // operands) takes the exact path for every weight
            const float r64 = (m >= 0x1p-100f && tab.bucket_ok) ? __builtin_amdgcn_rcpf(m) * 64.0f
                                                                : __builtin_nanf("");
            packed4 = code4(v[i], m, r64);
        }
        s_codes[local * 16 + (lane & 15)] = (uint16_t)packed4;
        if ((lane & 15) == 0 && blk0 + local < nb) s_abs[local] = m;
    }
    __syncthreads();
    // the group's codes: 256 blocks x 32 bytes, 2 pieces of 16 bytes per thread
    // (piece p holds half of block p / 2); absmax: one value per thread
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int piece = h * 256 + tid;
        if (piece / 2 < nloc)
            reinterpret_cast<uint4 *>(codes + blk0 * (kBlock / 2))[piece] = reinterpret_cast<const uint4 *>(s_codes)[piece];
    }
    if (tid < nloc) absmax[blk0 + tid] = s_abs[tid];
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

// Blocks of B = 128 or 256 weights (the path for block sizes other than 64):
// one workgroup per group of 256 blocks, thread t owns block blk0 + t: its
// absmax (a max over B weights), then each weight's code by the definition --
// the IEEE quotient x = w / absmax counted against the 15 thresholds -- two
// codes per byte, and the group's fp64 partial sum by the stride-halving tree
// in LDS (a[i] += a[i + h], h = 128 .. 1), the same additions as the 64-weight
// kernel's.  A plain kernel: each thread streams its own block.
template <int B>
__global__ __launch_bounds__(256) void nf4_quantize_wide(const float *__restrict__ w, int64_t nb, Nf4Consts tab,
                                                         uint8_t *__restrict__ codes, float *__restrict__ absmax,
                                                         double *__restrict__ group_sum) {
    __shared__ double s_tree[kGroup];
    const int t = threadIdx.x;
    const int64_t blk = (int64_t)blockIdx.x * kGroup + t;
    const bool valid = blk < nb;
    const float4 *src = reinterpret_cast<const float4 *>(w + (valid ? blk : 0) * B);
    float m = 0.0f;
    if (valid) {
        for (int i = 0; i < B / 4; ++i) {
            const float4 v = src[i];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        absmax[blk] = m;
        uint32_t *dst = reinterpret_cast<uint32_t *>(codes + blk * (B / 2));
        for (int i = 0; i < B / 8; ++i) {
            const float4 v0 = src[2 * i], v1 = src[2 * i + 1];
            const float x8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t q = 7u;  // an all-zero block: the exact-zero level
                if (m != 0.0f) {
                    const float x = x8[e] / m;
                    q = 0;
#pragma unroll
                    for (int j = 0; j < 15; ++j) q += x >= tab.thresh[j] ? 1u : 0u;
                }
                word |= q << (4 * e);
            }
            dst[i] = word;
        }
    }
    s_tree[t] = valid ? (double)m : 0.0;  // missing blocks of a ragged last group count as +0.0
    __syncthreads();
    for (int h = kGroup / 2; h >= 1; h >>= 1) {
        if (t < h) s_tree[t] = s_tree[t] + s_tree[t + h];
        __syncthreads();
    }
    if (t == 0) group_sum[blockIdx.x] = s_tree[0];
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

// dq_encode with the mean computed in every workgroup (a few group sums: the
// same stride-halving tree as dq_mean, so the same bits), which saves the
// one-workgroup launch.  padded <= 1024: thread t folds its entries t, t + 256,
// ... (the levels h >= 256), then the levels h < 256 run across threads in LDS.
constexpr int kMeanInline = 1024;

__device__ __forceinline__ float tree_mean(const double *__restrict__ group_sum, int64_t groups, int64_t padded,
                                           int64_t nb, double *s) {
    const int t = threadIdx.x;
    const int64_t T = padded < 256 ? padded : 256;
    const int per = (int)(padded / T);
    double v[kMeanInline / 256];
#pragma unroll
    for (int u = 0; u < kMeanInline / 256; ++u) {
        const int64_t i = t + T * u;
        v[u] = (t < T && u < per && i < groups) ? group_sum[i] : 0.0;
    }
#pragma unroll
    for (int h = kMeanInline / 512; h >= 1; h >>= 1) {
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
    return (float)(s[0] / (double)nb);
}

template <bool INLINE_MEAN>
__global__ __launch_bounds__(256) void dq_encode(const float *__restrict__ absmax, int64_t nb,
                                                 float *__restrict__ mean_p, const double *__restrict__ group_sum,
                                                 int64_t groups, int64_t padded, int fp8,
                                                 int8_t *__restrict__ c2, float *__restrict__ c1) {
    __shared__ float s_red[4];
    __shared__ double s_tree[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t j = (int64_t)blockIdx.x * kGroup + tid;
    const bool valid = j < nb;
    float mean;
    if constexpr (INLINE_MEAN) {
        mean = tree_mean(group_sum, groups, padded, nb, s_tree);
        if (blockIdx.x == 0 && tid == 0) *mean_p = mean;
    } else {
        mean = *mean_p;
    }
    const float centred = valid ? absmax[j] - mean : 0.0f;
    float a = fabsf(centred);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    if (lane == 0) s_red[wave] = a;
    __syncthreads();
    const float ag = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    // the largest code magnitude: 127 (int8), 448 (the largest finite e4m3 value)
    const float qmax = fp8 ? 448.0f : 127.0f;
    float c = qmax / ag;
    const bool zero = (ag == 0.0f) || !__builtin_isfinite(c);
    if (zero) c = qmax;  // an all-zero group stores zeros and a nonzero scale
    if (valid) {
        const float p = c * centred;  // one fp32 rounding
        int8_t code;
        if (fp8) {
            code = (int8_t)f32_to_e4m3(fminf(fmaxf(p, -448.0f), 448.0f));
        } else {
            const float q = fminf(fmaxf(rintf(p), -127.0f), 127.0f);  // round half to even
            code = (int8_t)(int)q;
        }
        c2[j] = zero ? (int8_t)0 : code;
    }
    if (tid == 0) c1[blockIdx.x] = c;
}

}  // namespace

hipError_t launch_quantize(const float *W0, int64_t n, int block, uint8_t *codes, int8_t *c2, float *c1,
                           float *mean, float *absmax_ws, double *group_sum_ws, int fmt, hipStream_t s) {
    const bool dq = fmt != kNoDq;
    const int fp8 = fmt == kDqFp8 ? 1 : 0;
    const int64_t nb = n / block;
    const int64_t groups = (nb + kGroup - 1) / kGroup;
    int64_t padded = 1;
    while (padded < groups) padded *= 2;
    if (dq && padded > (int64_t)kMeanThreads * kMeanPerThread) return hipErrorInvalidValue;
    // without double quantization the block absmax is the stored scale: no encode
    if (block == 128)
        hipLaunchKernelGGL(nf4_quantize_wide<128>, dim3((unsigned)groups), dim3(256), 0, s, W0, nb, nf4_consts(), codes,
                           dq ? absmax_ws : c1, group_sum_ws);
    else if (block == 256)
        hipLaunchKernelGGL(nf4_quantize_wide<256>, dim3((unsigned)groups), dim3(256), 0, s, W0, nb, nf4_consts(), codes,
                           dq ? absmax_ws : c1, group_sum_ws);
    else
        hipLaunchKernelGGL(nf4_quantize_groups, dim3((unsigned)groups), dim3(256), 0, s, W0, nb,
                           nf4_consts(), codes, dq ? absmax_ws : c1, group_sum_ws);
    if (!dq) return hipGetLastError();
    if (padded <= kMeanInline) {
        hipLaunchKernelGGL(dq_encode<true>, dim3((unsigned)groups), dim3(256), 0, s, absmax_ws, nb, mean, group_sum_ws,
                           groups, padded, fp8, c2, c1);
    } else {
        hipLaunchKernelGGL(dq_mean, dim3(1), dim3(kMeanThreads), 0, s, group_sum_ws, groups, padded, nb, mean);
        hipLaunchKernelGGL(dq_encode<false>, dim3((unsigned)groups), dim3(256), 0, s, absmax_ws, nb, mean, group_sum_ws,
                           groups, padded, fp8, c2, c1);
    }
    return hipGetLastError();
}

}  // namespace qnf4
