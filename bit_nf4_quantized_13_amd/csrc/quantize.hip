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

// Nearest level through a bucket table (a compare against each of the 15
// thresholds costs two instructions per weight; this costs a handful).
// x = fl32(w / absmax) lies in [-1, 1].  Bucket = sign, exponent and the top
// three mantissa bits of x: the floats of one bucket form an interval, and no
// bucket holds more than one threshold (the thresholds are >= 0.08 apart, a
// bucket at most 0.0625 wide), so code = base + (x >= T) with (base, T) read
// from the table.  |x| < 2^-5 (exponent <= 121) is one bucket per sign: all of
// it lies strictly between the two thresholds around zero (code 7).
// Index: clamp(bits[20..30] - (121 << 3), 0, 55) + 56 * sign.
//
// The division is skipped where it cannot matter: x' = w * rcp(absmax) is
// within a few ulp of x, so the code of x' is the code of x unless a threshold
// lies within that distance.  Each entry carries a band [lo, hi] around its
// threshold (2^-20 relative, far wider than the error); an x' inside the band
// takes the exact path (IEEE division), and so does a whole bucket that has a
// threshold near one of its edges (band = everything; none does for the NF4
// table).
// a lane's value after a DPP lane permutation within its row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kLutEntries = 112;
constexpr float kBand = 0x1p-20f;

struct LutEntry {
    uint32_t base;
    float thresh;  // the one threshold inside the bucket, or +inf
    float lo, hi;  // where x' must go the exact way
};

__device__ __forceinline__ uint32_t lut_index(float x) {
    const uint32_t u = __float_as_uint(x);
    const int k11 = (int)((u >> 20) & 0x7FFu) - (121 << 3);
    const int c = k11 < 0 ? 0 : (k11 > 55 ? 55 : k11);
    return (uint32_t)c + 56u * (u >> 31);
}

// Entry i of the table: the bucket's smallest and largest float decide the
// base count and the threshold inside it.
__device__ void lut_entry(int i, const Nf4Consts &t, LutEntry *out) {
    const uint32_t sign = i >= 56 ? 1u : 0u;
    const int c = i - 56 * (int)sign;
    float lo, hi;  // the bucket's smallest and largest value
    if (c < 8) {   // exponent <= 121 (both signs): all of (-2^-5, 2^-5)
        lo = -0x1.fffffep-6f;
        hi = 0x1.fffffep-6f;
    } else {
        const uint32_t k = (uint32_t)(c + (121 << 3));  // exponent and mantissa top bits
        const uint32_t b0 = (sign << 31) | (k << 20), b1 = b0 | 0xFFFFFu;
        const float f0 = __uint_as_float(b0), f1 = __uint_as_float(b1);
        lo = sign ? f1 : f0;
        hi = sign ? f0 : f1;
    }
    uint32_t base = 0;
    float inside = __builtin_inff();
    bool edge = false;
    for (int j = 0; j < 15; ++j) {
        const float tj = t.thresh[j];
        if (tj <= lo) ++base;
        else if (tj <= hi) inside = tj;
        const float m = fabsf(tj) * (4.0f * kBand);
        if (fabsf(tj - lo) <= m || fabsf(tj - hi) <= m) edge = true;
    }
    out->base = base;
    out->thresh = inside;
    if (edge) {
        out->lo = -__builtin_inff();
        out->hi = __builtin_inff();
    } else if (inside == __builtin_inff()) {
        out->lo = __builtin_inff();  // no threshold: an empty band
        out->hi = -__builtin_inff();
    } else {
        out->lo = inside - fabsf(inside) * kBand;
        out->hi = inside + fabsf(inside) * kBand;
    }
}

// Each wave owns 64 consecutive blocks of the group: 8 rounds of 8 blocks.
// In a round lane l reads float4 #l of blocks 0-3 and float4 #l of blocks
// 4-7 (16 lanes per block), so every load instruction covers 1 KiB
// contiguously.
__global__ __launch_bounds__(256) void nf4_quantize_groups(
    const float *__restrict__ w, int64_t nb, Nf4Consts tab, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, double *__restrict__ group_sum) {
    __shared__ float s_abs[kGroup];
    __shared__ LutEntry lut[kLutEntries];
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
    if (tid < kLutEntries) lut_entry(tid, tab, &lut[tid]);
    __syncthreads();  // s_abs cleared and the table built before any lane uses them
    // codes of four weights of one block: the four table reads in flight
    // together, one branch for the (rare) exact path
    auto code4 = [&](const float4 &wv, float m, float r) {
        const float w4[4] = {wv.x, wv.y, wv.z, wv.w};
        float xa[4];
        LutEntry e[4];
        uint32_t q[4];
        bool slow = false;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            xa[c] = w4[c] * r;
            e[c] = lut[lut_index(xa[c])];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            q[c] = e[c].base + (xa[c] >= e[c].thresh ? 1u : 0u);
            // near a threshold (or x' not a number): decide with the exact quotient
            slow |= !((xa[c] > e[c].hi) | (xa[c] < e[c].lo));
        }
        if (__builtin_expect(slow, 0)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = w4[c] / m;
                const LutEntry ex = lut[lut_index(x)];
                q[c] = ex.base + (x >= ex.thresh ? 1u : 0u);
            }
        }
        return q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int local = wave * 64 + (i >> 1) * 8 + (i & 1) * 4 + (lane >> 4);
        const int64_t blk = blk0 + local;
        float m = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
        m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1,0,3,2]
        m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2,3,0,1]
        m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
        m = fmaxf(m, dpp_f32<0x140>(m));  // row_mirror: the max of the 16 lanes of the block
        uint32_t packed4 = 0x7777u;  // exact-zero level for an all-zero block
        if (m != 0.0f) {
            // an absmax below 2^-100 (reciprocal near overflow, subnormal
            // operands) takes the exact path for every weight
            const float r = m >= 0x1p-100f ? __builtin_amdgcn_rcpf(m) : __builtin_nanf("");
            packed4 = code4(v[i], m, r);
        }
        if (blk < nb) {
            const uint16_t packed = (uint16_t)packed4;
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

hipError_t launch_quantize(const float *W0, int64_t n, uint8_t *codes, int8_t *c2, float *c1,
                           float *mean, float *absmax_ws, double *group_sum_ws, int fmt, hipStream_t s) {
    const bool dq = fmt != kNoDq;
    const int fp8 = fmt == kDqFp8 ? 1 : 0;
    const int64_t nb = n / kBlock;
    const int64_t groups = (nb + kGroup - 1) / kGroup;
    int64_t padded = 1;
    while (padded < groups) padded *= 2;
    if (dq && padded > (int64_t)kMeanThreads * kMeanPerThread) return hipErrorInvalidValue;
    // without double quantization the block absmax is the stored scale: no encode
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
