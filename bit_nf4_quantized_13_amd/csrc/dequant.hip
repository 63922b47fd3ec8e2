// Standalone doubleDequant: packed NF4 codes + c2 + c1 + mean -> dense bf16.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Double quantization and
// double dequantization": scales[j] = dequant(c2[j], c1[j / 256]) + mean, then
// W[i] = BF16(C[W[i]] * scales[i / 64]).  Here dequant(c2, c1) = c2 / c1 (the
// Int8 rule of "First, how does k-bit quantization work?"); every operation is
// one IEEE fp32 operation and the final rounding is round-to-nearest-even, so
// the output is bit-identical to the expansion inside the fused GEMMs.
//
// HBM-bound: 0.5 + 1/64 + 4/16384 bytes read and 2 bytes written per weight.
// Each work item is 4 code bytes (8 weights) -> one 16-byte store, so loads
// and stores are both contiguous across a wave.
#include "launch.hpp"

namespace qnf4 {
namespace {

__global__ __launch_bounds__(256) void nf4_dequantize_kernel(
    const uint32_t *__restrict__ codes4, const int8_t *__restrict__ c2,
    const float *__restrict__ c1, const float *__restrict__ mean_p, int fmt, int bshift, int64_t items,
    Nf4Consts tab, uint4 *__restrict__ out) {
    __shared__ float lut[16];
    if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
    __syncthreads();
    const float mean = fmt != kNoDq ? *mean_p : 0.0f;
    const __amdgpu_buffer_rsrc_t rout = out_rsrc(out, items * 16);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += stride) {
        const uint32_t c = codes4[i];
        const int64_t blk = i >> 3;  // 8 items per 64-weight block
        const float sh = block_scale(fmt, c2, c1, mean, blk, bshift);
        uint4 o;
        o.x = pack_bf16x2(lut[c & 15] * sh, lut[(c >> 4) & 15] * sh);
        o.y = pack_bf16x2(lut[(c >> 8) & 15] * sh, lut[(c >> 12) & 15] * sh);
        o.z = pack_bf16x2(lut[(c >> 16) & 15] * sh, lut[(c >> 20) & 15] * sh);
        o.w = pack_bf16x2(lut[(c >> 24) & 15] * sh, lut[c >> 28] * sh);
        store16_dev(rout, (uint32_t)(i * 16), o);
    }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *codes, const int8_t *c2, const float *c1,
                             const float *mean, int fmt, int bshift, int64_t n, uint16_t *out, hipStream_t s) {
    const int64_t items = n / 8;
    int64_t grid = (items + 255) / 256;
    if (grid > 256 * 64) grid = 256 * 64;
    hipLaunchKernelGGL(nf4_dequantize_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t *>(codes), c2, c1, mean, fmt, bshift, items, nf4_consts(),
                       reinterpret_cast<uint4 *>(out));
    return hipGetLastError();
}

}  // namespace qnf4
