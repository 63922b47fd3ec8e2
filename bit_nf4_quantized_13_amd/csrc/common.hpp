// Shared device-side definitions of the QLoRA NF4 library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qnf4 {

// NF4 levels C[0..15] and decision thresholds T[0..14] (x >= T[j] <=> x is
// nearer to C[j+1] than to C[j], ties to the smaller index).  Passed to the
// kernels by value, so they arrive in scalar registers.
struct Nf4Consts {
    float level[16];
    float thresh[15];
    // 1 when every threshold, as y = T 64 + 64 in fp32, lies more than 2^-11
    // from an integer (the quantize kernel's bucket table relies on it)
    int bucket_ok;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Large outputs stored with device scope (sc1: written through the XCD's L2
// into the memory-side cache): the launch then does not end on a writeback of
// its dirty L2 lines, and the next kernel finds the data in the memory-side
// cache as before.  out_rsrc covers [base, base + bytes) (bytes < 2^32).
constexpr int kDeviceScopeStore = 16;  // cache-policy bits of the store: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
__device__ __forceinline__ void store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, byte_off, 0, kDeviceScopeStore);
}

// Two fp32 values -> packed bf16x2 (lo in bits 0..15), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float bf16_round(float f) {
    return bf16_bits_to_f32(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// How the block constants of a weight are stored.
enum ScaleFormat : int {
    kNoDq = 0,    // one fp32 absmax per block, in the c1 array
    kDqInt8 = 1,  // double quantization, c2 as int8
    kDqFp8 = 2,   // double quantization, c2 as OCP FP8 e4m3 (raw bytes)
};

// OCP FP8 e4m3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, the
// exponent field 0 holding the subnormals m * 2^-9, S.1111.111 = NaN, no
// infinities) -> fp32: v_cvt_f32_fp8 reads this format on gfx950, exactly, for
// byte SEL of a dword (every one of the 256 codes was checked against the
// format's definition; the library's tests read all finite codes back).
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

// fp32 -> OCP FP8 e4m3, round to nearest, ties to the even code, for finite
// |x| <= 448 (the largest finite e4m3 value; callers clamp first).  Below
// 2^-6 the grid is the multiples of 2^-9 (code = the multiple, 8 being the
// smallest normal); above it the 3 leading mantissa bits are kept and the
// carry of the rounding runs into the exponent field.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t bits = __float_as_uint(x), sign = (bits >> 24) & 0x80u;
    const float a = fabsf(x);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);  // exact scaling, round half to even
    } else {
        const uint32_t ab = bits & 0x7FFFFFFFu;
        const uint32_t t = (((ab >> 23) - 120u) << 3) | ((ab >> 20) & 7u);
        const uint32_t rem = ab & 0xFFFFFu;
        code = t + ((rem > 0x80000u || (rem == 0x80000u && (t & 1u))) ? 1u : 0u);
    }
    return code | sign;
}

// The value of a stored c2 byte (byte SEL of a dword).
template <int SEL = 0>
__device__ __forceinline__ float c2_value(uint32_t word, bool fp8) {
    return fp8 ? e4m3_byte_to_f32<SEL>(word) : (float)(int8_t)((word >> (8 * SEL)) & 0xFFu);
}

// Dequantized block scale (doubleDequant): fp32(c2 / c1) + mean, two IEEE
// fp32 operations (the library is compiled with -ffp-contract=off).
__device__ __forceinline__ float dq_scale(float c2, float c1, float mean) {
    return c2 / c1 + mean;
}

// The scale of the 64-weight sub-block j64 of a stored weight whose blocks
// hold 64 << bshift weights (block j64 >> bshift): doubleDequant's dq_scale,
// or, for a weight stored without double quantization, the fp32 block absmax
// itself, kept one per block in the c1 array (c2 and the mean unused).
__device__ __forceinline__ float block_scale(int fmt, const int8_t *c2, const float *c1, float mean, int64_t j64,
                                             int bshift = 0) {
    const int64_t blk = j64 >> bshift;
    if (fmt == kNoDq) return c1[blk];
    return dq_scale(c2_value((uint8_t)c2[blk], fmt == kDqFp8), c1[blk >> 8], mean);
}

}  // namespace qnf4
