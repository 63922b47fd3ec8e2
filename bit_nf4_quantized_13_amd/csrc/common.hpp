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
    float pad_;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Dequantized block scale (doubleDequant): fp32(c2 / c1) + mean, two IEEE
// fp32 operations (the library is compiled with -ffp-contract=off).
__device__ __forceinline__ float dq_scale(int8_t c2, float c1, float mean) {
    return (float)c2 / c1 + mean;
}

// The scale of block blk of a stored weight: doubleDequant's dq_scale, or,
// for a weight stored without double quantization, the fp32 block absmax
// itself, kept one per block in the c1 array (c2 and the mean unused).
__device__ __forceinline__ float block_scale(bool dq, const int8_t *c2, const float *c1, float mean, int64_t blk) {
    return dq ? dq_scale(c2[blk], c1[blk >> 8], mean) : c1[blk];
}

}  // namespace qnf4
