// Decode-shaped forward (M <= 16 tokens): Y = X What^T + s U B^T, streaming the
// packed NF4 weights from HBM once.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Double quantization and
// double dequantization": What = doubleDequant(c1, c2, W_NF4) in BF16 feeds the
// matrix multiplication; with M <= 16 the product is bound by the bytes of the
// packed weights, so the weights are expanded in registers straight into the
// MFMA operand and never written anywhere.
//
// One 256-thread workgroup per 16 rows of W0.  The four waves split k into
// contiguous quarters (whole 128-deep groups).  Per group a wave reads its
// 16 rows x 64 code bytes with one coalesced 16-byte load per lane (four lanes
// per row) and moves them into the MFMA operand layout with ds_bpermute; the
// loads of the next group are in flight while the current one is expanded.
//
// MFMA v_mfma_f32_16x16x32_bf16, g = lane / 16, with the weight rows as the
// first operand: lane (n = lane % 16, g) holds What[n][8 codes], X the second
// operand: lane (m = lane % 16, g) holds X[m][8 values]; result lane (m, g),
// register v: D[n = 4 g + v][m].  Within a 128-deep group the k order is
// permuted so that lane group g takes the 32 contiguous k = 32 g .. 32 g + 31
// (one 16-byte code read per lane feeds 4 MFMAs); both operands agree.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int DEC_ROWS = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ float level(uint32_t addr, int lv) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)addr, lv));
}
// 4 * nibble e of w as a ds_bpermute byte address (bits 2..5; bits 0..1 are
// dropped by the lane-index division)
__device__ __forceinline__ uint32_t code_addr(uint32_t w, int e) {
    if (e == 0) return (w << 2) & 0x3Cu;
    if (e == 7) return w >> 26;
    return __builtin_amdgcn_ubfe(w, 4 * e - 2, 6);
}

struct DecodeArgs {
    const uint8_t *codes;  // W0 [d x k] packed NF4
    const int8_t *c2;
    const float *c1;
    const float *mean;
    int64_t d, k;
    const uint16_t *x;     // [M x k] bf16
    int64_t M;
    const float *U;        // [M x r] fp32
    const uint16_t *B;     // [d x r] bf16
    int r;
    float s;
    uint16_t *y;           // [M x d] bf16
};

// X slab in LDS: M rows x up to DEC_SLAB_K k, rows padded by 16 bytes so that
// the 16 fragment rows of one read land in 16 different bank groups.
constexpr int DEC_SLAB_K = 4096;
constexpr int DEC_MAX_GROUPS = 8;  // 128-deep groups per wave per slab (k per wave <= 1024)

template <int NT>  // 16-row weight tiles per workgroup (each wave does all of them)
__global__ __launch_bounds__(256) void nf4_decode_kernel(DecodeArgs p, Nf4Consts tab) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_smem[];
    __shared__ f32x4 red[4][NT][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * DEC_ROWS * NT;
    const int64_t kb = p.k / 64;
    const int64_t M = p.M;
    const int xrow_bytes = DEC_SLAB_K * 2 + 16;

    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);
    const float mean = *p.mean;

    const int64_t rows_here = (p.d - n0) < DEC_ROWS * NT ? (p.d - n0) : DEC_ROWS * NT;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes + n0 * (p.k / 2), rows_here * (p.k / 2));
    const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(p.c2 + n0 * kb, rows_here * kb);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, M * p.k * 2);
    // coalesced code read: lane l takes row l / 4 of the tile, bytes 16 (l % 4) ..
    // of the group's 64; the MFMA wants lane (n, g) = row n, piece g = lane 4 n + g
    const uint32_t code_voff = (uint32_t)((lane >> 2) * (p.k / 2) + 16 * (lane & 3));
    const int perm_addr = (4 * r16 + g) * 4;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t s0 = 0; s0 < p.k; s0 += DEC_SLAB_K) {
        const int64_t sk = (p.k - s0) < DEC_SLAB_K ? (p.k - s0) : DEC_SLAB_K;  // multiple of 64
        const int64_t sblocks = sk / 64;
        // this wave's blocks of the slab [b0, b1), whole 128-deep groups
        const int64_t per = ((sblocks + 3) / 4 + 1) / 2 * 2;
        const int64_t b0 = wave * per < sblocks ? wave * per : sblocks;
        const int64_t b1 = (wave + 1) * per < sblocks ? (wave + 1) * per : sblocks;
        const int ngroups = (int)((b1 - b0 + 1) / 2);

        // X slab -> LDS: row m, 16-byte pieces; transfer covers 64 pieces of one row
        if (s0 > 0) __syncthreads();  // previous slab's fragment reads done
        {
            const int64_t pieces = sk / 8;  // per row
            for (int64_t c = wave; c < M * ((pieces + 63) / 64); c += 4) {
                const int64_t m = c / ((pieces + 63) / 64), pc = (c % ((pieces + 63) / 64)) * 64;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx,
                    reinterpret_cast<__attribute__((address_space(3))) void *>(
                        reinterpret_cast<uintptr_t>(dyn_smem + m * xrow_bytes + pc * 16)),
                    16, (uint32_t)((m * p.k + s0 + (pc + lane) * 8) * 2), 0, 0, 0);
            }
        }
        // all codes and block constants of this wave's groups, in flight together
        uint4 cw[NT][DEC_MAX_GROUPS];
        int c2v[NT][DEC_MAX_GROUPS];
        float c1v[NT][DEC_MAX_GROUPS];
#pragma unroll
        for (int q = 0; q < DEC_MAX_GROUPS; ++q) {
            if (q >= ngroups) break;
            const int64_t bq = s0 / 64 + b0 + 2 * q;  // first block of the group (row-relative)
            const int64_t blk = bq + (g >> 1);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                cw[t][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rc, code_voff + (uint32_t)(16 * t * (p.k / 2)) + (uint32_t)(bq * 32), 0, 0));
                const int row = 16 * t + r16;
                c2v[t][q] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rs2, (uint32_t)(row * kb + blk), 0, 0);
                const bool ok = n0 + row < p.d;
                const int64_t jb = ok ? (n0 + row) * kb + (blk < kb ? blk : kb - 1) : 0;
                c1v[t][q] = p.c1[jb >> 8];
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // X slab in LDS
#pragma unroll
        for (int q = 0; q < DEC_MAX_GROUPS; ++q) {
            if (q >= ngroups) break;
            const bool live_k = b0 + 2 * q + (g >> 1) < b1;  // missing half of an odd tail
            // X[m][32 g + 8 i .. +7] of the group, m = r16 (rows past M: zero)
            const int64_t kx = (b0 + 2 * q) * 64 + 32 * g;
            uint4 xf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xf[i] = (r16 < M && live_k)
                            ? *reinterpret_cast<const uint4 *>(dyn_smem + r16 * xrow_bytes + (kx + 8 * i) * 2)
                            : uint4{0, 0, 0, 0};
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bool live = live_k && (n0 + 16 * t + r16 < p.d);
                const float sc = live ? dq_scale((int8_t)c2v[t][q], c1v[t][q], mean) : 0.0f;
                uint32_t cws[4];
                cws[0] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)cw[t][q].x);
                cws[1] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)cw[t][q].y);
                cws[2] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)cw[t][q].z);
                cws[3] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)cw[t][q].w);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float w8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) w8[e] = level(code_addr(cws[i], e), lv) * sc;
                    const uint4 wv{pack_bf16x2(w8[0], w8[1]), pack_bf16x2(w8[2], w8[3]), pack_bf16x2(w8[4], w8[5]),
                                   pack_bf16x2(w8[6], w8[7])};
                    acc[t] = mfma16(wv, xf[i], acc[t]);
                }
            }
        }
    }
    // cross-wave sum (fixed order), adapter term, bf16 store
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave < NT) {
        const int t = wave;
        const f32x4 v = (red[0][t][lane] + red[1][t][lane]) + (red[2][t][lane] + red[3][t][lane]);
        const int m = r16;
        if (m < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t n = n0 + 16 * t + 4 * g + e;
                if (n >= p.d) continue;
                float ad = 0.0f;
                for (int j = 0; j < p.r; ++j)
                    ad = __builtin_fmaf(p.U[(int64_t)m * p.r + j], bf16_bits_to_f32(p.B[n * p.r + j]), ad);
                const float out = v[e] + p.s * ad;
                p.y[(int64_t)m * p.d + n] = (uint16_t)(pack_bf16x2(out, 0.0f) & 0xFFFFu);
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const float *U,
                             const uint16_t *B, int r, float s, uint16_t *Y, hipStream_t st) {
    if (M > 16) return hipErrorInvalidValue;
    DecodeArgs a;
    a.codes = w.codes;
    a.c2 = w.c2;
    a.c1 = w.c1;
    a.mean = w.mean;
    a.d = w.d;
    a.k = w.k;
    a.x = x;
    a.M = M;
    a.U = U;
    a.B = B;
    a.r = r;
    a.s = s;
    a.y = Y;
    // two 16-row tiles per workgroup once there are enough rows to fill the chip
    const int nt = w.d >= 2 * DEC_ROWS * 512 ? 2 : 1;
    const dim3 grid((unsigned)((w.d + DEC_ROWS * nt - 1) / (DEC_ROWS * nt)));
    const size_t lds = (size_t)M * (DEC_SLAB_K * 2 + 16);
    if (nt == 2) hipLaunchKernelGGL(nf4_decode_kernel<2>, grid, dim3(256), lds, st, a, nf4_consts());
    else hipLaunchKernelGGL(nf4_decode_kernel<1>, grid, dim3(256), lds, st, a, nf4_consts());
    return hipGetLastError();
}

}  // namespace qnf4
