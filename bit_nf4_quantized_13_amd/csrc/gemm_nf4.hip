// Fused NF4-dequant GEMMs of the QLoRA layer on bf16 MFMA (gfx950):
//     forward:  Y  = X What^T + s U B^T     (U = X A^T)
//     dX:       dX = dY What  + s G A       (G = dY B)
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Double quantization and
// double dequantization": the frozen NF4 weights are reconstructed in BF16 by
// doubleDequant for the matrix multiplication (Y = X doubleDequant(c1, c2,
// W_NF4) + X L1 L2, adapter scale alpha/r from "How does alpha/r control
// adapter strength?"), and backpropagation runs through the reconstructed
// weights into the adapters only.
//
// Design (MI355X, one 256-thread workgroup per 512 x 128 output tile):
//  * Wave w owns output rows [128 w, 128 w + 128) and all 128 columns: 4 x 4
//    MFMA 32x32x16 tiles, fp32 accumulators in 256 AGPRs.  A 512-row tile means
//    every expanded weight feeds 512 rows, halving the expansion work per MFMA
//    relative to a 256-row tile.
//  * The activation tile (X or dY, 512 x 64 bf16) goes global -> LDS by DMA
//    (buffer_load ... lds, 1 KiB = 8 rows per instruction, XOR-swizzled 16-byte
//    chunks), double-buffered and issued one k-step ahead.
//  * The weight operand is expanded once per workgroup into a double-buffered
//    LDS bf16 tile [128 n][64 k]: the packed codes and block scales of step k
//    are loaded into registers two steps ahead, and the expansion of step k+1 --
//    BF16(C[code] * scale), bit-identical to qlora_nf4_dequantize -- runs
//    between the MFMAs of step k.  The 16 levels live in a VGPR (lane j holds
//    C[j % 16]) and are looked up with ds_bpermute, so the two operand rings
//    use exactly the 160 KiB of LDS.  Forward: a thread expands 32 consecutive
//    weights of one row.  dX (the reduction runs over W0 rows): a thread
//    expands 4 rows x 8 columns and writes them k-contiguous, i.e. the
//    transpose happens in registers.
//  * k order inside a 64-deep step is permuted (lane half h takes k = 32 h ..
//    32 h + 31 as four 8-wide MFMA slices) for both tiles.
//  * The adapter term is appended as extra k-steps with operands
//    [hi(sV) | lo(sV)] and [W' | W'] (hi = bf16(v), lo = bf16(v - hi)).
//  * Workgroups are renumbered so each XCD walks a contiguous run of tiles.
//
// MFMA v_mfma_f32_32x32x16_bf16 layout (wave64):
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) .. +7]
//   B (16 x 32): lane l holds B[8 (l / 32) .. +7][l % 32]
//   D (32 x 32): lane l, register v: D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
#include <type_traits>

#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int BM = 512, BN = 128, BK = 64;

struct GemmArgs {
    const uint16_t *a;      // activation operand [M x Kd] bf16 (X or dY)
    int64_t M, N, Kd;       // output [M x N]; forward: N = d, Kd = k; dX: N = k, Kd = d
    const uint8_t *codes;   // W0 [d x k] packed NF4
    const float *shat;      // dequantized block scales [d * k / 64]
    int64_t d, k;
    const float *ext_v;     // U (forward) or G (dX): [M x r] fp32
    const uint16_t *ext_w;  // B [d x r] (forward) or A [r x k] (dX)
    int r;
    float s;
    uint16_t *out;          // Y or dX [M x N] bf16
};

template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t comp(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Raw buffer resource over [base, base + bytes): 32-bit offsets, descriptor in
// scalar registers (readfirstlane: the operands are wave-uniform), reads past
// the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}

__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(const void *p) {
    return reinterpret_cast<__attribute__((address_space(3))) void *>(reinterpret_cast<uintptr_t>(p));
}
// global -> LDS transfer: lane l writes LDS bytes [dst + size*l, +size)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst), 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void *dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst), 4, voff, 0, 0, 0);
}

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t T) {
    const int64_t x = b % 8, y = b / 8, q = T / 8, rem = T % 8;
    return x * q + (x < rem ? x : rem) + y;
}

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector-memory operations
// outstanding, no LDS operation outstanding.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (0x7 << 4); }

// 8 codes of one dword (element i in nibble i) -> 8 levels C[code].  `lv`
// holds C[lane % 16] in every lane; ds_bpermute returns lane q's value for a
// byte index 4 q.  Byte j of e4 / o4 is 4 * nibble(2j) / 4 * nibble(2j+1); the
// masks go through an opaque v_and so the compiler keeps the one-instruction
// v_bfe_u32 byte extracts.
__device__ __forceinline__ uint32_t opaque_and(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}
// Marks the point where a value loaded steps earlier is first used: nothing
// computed from it can be hoisted above this point (where the load would
// still be in flight and its wait would stall the MFMA stream).
template <typename T>
__device__ __forceinline__ T pin(T v) {
    asm volatile("" : "+v"(v));
    return v;
}
struct Levels8 {
    float v[8];
};
__device__ __forceinline__ float level(uint32_t byte_index, int lv) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)byte_index, lv));
}
__device__ __forceinline__ Levels8 fetch_levels(uint32_t w, int lv) {
    const uint32_t e4 = opaque_and(w << 2, 0x3C3C3C3Cu);
    const uint32_t o4 = opaque_and(w >> 2, 0x3C3C3C3Cu);
    Levels8 l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        l.v[2 * j] = level(__builtin_amdgcn_ubfe(e4, 8 * j, 8), lv);
        l.v[2 * j + 1] = level(__builtin_amdgcn_ubfe(o4, 8 * j, 8), lv);
    }
    return l;
}

template <bool DX>
__global__ __launch_bounds__(256) void nf4_gemm_kernel(GemmArgs p, Nf4Consts tab) {
    __shared__ uint4 sA0[BM * 8], sA1[BM * 8];  // activation tiles (2 x 64 KiB)
    __shared__ uint4 sB0[BN * 8], sB1[BN * 8];  // expanded weight tiles (2 x 16 KiB)

    auto At = [&](auto S) __attribute__((always_inline)) -> uint4 * {
        if constexpr (decltype(S)::value == 0) return sA0;
        else return sA1;
    };
    auto Bt = [&](auto S) __attribute__((always_inline)) -> uint4 * {
        if constexpr (decltype(S)::value == 0) return sB0;
        else return sB1;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ml = lane & 31, h = lane >> 5;
    const int64_t tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
    const int64_t t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int64_t mt = t / tiles_n, nt = t % tiles_n;
    const int64_t m_base = mt * BM, n_base = nt * BN;
    const int64_t nK = (p.Kd + BK - 1) / BK;
    const int64_t kb = p.k / 64;  // NF4 blocks per W0 row

    // NF4 level table: lane j holds C[j % 16]
    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);

    // ---- activation tile: DMA, 8 rows per instruction ---------------------------
    // instruction i of wave w fills rows 8 g .. 8 g + 7, g = 16 w + i; lane l lands
    // in slot l = row 8 g + l/8, physical chunk l%8, logical chunk (l%8) ^ (l/8).
    // Rows past M read as zero.  Pieces past Kd (dX with d % 64 != 0) read the
    // next row's data: finite values that meet weight rows that are exactly zero.
    const int64_t rows_here = (p.M - m_base) < BM ? (p.M - m_base) : BM;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + m_base * p.Kd, rows_here * p.Kd * 2);
    const uint32_t voff_a =
        (uint32_t)((((128 * wave + (lane >> 3)) * p.Kd) + 8 * ((lane & 7) ^ (lane >> 3))) * 2);
    const uint32_t group_bytes = (uint32_t)(8 * p.Kd * 2);
    auto issue_a = [&](int64_t kt, auto S) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dma16(ra, At(S) + (16 * wave + i) * 64, voff_a + i * group_bytes + (uint32_t)kt * (BK * 2));
    };

    // ---- weight operand: codes and block scales, register loads -----------------
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes, p.d * p.k / 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.shat, p.d * kb * 4);
    // forward: thread t -> weight row n_base + t/2, k = 32 (t%2) .. +31 of the step
    //   (rows past d clamp to d-1: finite values in columns never stored)
    // dX: thread t -> W0 rows kt*64 + 4 (t/16) .. +3, columns n_base + 8 (t%16) .. +7
    //   (rows past d read as zero codes and zero scales: exactly zero weights)
    struct Wdata {
        uint32_t c[4];
        float s[4];
    };
    uint32_t voff_c[4], voff_s[4];
    uint32_t step_c, step_s;
    if constexpr (!DX) {
        int64_t n = n_base + (tid >> 1);
        n = n < p.d ? n : p.d - 1;
        voff_c[0] = (uint32_t)(n * kb * 32 + 16 * (tid & 1));
        voff_s[0] = (uint32_t)(n * kb * 4);
        step_c = 32;
        step_s = 4;
    } else {
        const int rg = tid >> 4, cg = tid & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t row = 4 * rg + e;
            voff_c[e] = (uint32_t)((row * p.k + n_base + 8 * cg) / 2);
            voff_s[e] = (uint32_t)((row * kb + (n_base + 8 * cg) / 64) * 4);
        }
        step_c = (uint32_t)(64 * p.k / 2);
        step_s = (uint32_t)(64 * kb * 4);
    }
    auto load_w = [&](int64_t kt, Wdata &wd) __attribute__((always_inline)) {
        const uint32_t k32 = (uint32_t)kt;
        if constexpr (!DX) {
            const uint4 c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, voff_c[0] + k32 * step_c, 0, 0));
            wd.c[0] = c.x; wd.c[1] = c.y; wd.c[2] = c.z; wd.c[3] = c.w;
            wd.s[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff_s[0] + k32 * step_s, 0, 0));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wd.c[e] = __builtin_amdgcn_raw_buffer_load_b32(rc, voff_c[e] + k32 * step_c, 0, 0);
                wd.s[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff_s[e] + k32 * step_s, 0, 0));
            }
        }
    };
    constexpr int kWloads = DX ? 8 : 2;  // register loads per thread per step

    // ---- expansion of one step's weight tile into LDS (4 slices) ----------------
    auto expand_slice = [&](const Wdata &wd, int c, auto SB) __attribute__((always_inline)) {
        if constexpr (!DX) {
            const Levels8 l = fetch_levels(pin(wd.c[c]), lv);
            const float sc = pin(wd.s[0]);
            uint4 o;
            o.x = pack_bf16x2(l.v[0] * sc, l.v[1] * sc);
            o.y = pack_bf16x2(l.v[2] * sc, l.v[3] * sc);
            o.z = pack_bf16x2(l.v[4] * sc, l.v[5] * sc);
            o.w = pack_bf16x2(l.v[6] * sc, l.v[7] * sc);
            Bt(SB)[swz(tid >> 1, 4 * (tid & 1) + c)] = o;
        } else {
            // columns 2c, 2c+1 of this thread's 8; 4 k-consecutive values each
            const int rg = tid >> 4, cg = tid & 15;
            uint32_t cw[4];
            float sc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cw[e] = pin(wd.c[e]);
                sc[e] = pin(wd.s[e]);
            }
#pragma unroll
            for (int f = 2 * c; f < 2 * c + 2; ++f) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = level(4 * __builtin_amdgcn_ubfe(cw[e], 4 * f, 4), lv) * sc[e];
                const uint2 o = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                const int n = 8 * cg + f;
                uint2 *dst = reinterpret_cast<uint2 *>(Bt(SB) + swz(n, rg >> 1)) + (rg & 1);
                *dst = o;
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

    auto read_a = [&](auto S, int ks, uint4 (&a)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = At(S)[swz(128 * wave + 32 * i + ml, 4 * h + ks)];
    };
    auto read_b = [&](auto S, int ks, uint4 (&b)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bt(S)[swz(32 * j + ml, 4 * h + ks)];
    };
    auto mfma_slice = [&](const uint4 (&a)[4], const uint4 (&b)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    };
    auto slices = [&](auto S, auto expand) __attribute__((always_inline)) {
        uint4 a[4], b[4];
        read_a(S, 0, a);
        read_b(S, 0, b);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 an[4], bn[4];
            if (ks < 3) {
                read_a(S, ks + 1, an);
                read_b(S, ks + 1, bn);
            }
            mfma_slice(a, b);
            expand(ks);
            if (ks < 3) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = an[i];
                    b[i] = bn[i];
                }
            }
        }
    };

    // One step kt (S = kt % 2): MFMAs on tiles S; A(kt+1) DMA into tile S^1 (last
    // read in step kt-1); expand step kt+1 (weights loaded two steps ago, `wcur`)
    // into weight tile S^1; load the weight data of step kt+3 into `wnext`.
    // Indices past the last step repeat it (uniform operation counts).  Barrier
    // once this wave's A DMA has landed (its newer weight loads may be in flight).
    auto step = [&](int64_t kt, auto S, const Wdata &wcur, Wdata &wnext) __attribute__((always_inline)) {
        using S1 = IC<1 - decltype(S)::value>;
        issue_a(kt + 1 < nK ? kt + 1 : nK - 1, S1{});
        load_w(kt + 3 < nK ? kt + 3 : nK - 1, wnext);
        slices(S, [&](int ks) __attribute__((always_inline)) { expand_slice(wcur, ks, S1{}); });
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWloads));
        __builtin_amdgcn_s_barrier();
    };
    auto last_step = [&](auto S) __attribute__((always_inline)) {
        slices(S, [&](int) __attribute__((always_inline)) {});
    };

    // ---- prologue: A(0) and weight tile 0 ready; weights of steps 1, 2 loaded ----
    Wdata w0, w1, w2;
    issue_a(0, IC<0>{});
    load_w(0, w0);
    load_w(nK > 1 ? 1 : nK - 1, w1);
    load_w(nK > 2 ? 2 : nK - 1, w2);
#pragma unroll
    for (int c = 0; c < 4; ++c) expand_slice(w0, c, IC<0>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- main k-loop: 2 steps per trip; three rotating weight-data registers ----
    // step kt consumes weights of kt+1 and loads kt+3: w1 -> (kt+1), w2 -> (kt+2), w0 -> (kt+3)
    int64_t kt = 0;
    for (; kt + 6 < nK; kt += 6) {
        step(kt + 0, IC<0>{}, w1, w0);
        step(kt + 1, IC<1>{}, w2, w1);
        step(kt + 2, IC<0>{}, w0, w2);
        step(kt + 3, IC<1>{}, w1, w0);
        step(kt + 4, IC<0>{}, w2, w1);
        step(kt + 5, IC<1>{}, w0, w2);
    }
    // remaining steps (kt % 6 == 0): all but the last are full steps
    const int64_t rem = nK - kt;  // 1 .. 6
    if (rem >= 2) step(kt + 0, IC<0>{}, w1, w0);
    if (rem >= 3) step(kt + 1, IC<1>{}, w2, w1);
    if (rem >= 4) step(kt + 2, IC<0>{}, w0, w2);
    if (rem >= 5) step(kt + 3, IC<1>{}, w1, w0);
    if (rem >= 6) step(kt + 4, IC<0>{}, w2, w1);
    if (rem & 1) last_step(IC<0>{});
    else last_step(IC<1>{});

    // ---- adapter term: extra k-steps [hi(sV) | lo(sV)] x [W' | W'] --------------
    // Both tiles go through LDS in the main-loop layouts: A' in sA0 (thread t
    // fills tile rows t, t + 256), W' in sB0 (thread t fills weight-tile row
    // t/2, k = 32 (t%2) .. +31).
    const int r = p.r, r2 = 2 * p.r;
    __builtin_amdgcn_s_waitcnt(0);  // no DMA still in flight
    for (int e0 = 0; e0 < r2; e0 += BK) {
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int row = tid + 256 * rr;
            int64_t m = m_base + row;
            m = m < p.M ? m : p.M - 1;
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
                uint32_t wv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t pr = 0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int kk = e0 + 8 * ch + 2 * e + hh;
                        uint32_t bits = 0;
                        if (kk < r2) {
                            const float v = p.s * p.ext_v[m * r + (kk < r ? kk : kk - r)];
                            const uint32_t hb = pack_bf16x2(v, 0.0f) & 0xFFFFu;
                            bits = kk < r ? hb : (pack_bf16x2(v - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
                        }
                        pr |= bits << (16 * hh);
                    }
                    wv[e] = pr;
                }
                sA0[swz(row, ch)] = uint4{wv[0], wv[1], wv[2], wv[3]};
            }
        }
        {
            int64_t n = n_base + (tid >> 1);
            n = n < p.N ? n : p.N - 1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t wv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t pr = 0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int kk = e0 + 32 * (tid & 1) + 8 * c + 2 * e + hh;
                        uint32_t bits = 0;
                        if (kk < r2) {
                            const int jj = kk < r ? kk : kk - r;
                            bits = DX ? p.ext_w[(int64_t)jj * p.k + n] : p.ext_w[n * r + jj];
                        }
                        pr |= bits << (16 * hh);
                    }
                    wv[e] = pr;
                }
                sB0[swz(tid >> 1, 4 * (tid & 1) + c)] = uint4{wv[0], wv[1], wv[2], wv[3]};
            }
        }
        __syncthreads();
        last_step(IC<0>{});
    }

    // ---- epilogue: fp32 -> bf16 ----------------------------------------------------
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n_base + 32 * j + ml;
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m_base + 128 * wave + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (m < p.M) p.out[m * p.N + n] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu);
            }
    }
}

// dequantized block scales: shat[j] = fp32(c2[j] / c1[j / 256]) + mean
__global__ __launch_bounds__(256) void dq_scales_kernel(const int8_t *__restrict__ c2,
                                                        const float *__restrict__ c1,
                                                        const float *__restrict__ mean_p, int64_t nb,
                                                        float *__restrict__ shat) {
    const float mean = *mean_p;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nb; j += (int64_t)gridDim.x * 256)
        shat[j] = dq_scale(c2[j], c1[j >> 8], mean);
}

hipError_t launch(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, const float *V,
                  const uint16_t *ext_w, int r, float s, uint16_t *out, float *shat, hipStream_t st) {
    const int64_t nb = w.d * w.k / 64;
    int64_t g = (nb + 255) / 256;
    if (g > 2048) g = 2048;
    hipLaunchKernelGGL(dq_scales_kernel, dim3((unsigned)g), dim3(256), 0, st, w.c2, w.c1, w.mean, nb, shat);
    GemmArgs p;
    p.a = a;
    p.M = M;
    p.N = dx ? w.k : w.d;
    p.Kd = dx ? w.d : w.k;
    p.codes = w.codes;
    p.shat = shat;
    p.d = w.d;
    p.k = w.k;
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
    return launch(false, w, x, M, U, B, r, s, Y, shat_ws, st);
}

hipError_t launch_gemm_dx(const Nf4Weights &w, const uint16_t *dy, int64_t M, const float *G,
                          const uint16_t *A, int r, float s, uint16_t *dX, float *shat_ws,
                          hipStream_t st) {
    return launch(true, w, dy, M, G, A, r, s, dX, shat_ws, st);
}

}  // namespace qnf4
