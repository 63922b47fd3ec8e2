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
//  * Wave w owns output rows [128 w, 128 w + 128) and all 128 columns: 8 x 8
//    MFMA 16x16x32 tiles, fp32 accumulators in 256 AGPRs.
//  * The activation operand (X or dY) goes straight from global memory into
//    registers in the MFMA operand layout: a wave reads only its own rows, so
//    no LDS staging is needed.  With the 16x16x32 layout one 16-byte load per
//    lane covers 16 rows x 64 bytes; the 16 loads of the next k-step are spread
//    one per MFMA group so the vector-memory path never blocks MFMA issue.
//  * The weight operand is expanded once per workgroup into LDS as bf16
//    [128 n][64 k] tiles -- BF16(C[code] * scale), bit-identical to
//    qlora_nf4_dequantize -- in a ring of 4 stages, two k-steps ahead of its
//    use, so one barrier per two k-steps suffices.  Packed codes and block
//    scales arrive in registers four steps ahead.  The 16 levels live in a
//    VGPR (lane j holds C[j % 16]) and are looked up with ds_bpermute; the
//    lookup, the multiply and the LDS write of each 8-weight piece are spread
//    over four MFMA groups so their latency hides behind the MFMAs.
//    Forward: a thread expands 32 consecutive weights of one W0 row.  dX (the
//    reduction runs over W0 rows): a thread expands 4 rows x 8 columns and
//    writes them k-contiguous, i.e. the transpose happens in registers.
//  * The MFMA takes the weight fragment as its first operand, so each lane
//    ends with 4 consecutive output columns of one row (8-byte stores).
//  * The adapter term is appended as extra k-steps whose operands the
//    preparation kernel lays out in memory: [hi(sV) | lo(sV) | 0] and
//    [W' | W' | 0] (hi = bf16(v), lo = bf16(v - hi), rows padded to a
//    multiple of 64).
//  * Workgroups are renumbered so each XCD walks a contiguous run of tiles.
//
// MFMA v_mfma_f32_16x16x32_bf16 layout (wave64), g = lane / 16:
//   first operand  (16 x 32): lane l holds P[l % 16][8 g .. 8 g + 7]
//   second operand (32 x 16): lane l holds Q[8 g .. 8 g + 7][l % 16]
//   result         (16 x 16): lane l, register v: D[4 g + v][l % 16]
// k order inside a 64-deep step: slice s (32 k) lane group g takes
// k = 32 s + 8 g .. + 7, identically for both operands.
#include <type_traits>

#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int BM = 512, BN = 128, BK = 64;
constexpr int NTHREADS = 512;                 // 8 waves, two per SIMD
constexpr int WM = BM / (NTHREADS / 64);      // rows per wave (64)
constexpr int MI = WM / 16;                   // 16-row MFMA tiles per wave (4)
constexpr int A_STAGE = BM * BK * 2;          // 64 KiB activation tile
constexpr int B_STAGE = BN * BK * 2;          // 16 KiB weight tile

struct GemmArgs {
    const uint16_t *a;      // activation operand [M x Kd] bf16 (X or dY)
    int64_t M, N, Kd;       // output [M x N]; forward: N = d, Kd = k; dX: N = k, Kd = d
    const uint8_t *codes;   // W0 [d x k] packed NF4
    const float *shat;      // dequantized block scales [d * k / 64]
    int64_t d, k;
    const uint16_t *ext_a;  // [M x Ke] bf16: [hi(s V) | lo(s V) | 0]
    const uint16_t *ext_b;  // [N x Ke] bf16: [W' | W' | 0]
    int64_t Ke;             // multiple of 64
    const uint16_t *wbf;    // dequantized weight operand [N x ldw] bf16 (non-expanding kernel)
    int64_t ldw;            // forward: What [d x k], ldw = k; dX: What^T [k x ldw], ldw = d rounded up to 64
    uint16_t *out;          // Y or dX [M x N] bf16
};

template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// c += a b in place.  Written as one instruction with the accumulator tied to
// an AGPR tuple: with 64 accumulator tiles the register allocator otherwise
// splits the chains and shuttles them between AGPRs and VGPRs.  The operands
// come straight from memory loads (no VALU producer), and each accumulator is
// touched once per 64 MFMAs, so no extra wait states are needed.
__device__ __forceinline__ void mfma16_acc(uint4 a, uint4 b, f32x4 &c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(c)
                 : "v"(__builtin_bit_cast(u32x4, a)), "v"(__builtin_bit_cast(u32x4, b)));
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
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Workgroup -> output tile.  Consecutive workgroups go to the 8 XCDs in turn;
// each XCD takes a contiguous run u of the tile order, and the tile order walks
// bands of 8 tile columns, all tile rows of a band before the next band.  An
// XCD's concurrently running tiles then share 4-8 activation slabs and 8
// weight slabs in its L2 instead of one slab of one and 32 of the other.
__device__ __forceinline__ void tile_of(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t &mt, int64_t &nt) {
    const int64_t T = tiles_m * tiles_n;
    const int64_t x = b % 8, y = b / 8, q = T / 8, rem = T % 8;
    const int64_t u = x * q + (x < rem ? x : rem) + y;
    constexpr int64_t GN = 8;
    const int64_t band = u / (tiles_m * GN);
    const int64_t w = (tiles_n - band * GN) < GN ? (tiles_n - band * GN) : GN;
    const int64_t r = u - band * tiles_m * GN;
    mt = r / w;
    nt = band * GN + r % w;
}

// Marks the point where a value loaded steps earlier is first used: nothing
// computed from it can be hoisted above this point (where the load would
// still be in flight and its wait would stall the MFMA stream).
template <typename T>
__device__ __forceinline__ T pin(T v) {
    asm volatile("" : "+v"(v));
    return v;
}
// C[code] for a byte address whose bits 2..5 hold the code: `lv` holds
// C[lane % 16] in every lane and ds_bpermute returns lane (addr / 4)'s value.
__device__ __forceinline__ float level(uint32_t addr, int lv) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)addr, lv));
}
// 4 * nibble e of w as a ds_bpermute byte address (bits 2..5; bits 0..1 are
// dropped by the lane-index division): bits 4e-2 .. 4e+3 of w.
__device__ __forceinline__ uint32_t code_addr(uint32_t w, int e) {
    if (e == 0) return (w << 2) & 0x3Cu;
    if (e == 7) return w >> 26;
    return __builtin_amdgcn_ubfe(w, 4 * e - 2, 6);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ uint4 lds_read16(uint32_t byte_addr) {
    __builtin_assume((byte_addr & 15) == 0);
    return __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4 *>(byte_addr));
}
__device__ __forceinline__ void lds_write16(uint32_t byte_addr, uint4 v) {
    __builtin_assume((byte_addr & 15) == 0);
    *reinterpret_cast<lds_u32x4 *>(byte_addr) = __builtin_bit_cast(u32x4, v);
}
__device__ __forceinline__ void lds_write8(uint32_t byte_addr, uint2 v) {
    *reinterpret_cast<lds_u32x2 *>(byte_addr) = __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ void lds_write4(uint32_t byte_addr, uint32_t v) {
    *reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(byte_addr) = v;
}

// global -> LDS transfer of 16 bytes per lane: lane l writes LDS bytes
// [dst + 16 l, +16) (dst is wave-uniform and goes to M0)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, reinterpret_cast<__attribute__((address_space(3))) void *>(reinterpret_cast<uintptr_t>(dst)), 16, voff,
        soff, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding): at most `vm` vector-memory operations
// outstanding, no LDS operation outstanding.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (0x7 << 4); }
// at most `vm` vector-memory operations outstanding, LDS operations untouched
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// EXPAND: the weight tile of each k-step is expanded from the packed codes in
// the workgroup (one expansion per output tile row: the choice when the grid
// has a single tile row).  Otherwise it is transferred like the activation
// tile from a dequantized bf16 copy written once per call.
template <bool DX, bool EXPAND>
__global__ __launch_bounds__(NTHREADS) void nf4_gemm_kernel(GemmArgs p, Nf4Consts tab) {
    // Two stages of the activation tile [512 rows][64 k] and of the weight tile
    // [128 rows][64 k] (160 KiB).  One object per buffer so that the compiler can
    // tell them apart when it places waits for the global->LDS transfers.
    __shared__ u32x4 sA0[A_STAGE / 16], sA1[A_STAGE / 16];
    __shared__ u32x4 sB0[B_STAGE / 16], sB1[B_STAGE / 16];
    auto Aof = [&](auto S) __attribute__((always_inline)) -> u32x4 * {
        if constexpr (decltype(S)::value == 0) return sA0;
        else return sA1;
    };
    auto Bof = [&](auto S) __attribute__((always_inline)) -> u32x4 * {
        if constexpr (decltype(S)::value == 0) return sB0;
        else return sB1;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + BM - 1) / BM;
    int64_t mt, nt;
    tile_of(blockIdx.x, tiles_m, tiles_n, mt, nt);
    const int64_t m_base = mt * BM, n_base = nt * BN;
    const int64_t nK = (p.Kd + BK - 1) / BK;
    const int64_t kb = p.k / 64;  // NF4 blocks per W0 row

    // NF4 level table: lane j holds C[j % 16]
    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);

    // ---- activation tile: global -> LDS transfers of 8 rows x 128 B ---------------
    // Wave w moves and reads only its own rows WM w .. WM w + WM - 1 (transfer b:
    // rows WM w + 8 b ..).  Lane l lands in row 8 b + l / 8, physical chunk l % 8,
    // which holds logical chunk (l % 8) ^ ((row >> 1) & 7) = (l % 8) ^ ((l / 16 + 4 b) & 7).
    // Rows past M read as zero.  Pieces past Kd (dX with d % 64 != 0) read the
    // next row's data: finite values that meet weight rows that are exactly zero.
    const int64_t rows_here = (p.M - m_base) < BM ? (p.M - m_base) : BM;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + m_base * p.Kd, rows_here * p.Kd * 2);
    const int dma_row = WM * wave + (lane >> 3);  // + 8 b
    const uint32_t voff_a0 = (uint32_t)(((int64_t)dma_row * p.Kd + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
    const uint32_t voff_a1 = (uint32_t)(((int64_t)dma_row * p.Kd + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
    const uint32_t row8_bytes = (uint32_t)(8 * p.Kd * 2);
    auto issue_a = [&](int64_t kt, auto S, int b) __attribute__((always_inline)) {
        dma16(ra, Aof(S) + (WM * wave + 8 * b) * 8, (b & 1) ? voff_a1 : voff_a0,
              (uint32_t)b * row8_bytes + (uint32_t)kt * (BK * 2));
    };
    // fragment reads (A: row WM w + 16 i + r16; B: row 16 j + r16; chunk 4 s + g),
    // physical chunk (4 s + g) ^ ((r16 >> 1) & 7) in both tiles
    const int frag0 = r16 * 8 + ((0 + g) ^ ((r16 >> 1) & 7));  // in 16-byte units
    const int frag1 = r16 * 8 + ((4 + g) ^ ((r16 >> 1) & 7));
    const int arow = WM * wave * 8;
    auto read_a = [&](auto S, int s, int i) __attribute__((always_inline)) -> uint4 {
        return __builtin_bit_cast(uint4, Aof(S)[arow + (s ? frag1 : frag0) + 128 * i]);
    };

    // ---- weight tiles [128 n][64 k], same chunk layout ------------------------------
    auto read_b = [&](auto S, int s, int j) __attribute__((always_inline)) -> uint4 {
        return __builtin_bit_cast(uint4, Bof(S)[(s ? frag1 : frag0) + 128 * j]);
    };
    // transfer (non-expanding kernel): rows n_base .., 8 per transfer, wave w moves
    // rows 16 w .. 16 w + 15; rows past N read as zero
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(p.wbf + n_base * p.ldw, EXPAND ? 0 : ((p.N - n_base) < BN ? (p.N - n_base) : BN) * p.ldw * 2);
    const int wrow = 16 * wave + (lane >> 3);  // + 8 u
    const uint32_t voff_w0 = (uint32_t)(((int64_t)wrow * p.ldw + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
    const uint32_t voff_w1 = (uint32_t)(((int64_t)wrow * p.ldw + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
    const uint32_t wrow8_bytes = (uint32_t)(8 * p.ldw * 2);
    auto issue_w = [&](int64_t kt, auto S, int u) __attribute__((always_inline)) {
        dma16(rw, Bof(S) + (16 * wave + 8 * u) * 8, u ? voff_w1 : voff_w0,
              (uint32_t)u * wrow8_bytes + (uint32_t)kt * (BK * 2));
    };

    // ---- weight data (expanding kernel): codes and block scales, register loads ------
    // forward: thread t -> weight row n_base + t/4, k = 16 (t%4) .. +15 of the step
    //   (rows past d clamp to d-1: finite values in columns never stored)
    // dX: thread t -> W0 rows kt*64 + 2 (t/16) .. +1, columns n_base + 8 (t%16) .. +7
    //   (rows past d read as zero codes and zero scales: exactly zero weights)
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes, p.d * p.k / 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.shat, p.d * kb * 4);
    struct Wdata {
        uint32_t c[2];
        float s[2];
    };
    uint32_t voff_c, voff_s, step_c, step_s, row_c = 0, row_s = 0;
    uint32_t wr_off[8];  // stage-relative LDS offsets of this thread's expansion writes
                         // (forward: 16-byte units; dX: 4-byte units)
    if constexpr (!DX) {
        int64_t n = n_base + (tid >> 2);
        n = n < p.d ? n : p.d - 1;
        voff_c = (uint32_t)(n * kb * 32 + 8 * (tid & 3));
        voff_s = (uint32_t)(n * kb * 4);
        step_c = 32;
        step_s = 4;
        const int row = tid >> 2;
#pragma unroll
        for (int c = 0; c < 2; ++c) wr_off[c] = (uint32_t)(row * 8 + ((2 * (tid & 3) + c) ^ ((row >> 1) & 7)));
#pragma unroll
        for (int c = 2; c < 8; ++c) wr_off[c] = 0;
    } else {
        const int rg = tid >> 4, cg = tid & 15;
        voff_c = (uint32_t)(((int64_t)(2 * rg) * p.k + n_base + 8 * cg) / 2);
        voff_s = (uint32_t)(((int64_t)(2 * rg) * kb + (n_base + 8 * cg) / 64) * 4);
        row_c = (uint32_t)(p.k / 2);
        row_s = (uint32_t)(kb * 4);
        step_c = (uint32_t)(64 * p.k / 2);
        step_s = (uint32_t)(64 * kb * 4);
        // column f of the thread's 8 -> tile row n = 8 cg + f, k = 2 rg, 2 rg + 1
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const int n = 8 * cg + f;
            wr_off[f] = (uint32_t)(n * 32 + 4 * ((rg >> 2) ^ ((n >> 1) & 7)) + (rg & 3));
        }
    }
    auto load_w = [&](int64_t kt, Wdata &wd) __attribute__((always_inline)) {
        const uint32_t k32 = (uint32_t)kt;
        if constexpr (!DX) {
            const uint2 c = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, voff_c, k32 * step_c, 0));
            wd.c[0] = c.x;
            wd.c[1] = c.y;
            wd.s[0] = __uint_as_float(load4(rs, voff_s, k32 * step_s));
            wd.s[1] = 0.0f;
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                wd.c[e] = load4(rc, voff_c, k32 * step_c + e * row_c);
                wd.s[e] = __uint_as_float(load4(rs, voff_s, k32 * step_s + e * row_s));
            }
        }
    };

    constexpr int kWloads = EXPAND ? (DX ? 4 : 2) : 0;  // register loads of weight data per step

    // One 8-weight piece of the expansion in three phases spread over MFMA
    // groups: 0 = code lookups, 1 = scale multiplies, 2 = bf16 pack + LDS write.
    // forward piece c: 8 consecutive k of one row (code word c).
    // dX piece c: columns 4c .. 4c+3 of the thread's 8, two k-consecutive rows each.
    float lvl[8];
    auto expand_phase = [&](const Wdata &wd, int c, int phase, u32x4 *stage) __attribute__((always_inline)) {
        if constexpr (!DX) {
            if (phase == 0) {
                const uint32_t x = pin(wd.c[c]);
#pragma unroll
                for (int e = 0; e < 8; ++e) lvl[e] = level(code_addr(x, e), lv);
            } else if (phase == 1) {
                const float sc = pin(wd.s[0]);
#pragma unroll
                for (int e = 0; e < 8; ++e) lvl[e] = lvl[e] * sc;
            } else {
                const uint4 o{pack_bf16x2(lvl[0], lvl[1]), pack_bf16x2(lvl[2], lvl[3]),
                              pack_bf16x2(lvl[4], lvl[5]), pack_bf16x2(lvl[6], lvl[7])};
                stage[wr_off[c]] = __builtin_bit_cast(u32x4, o);
            }
        } else {
            if (phase == 0) {
                const uint32_t x0 = pin(wd.c[0]), x1 = pin(wd.c[1]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    lvl[2 * q] = level(code_addr(x0, 4 * c + q), lv);
                    lvl[2 * q + 1] = level(code_addr(x1, 4 * c + q), lv);
                }
            } else if (phase == 1) {
                const float s0 = pin(wd.s[0]), s1 = pin(wd.s[1]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    lvl[2 * q] = lvl[2 * q] * s0;
                    lvl[2 * q + 1] = lvl[2 * q + 1] * s1;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    reinterpret_cast<uint32_t *>(stage)[wr_off[4 * c + q]] = pack_bf16x2(lvl[2 * q], lvl[2 * q + 1]);
            }
        }
    };

    // Accumulators: first written by step 0 (MFMA with a zero addend), then
    // accumulated in place (mfma16_acc).
    f32x4 acc[MI][8];
    uint4 af[2][MI];   // activation fragments: current slice, next slice
    uint4 bq[4];       // weight fragments, two groups ahead
    Wdata w0, w1, w2;  // weight data, rotating over three steps

    auto Wset = [&](auto W) __attribute__((always_inline)) -> Wdata & {
        if constexpr (decltype(W)::value == 0) return w0;
        else if constexpr (decltype(W)::value == 1) return w1;
        else return w2;
    };

    // One k-step kt with R = kt % 6 (every buffer index static), S = kt % 2:
    //  * MFMAs on tiles A[S], B[S]; A fragments of slice 1 read during slice 0;
    //  * transfers A(kt+1) into A[S^1];
    //  * non-expanding: transfers the weight tile of step kt+1 into B[S^1];
    //    expanding: loads the weight data of step kt+3 into set kt % 3 and
    //    expands step kt+1 (set (kt+1) % 3) into B[S^1];
    //  * waits for its own transfers, reads the first A fragments of step kt+1,
    //    then meets the other waves at the barrier.
    // Indices past the last step repeat it (uniform operation counts).
    auto step = [&](int64_t kt, auto RR, auto FIRST) __attribute__((always_inline)) {
        constexpr int R = decltype(RR)::value;
        constexpr bool first = decltype(FIRST)::value != 0;
        using S = IC<R % 2>;
        using S1 = IC<1 - R % 2>;
        const Wdata &wc = Wset(IC<(R + 1) % 3>{});
        Wdata &wl = Wset(IC<R % 3>{});
        u32x4 *const st_w = Bof(S1{});
        const int64_t kn = kt + 1 < nK ? kt + 1 : nK - 1;
        const int64_t kw = kt + 3 < nK ? kt + 3 : nK - 1;
#pragma unroll
        for (int grp = 0; grp < 16; ++grp) {
            const int s = grp >> 3, j = grp & 7;
            if (grp + 2 < 16) bq[(grp + 2) & 3] = read_b(S{}, (grp + 2) >> 3, (grp + 2) & 7);
            if (grp == 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i) af[1][i] = read_a(S{}, 1, i);
            }
            if constexpr (EXPAND) {
                if (grp < 8) issue_a(kn, S1{}, grp);
                if (grp == 8) load_w(kw, wl);  // after the transfers: the end-of-step wait counts on it
                if (j == 1) expand_phase(wc, s, 0, st_w);
                if (j == 4) expand_phase(wc, s, 1, st_w);
                if (j == 6) expand_phase(wc, s, 2, st_w);
            } else {
                if (grp < 2) issue_w(kn, S1{}, grp);
                if (grp >= 2 && grp < 10) issue_a(kn, S1{}, grp - 2);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (first && s == 0) acc[i][j] = mfma16(bq[grp & 3], af[s][i], f32x4{0.f, 0.f, 0.f, 0.f});
                else mfma16_acc(bq[grp & 3], af[s][i], acc[i][j]);
            }
            sched_fence();
        }
        // this wave's transfers of step kt+1 landed (the weight-data loads of
        // this step, issued after them, may still be in flight); expansion
        // writes done
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWloads));
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = read_a(S1{}, 0, i);
        __builtin_amdgcn_s_barrier();
        bq[0] = read_b(S1{}, 0, 0);
        bq[1] = read_b(S1{}, 0, 1);
        sched_fence();
    };

    // ---- prologue: A(0) and weight tile 0 in LDS; weight data of steps 1, 2 loaded ----
    if constexpr (EXPAND) {
        load_w(0, w0);
#pragma unroll
        for (int b = 0; b < 8; ++b) issue_a(0, IC<0>{}, b);
        load_w(nK > 1 ? 1 : 0, w1);
        load_w(nK > 2 ? 2 : nK - 1, w2);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ph = 0; ph < 3; ++ph) expand_phase(w0, c, ph, sB0);
    } else {
        issue_w(0, IC<0>{}, 0);
        issue_w(0, IC<0>{}, 1);
#pragma unroll
        for (int b = 0; b < 8; ++b) issue_a(0, IC<0>{}, b);
    }
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int i = 0; i < MI; ++i) af[0][i] = read_a(IC<0>{}, 0, i);
    __syncthreads();
    bq[0] = read_b(IC<0>{}, 0, 0);
    bq[1] = read_b(IC<0>{}, 0, 1);

    // ---- main k-loop: step 0 peeled, then six steps per trip -------------------------
    step(0, IC<0>{}, IC<1>{});
    int64_t kt = 1;
    for (; kt + 6 <= nK; kt += 6) {
        step(kt + 0, IC<1>{}, IC<0>{});
        step(kt + 1, IC<2>{}, IC<0>{});
        step(kt + 2, IC<3>{}, IC<0>{});
        step(kt + 3, IC<4>{}, IC<0>{});
        step(kt + 4, IC<5>{}, IC<0>{});
        step(kt + 5, IC<0>{}, IC<0>{});
    }
    if (kt < nK) step(kt, IC<1>{}, IC<0>{});
    if (kt + 1 < nK) step(kt + 1, IC<2>{}, IC<0>{});
    if (kt + 2 < nK) step(kt + 2, IC<3>{}, IC<0>{});
    if (kt + 3 < nK) step(kt + 3, IC<4>{}, IC<0>{});
    if (kt + 4 < nK) step(kt + 4, IC<5>{}, IC<0>{});

    // ---- adapter term: Ke/64 extra k-steps, operands laid out in memory ------------
    {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rea = make_rsrc(p.ext_a + m_base * p.Ke, rows_here * p.Ke * 2);
        const uint32_t voff_e0 = (uint32_t)(((int64_t)dma_row * p.Ke + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
        const uint32_t voff_e1 = (uint32_t)(((int64_t)dma_row * p.Ke + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
        const uint32_t row8_e = (uint32_t)(8 * p.Ke * 2);
        // weight-side operand rows n_base .. +127 (clamped to N-1): transfer u of
        // wave w covers rows 16 w + 8 u .. + 7
        const __amdgpu_buffer_rsrc_t reb = make_rsrc(p.ext_b, p.N * p.Ke * 2);
        uint32_t voff_eb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = 16 * wave + 8 * u + (lane >> 3);
            int64_t n = n_base + row;
            n = n < p.N ? n : p.N - 1;
            voff_eb[u] = (uint32_t)((n * p.Ke + 8 * ((lane & 7) ^ ((row >> 1) & 7))) * 2);
        }
        const int64_t nE = p.Ke / BK;
        for (int64_t e = 0; e < nE; ++e) {
#pragma unroll
            for (int b = 0; b < 8; ++b)
                dma16(rea, sA0 + (WM * wave + 8 * b) * 8, (b & 1) ? voff_e1 : voff_e0,
                      (uint32_t)b * row8_e + (uint32_t)e * (BK * 2));
#pragma unroll
            for (int u = 0; u < 2; ++u) dma16(reb, sB0 + (16 * wave + 8 * u) * 8, voff_eb[u], (uint32_t)e * (BK * 2));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int i = 0; i < MI; ++i) af[0][i] = read_a(IC<0>{}, s, i);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint4 b = read_b(IC<0>{}, s, j);
#pragma unroll
                    for (int i = 0; i < MI; ++i) mfma16_acc(b, af[0][i], acc[i][j]);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // the epilogue reads the accumulators with VALU instructions: let the
        // last MFMAs (inline asm, invisible to the hazard recognizer) drain
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    }

    // ---- epilogue: lane holds D[m = 16 i + r16][n = 16 j + 4 g .. + 3] ----------------
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int64_t m = m_base + WM * wave + 16 * i + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = n_base + 16 * j + 4 * g;
            if (n >= p.N) continue;
            const uint2 o{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
            *reinterpret_cast<uint2 *>(p.out + m * p.N + n) = o;
        }
    }
}

// Transposed dequantized weight operand for the non-expanding dX GEMM: What^T
// [k x ldw] with zero columns d .. ldw-1, bf16, bit-identical to
// qlora_nf4_dequantize (the block scale is doubleDequant's, computed here from
// c2, c1 and the mean).  One workgroup per 64 W0 rows x 256 columns; thread t
// expands an 8 x 8 block: rows 8 (t % 8) .., columns 8 (t / 8) .. (inside one
// NF4 block, so one scale per row).  Code reads are 32 contiguous bytes per
// row for 8 lanes; the 8 x 8 block is transposed in registers (v_perm) and
// stored as 16-byte column pieces, so no LDS is involved and every store is a
// contiguous 128-byte row segment per 8 lanes.  (The forward's What, laid out
// like the codes, is written by a plain stride loop in prep_kernel.)  Narrower
// blocks (8 x 4) and two tiles per workgroup with the next one's loads
// overlapping were both slower.
__device__ __forceinline__ void dequant_tile_t(int64_t bid, const uint8_t *__restrict__ codes, int fmt, int bshift,
                                               const int8_t *__restrict__ c2, const float *__restrict__ c1,
                                               float mean, int64_t d, int64_t k, int64_t ldw, const Nf4Consts &tab,
                                               uint16_t *__restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t ct = (k + 255) / 256;
    const int64_t tk = bid % ct, td = bid / ct;
    const int ng = tid & 7, kg = tid >> 3;
    const int64_t n0 = td * 64 + 8 * ng;   // first of this thread's 8 W0 rows
    const int64_t k0 = tk * 256 + 8 * kg;  // first of its 8 columns
    if (k0 >= k) return;                   // k % 64 == 0: whole 8-column groups
    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);
    const int64_t kb = k / 64;
    uint32_t cw[8];
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t n = n0 + e;
        const int64_t jb = n * kb + k0 / 64;
        cw[e] = n < d ? *reinterpret_cast<const uint32_t *>(codes + n * (k / 2) + k0 / 2) : 0u;
        sc[e] = n < d ? block_scale(fmt, c2, c1, mean, jb, bshift) : 0.0f;
    }
    // v[e][q]: row e, columns 2 q, 2 q + 1 (bf16 pair)
    uint32_t v[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = pack_bf16x2(level(code_addr(cw[e], 2 * q), lv) * sc[e],
                                           level(code_addr(cw[e], 2 * q + 1), lv) * sc[e]);
            v[e][q] = n0 + e < d ? x : 0u;  // rows past d: zero columns of What^T
        }
    // column c of the block: rows 0..7 packed as 4 bf16 pairs
    // (rows 2 e2, 2 e2 + 1) = low halves (c even) or high halves (c odd)
    // of v[2 e2][c / 2] and v[2 e2 + 1][c / 2]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
            o[e2] = (c & 1) ? __builtin_amdgcn_perm(v[2 * e2 + 1][c >> 1], v[2 * e2][c >> 1], 0x07060302u)
                            : __builtin_amdgcn_perm(v[2 * e2 + 1][c >> 1], v[2 * e2][c >> 1], 0x05040100u);
        *reinterpret_cast<uint4 *>(out + (k0 + c) * ldw + n0) = uint4{o[0], o[1], o[2], o[3]};
    }
}

// Preparation of one dequant-GEMM call, one launch over consecutive
// workgroup ranges (each range may be empty):
//   shat[j] = fp32(c2[j] / c1[j / 256]) + mean         (j < nb; the expanding GEMM)
//   ext_a[m][c] = hi(s V[m][c]), lo(s V[m][c - r]) or 0 by column  (M x Ke)
//   ext_b[n][c] = W'[n][c mod r] for c < 2r, else 0                (N x Ke)
//   the dequantized weight operand, What or What^T                 (the non-expanding GEMM)
//   up to two column reductions out = scale sum_splits part        (the dX call's dB, dA)
// where W'[n][j] = B[n][j] (forward, B [d x r]) or A[j][n] (dX, A [r x k]).
struct PrepArgs {
    int fmt;     // ScaleFormat of the block constants
    int bshift;  // blocks of 64 << bshift weights
    const int8_t *c2;
    const float *c1;
    const float *mean;
    int64_t nb;
    float *shat;
    const float *V;
    int64_t M;
    int r;
    float s;
    uint16_t *ext_a;
    const uint16_t *W;
    int64_t N;
    uint16_t *ext_b;
    int64_t Ke;
    const uint8_t *codes;  // dequantized operand
    int64_t d, k, ldw;
    uint16_t *wbf;
    ColsReduceJob red[2];
    int64_t g_shat, g_a, g_b, g_t, g_r0;  // workgroups per range (the second reduction takes the rest)
};

// out = scale * sum over splits of part[sp][j][n] (split order), e = (j, n)
// with n fastest; stored out[n][j] (trans = 0) or out[j][n] (trans = 1)
__device__ __forceinline__ void cols_reduce(const ColsReduceJob &jb, int64_t e) {
    const int64_t RN = (int64_t)jb.R * jb.N;
    if (e >= RN) return;
    constexpr int kMax = 32;
    float v[kMax];
    const int sp = jb.splits;
#pragma unroll
    for (int q = 0; q < kMax; ++q) v[q] = q < sp ? jb.part[(int64_t)q * RN + e] : 0.0f;
    float sum = v[0];
#pragma unroll
    for (int q = 1; q < kMax; ++q)
        if (q < sp) sum += v[q];
    for (int q = kMax; q < sp; ++q) sum += jb.part[(int64_t)q * RN + e];
    const int64_t j = e / jb.N, n = e - j * jb.N;
    if (jb.trans) jb.out[e] = jb.scale * sum;
    else jb.out[n * jb.R + j] = jb.scale * sum;
}

template <bool DX>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a, Nf4Consts tab) {
    int64_t b = blockIdx.x;
    if (b < a.g_shat) {
        const int64_t x = b * 256 + threadIdx.x;
        if (x < a.nb) a.shat[x] = block_scale(a.fmt, a.c2, a.c1, a.fmt != kNoDq ? *a.mean : 0.0f, x, a.bshift);
        return;
    }
    b -= a.g_shat;
    if (b < a.g_a + a.g_b) {
        const uint32_t cgs = (uint32_t)(a.Ke / 8);  // 8-column groups per row
        const bool is_a = b < a.g_a;
        const int64_t x = (b - (is_a ? 0 : a.g_a)) * 256 + threadIdx.x;
        const int64_t rows = is_a ? a.M : a.N;
        const int64_t row = x / cgs;
        if (row >= rows) return;
        const int c0 = (int)(x - row * cgs) * 8;
        uint32_t v[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t pr = 0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = c0 + 2 * h + q;
                uint32_t bits = 0;
                if (c < 2 * a.r) {
                    const int jj = c < a.r ? c : c - a.r;
                    if (is_a) {
                        const float f = a.s * a.V[row * a.r + jj];
                        const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
                        bits = c < a.r ? hb : (pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
                    } else {
                        bits = DX ? a.W[(int64_t)jj * a.N + row] : a.W[row * a.r + jj];
                    }
                }
                pr |= bits << (16 * q);
            }
            v[h] = pr;
        }
        uint16_t *dst = (is_a ? a.ext_a : a.ext_b) + row * a.Ke + c0;
        *reinterpret_cast<uint4 *>(dst) = uint4{v[0], v[1], v[2], v[3]};
        return;
    }
    b -= a.g_a + a.g_b;
    if (b < a.g_t) {
        const float mean = a.fmt != kNoDq ? *a.mean : 0.0f;
        if constexpr (DX) {
            dequant_tile_t(b, a.codes, a.fmt, a.bshift, a.c2, a.c1, mean, a.d, a.k, a.ldw, tab, a.wbf);
        } else {
            // What [d x k], row-major like the codes: a stride loop over 8-weight
            // items (one code dword -> one 16-byte store), the levels in LDS
            __shared__ float lut[16];
            if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
            __syncthreads();
            const int64_t items = a.d * a.k / 8;
            const uint32_t *codes4 = reinterpret_cast<const uint32_t *>(a.codes);
            uint4 *out = reinterpret_cast<uint4 *>(a.wbf);
            for (int64_t i = b * 256 + threadIdx.x; i < items; i += a.g_t * 256) {
                const uint32_t c = codes4[i];
                const float sh = block_scale(a.fmt, a.c2, a.c1, mean, i >> 3, a.bshift);  // 8 items per 64 weights
                uint4 o;
                o.x = pack_bf16x2(lut[c & 15] * sh, lut[(c >> 4) & 15] * sh);
                o.y = pack_bf16x2(lut[(c >> 8) & 15] * sh, lut[(c >> 12) & 15] * sh);
                o.z = pack_bf16x2(lut[(c >> 16) & 15] * sh, lut[(c >> 20) & 15] * sh);
                o.w = pack_bf16x2(lut[(c >> 24) & 15] * sh, lut[c >> 28] * sh);
                out[i] = o;
            }
        }
        return;
    }
    b -= a.g_t;
    const bool second = b >= a.g_r0;
    cols_reduce(a.red[second ? 1 : 0], (b - (second ? a.g_r0 : 0)) * 256 + threadIdx.x);
}

// core_only: launch the GEMM kernel alone on a workspace that a full launch
// with the same arguments prepared (block scales, adapter operands, bf16 copy)
hipError_t launch(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, const float *V,
                  const uint16_t *ext_w, int r, float s, uint16_t *out, const GemmWs &ws,
                  const ColsReduceJob *red, hipStream_t st, bool core_only = false) {
    GemmArgs p;
    p.a = a;
    p.M = M;
    p.N = dx ? w.k : w.d;
    p.Kd = dx ? w.d : w.k;
    p.codes = w.codes;
    p.shat = ws.shat;
    p.d = w.d;
    p.k = w.k;
    p.ext_a = ws.ext_a;
    p.ext_b = ws.ext_b;
    p.Ke = gemm_ext_cols(r);
    p.wbf = ws.wbf;
    p.ldw = dx ? (w.d + 63) / 64 * 64 : w.k;
    p.out = out;
    // 32-bit buffer offsets: a 512-row slab of the activation operand and the
    // whole adapter operand must stay below 2 GiB
    if ((int64_t)BM * p.Kd * 2 >= (int64_t(1) << 31) || p.N * p.Ke * 2 >= (int64_t(1) << 31) ||
        (int64_t)BM * p.Ke * 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;

    const int64_t tiles_m = (M + BM - 1) / BM, tiles = tiles_m * ((p.N + BN - 1) / BN);
    const bool expand = tiles_m == 1;
    if (!core_only) {
        PrepArgs q;
        q.fmt = w.fmt;
        q.bshift = w.bshift;
        q.c2 = w.c2;
        q.c1 = w.c1;
        q.mean = w.mean;
        q.nb = w.d * w.k / 64;
        q.shat = ws.shat;
        q.V = V;
        q.M = M;
        q.r = r;
        q.s = s;
        q.ext_a = ws.ext_a;
        q.W = ext_w;
        q.N = p.N;
        q.ext_b = ws.ext_b;
        q.Ke = p.Ke;
        q.codes = w.codes;
        q.d = w.d;
        q.k = w.k;
        q.ldw = p.ldw;
        q.wbf = ws.wbf;
        q.red[0] = red ? red[0] : ColsReduceJob{nullptr, 0, 1, 0, 0, 0.0f, nullptr};
        q.red[1] = red ? red[1] : ColsReduceJob{nullptr, 0, 1, 0, 0, 0.0f, nullptr};
        q.g_shat = expand ? (q.nb + 255) / 256 : 0;  // only the expanding GEMM reads the scales
        q.g_a = (M * (p.Ke / 8) + 255) / 256;
        q.g_b = (p.N * (p.Ke / 8) + 255) / 256;
        // the bf16 copy of What (forward: a stride loop over 8-weight items) or What^T (dX: 64 x 256 tiles)
        q.g_t = expand ? 0 : ((w.k + 255) / 256) * ((w.d + 63) / 64);
        q.g_r0 = (q.red[0].N * q.red[0].R + 255) / 256;
        const int64_t g_r1 = (q.red[1].N * q.red[1].R + 255) / 256;
        const dim3 pgrid((unsigned)(q.g_shat + q.g_a + q.g_b + q.g_t + q.g_r0 + g_r1));
        if (dx) hipLaunchKernelGGL(prep_kernel<true>, pgrid, dim3(256), 0, st, q, nf4_consts());
        else hipLaunchKernelGGL(prep_kernel<false>, pgrid, dim3(256), 0, st, q, nf4_consts());
    }
    const dim3 grid((unsigned)tiles), block(NTHREADS);
    if (expand) {
        if (dx) hipLaunchKernelGGL((nf4_gemm_kernel<true, true>), grid, block, 0, st, p, nf4_consts());
        else hipLaunchKernelGGL((nf4_gemm_kernel<false, true>), grid, block, 0, st, p, nf4_consts());
    } else {
        if (dx) hipLaunchKernelGGL((nf4_gemm_kernel<true, false>), grid, block, 0, st, p, nf4_consts());
        else hipLaunchKernelGGL((nf4_gemm_kernel<false, false>), grid, block, 0, st, p, nf4_consts());
    }
    return hipGetLastError();
}

}  // namespace

int64_t gemm_ext_cols(int r) { return (2 * (int64_t)r + BK - 1) / BK * BK; }

int64_t gemm_wbf_elems(int64_t M, int64_t d, int64_t k) {
    return (M + BM - 1) / BM > 1 ? k * ((d + 63) / 64 * 64) : 0;
}

hipError_t launch_gemm_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const float *U,
                           const uint16_t *B, int r, float s, uint16_t *Y, const GemmWs &ws,
                           hipStream_t st) {
    return launch(false, w, x, M, U, B, r, s, Y, ws, nullptr, st);
}

hipError_t launch_gemm_dx(const Nf4Weights &w, const uint16_t *dy, int64_t M, const float *G,
                          const uint16_t *A, int r, float s, uint16_t *dX, const GemmWs &ws,
                          const ColsReduceJob *red, hipStream_t st) {
    return launch(true, w, dy, M, G, A, r, s, dX, ws, red, st);
}

hipError_t launch_cols_reduce(const ColsReduceJob *red, hipStream_t st) {
    PrepArgs q{};
    q.red[0] = red[0];
    q.red[1] = red[1];
    q.g_r0 = (q.red[0].N * q.red[0].R + 255) / 256;
    const int64_t g_r1 = (q.red[1].N * q.red[1].R + 255) / 256;
    if (q.g_r0 + g_r1 == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel<false>, dim3((unsigned)(q.g_r0 + g_r1)), dim3(256), 0, st, q, nf4_consts());
    return hipGetLastError();
}

hipError_t launch_gemm_core(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, int r, uint16_t *out,
                            const GemmWs &ws, hipStream_t st) {
    return launch(dx, w, a, M, nullptr, nullptr, r, 0.0f, out, ws, nullptr, st, true);
}

}  // namespace qnf4
