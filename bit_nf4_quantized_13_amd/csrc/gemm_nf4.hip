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
// Design (MI355X, one 512-thread workgroup -- 8 waves, two per SIMD -- per
// output tile; k-steps of 64):
//  * Tiles: 512 x 128 when the weight tile is expanded in the kernel (M <=
//    512, one tile row), else 256 x 256, or 256 x 128 where 256 x 256 tiles
//    would leave CUs idle.  A wave owns 64 output rows and all 128 columns
//    (512 x 128) or one column half (256-row tiles): 4 x 8 (4 x 4) MFMA
//    16x16x32 tiles, fp32 accumulators in AGPRs.
//  * Both operand tiles live in LDS in two stages (activation [TM][64] and
//    weight [TN][64] bf16, up to 160 KiB): while step kt runs its MFMAs on one
//    stage, the tiles of step kt + 1 move into the other, one barrier per
//    step.  The activation tile (X or dY) goes global -> LDS by buffer_load
//    ... lds transfers (16 bytes a lane), XOR-swizzled by 16-byte chunks so
//    that the fragment reads are free of bank conflicts; each wave moves an
//    eighth of the rows.  The transfers of a step are spread over its MFMA
//    groups.
//  * The weight operand takes one of two forms.  With a single 512-row tile
//    of M (M <= 512) the kernel expands it from the packed codes (EXPAND):
//    codes and block scales arrive in registers three steps ahead, the 16
//    levels live in a VGPR (lane j holds C[j % 16]) and are looked up with
//    ds_bpermute, then one multiply by the scale and one RNE to bf16 --
//    bit-identical to qlora_nf4_dequantize -- and the LDS write, spread over
//    MFMA groups.  Forward: a thread expands 16 consecutive weights of one W0
//    row; dX (the reduction runs over W0 rows): 2 rows x 8 columns, written
//    k-contiguous (the transpose happens in registers).  With more row tiles
//    the preparation kernel writes What (or What^T) in bf16 once per call and
//    the weight tile moves by the same transfers as the activations:
//    expanding each weight tile once per row tile costs more than the MFMA
//    shadow holds (measured: 22 % slower forward, 35 % slower dX at M = 4096).
//  * The MFMA takes the weight fragment as its first operand, so each lane
//    ends with 4 consecutive output columns of one row (8-byte stores).
//  * The adapter term is appended as extra k-steps whose operands the
//    preparation kernel lays out in memory: [hi(sV) | lo(sV) | 0] and
//    [W' | W' | 0] (hi = bf16(v), lo = bf16(v - hi), rows padded to a
//    multiple of 64).
//  * Workgroups are renumbered so each XCD walks a contiguous run of tiles.
//  * Split K: a grid of at most 128 tiles (most CUs idle) runs each tile's
//    k-steps in up to 8 slices, slice-major; each slice writes its fp32 sums
//    as a plane of its own (the adapter's k-steps go to the last slice) and
//    ksplit_reduce_kernel adds the planes in slice order and rounds once.
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
// The bf16 output pieces are stored with device scope (sc1: written through
// the XCD's L2), so the launch ends without a writeback of dirty output lines:
// 1.2-1.4 us less per 4096^3 launch than write-back stores, same bits.
constexpr int kOutPolicy = 16;
constexpr int NTHREADS = 512;                 // 8 waves, two per SIMD
constexpr int WM = BM / (NTHREADS / 64);      // rows per wave (64)
constexpr int MI = WM / 16;                   // 16-row MFMA tiles per wave (4)

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
    float *out_f32;         // F32OUT kernels: the fp32 sums [S][M x N] instead of out (split K: one plane per
                            // slice, added by ksplit_reduce_kernel)
    int64_t ks_len;         // k-steps per slice of K (split K; else nK)
    int S;                  // slices of K
    unsigned long long *span;  // null, or a measurement span (span_start / span_end)
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
// F32OUT: the fp32 sums are stored unrounded (out_f32) for a caller that adds
// another term before the one bf16 rounding.
// TM x TN: output rows x columns per tile, the 8 waves in TM / 64 rows of
// 64-row blocks by 512 / TM columns:
//   TM x 128   (TM = 64, 128, 256, 512) the expanding kernel, which has a single
//              tile row (each weight tile expanded once): TM the smallest that
//              holds M, so few tokens do not run empty rows through the MFMAs;
//   256 x 256  waves 4 x 2 of 64 x 128 (non-expanding): the same MFMA and
//              fragment-read work per wave as 512 x 128 with a fifth fewer tile
//              bytes moved into LDS per k-step (32 + 32 KiB against 64 + 16 KiB);
//   256 x 128  waves 4 x 2 of 64 x 64 (non-expanding): half the work per
//              workgroup, for grids whose 256 x 256 tiles would leave CUs idle.
// Below 512 rows (SQ) several waves read each activation row.
template <bool DX, bool EXPAND, bool F32OUT = false, int TN = BN, int TM = BM>
__global__ __launch_bounds__(NTHREADS) void nf4_gemm_kernel(GemmArgs p, Nf4Consts tab) {
    static_assert((EXPAND && TN == 128 && (TM == 64 || TM == 128 || TM == 256 || TM == 512)) ||
                      (!EXPAND && TM == 256 && (TN == 256 || TN == 128)),
                  "tile shapes: TM x 128 (expanding), 256 x 256 and 256 x 128");
    constexpr bool SQ = TM < 512;
    constexpr int WGM = TM / 64;           // waves along the rows
    constexpr int WNC = TN / (8 / WGM);    // output columns per wave
    constexpr int NJ = WNC / 16;         // 16-column MFMA tiles per wave
    constexpr int WR = TN / 8;           // weight-tile rows each wave moves
    constexpr int AR = TM / 8;           // activation-tile rows each wave moves
    constexpr int B_STAGE = TN * BK * 2; // weight tile bytes
    constexpr int A_ST = TM * BK * 2;    // activation tile bytes
    // Two stages of the activation tile [TM rows][64 k] and of the weight tile
    // [TN rows][64 k] (up to 160 KiB).  One object per buffer so that the compiler
    // can tell them apart when it places waits for the global->LDS transfers.
    __shared__ u32x4 sA0[A_ST / 16], sA1[A_ST / 16];
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
    const int wm = wave % WGM, wn = wave / WGM;  // the wave's 64-row, WNC-column block
    const int r16 = lane & 15, g = lane >> 4;
    if (tid == 0) span_start(p.span);
    const int64_t tiles_n = (p.N + TN - 1) / TN, tiles_m = (p.M + TM - 1) / TM;
    // split K: workgroup b takes slice b / tiles of the k-steps for tile b % tiles
    // (slice-major, so that each slice's tiles keep the XCD-aware order)
    // (32-bit scalars: a grid below 2^31 workgroups, nK below 2^15; wider or
    // divergent-looking bounds cost the k-loop registers)
    const uint32_t tiles = (uint32_t)(tiles_m * tiles_n);
    const int slice = (int)((uint32_t)blockIdx.x / tiles);
    int64_t mt, nt;
    tile_of(blockIdx.x - slice * tiles, tiles_m, tiles_n, mt, nt);
    const int64_t m_base = mt * TM, n_base = nt * TN;
    const int nK = (int)((p.Kd + BK - 1) / BK);
    const int k_lo = __builtin_amdgcn_readfirstlane(slice * (int)p.ks_len);  // this workgroup's k-steps
    const int k_hi = __builtin_amdgcn_readfirstlane(k_lo + (int)p.ks_len < nK ? k_lo + (int)p.ks_len : nK);  // never empty
    const int64_t kb = p.k / 64;  // NF4 blocks per W0 row

    // NF4 level table: lane j holds C[j % 16]
    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);

    // ---- activation tile: global -> LDS transfers of 8 rows x 128 B ---------------
    // Wave w moves rows AR w .. AR w + AR - 1 (transfer b: rows AR w + 8 b ..): with
    // 512-row tiles exactly the rows it reads, with fewer rows (SQ) a share of rows
    // that several waves read.  Lane l lands in row AR w + 8 b + l / 8, physical
    // chunk l % 8, which holds logical chunk (l % 8) ^ ((row >> 1) & 7) =
    // (l % 8) ^ ((l / 16 + 4 (AR w / 8 + b)) & 7): voff_a0 or voff_a1 by the
    // parity of AR w / 8 + b.
    // Rows past M read as zero.  Pieces past Kd (dX with d % 64 != 0) read the
    // next row's data: finite values that meet weight rows that are exactly zero.
    const int64_t rows_here = (p.M - m_base) < TM ? (p.M - m_base) : TM;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + m_base * p.Kd, rows_here * p.Kd * 2);
    const int dma_row = AR * wave + (lane >> 3);  // + 8 b
    const uint32_t voff_a0 = (uint32_t)(((int64_t)dma_row * p.Kd + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
    const uint32_t voff_a1 = (uint32_t)(((int64_t)dma_row * p.Kd + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
    const uint32_t row8_bytes = (uint32_t)(8 * p.Kd * 2);
    const int apar = (AR / 8) * wave;  // 8-row groups before this wave's first: the parity of the swizzle term
    auto issue_a = [&](int64_t kt, auto S, int b) __attribute__((always_inline)) {
        dma16(ra, Aof(S) + (AR * wave + 8 * b) * 8, ((apar + b) & 1) ? voff_a1 : voff_a0,
              (uint32_t)b * row8_bytes + (uint32_t)kt * (BK * 2));
    };
    // fragment reads (A: row WM wm + 16 i + r16; B: row WNC wn + 16 j + r16; chunk
    // 4 s + g), physical chunk (4 s + g) ^ ((r16 >> 1) & 7) in both tiles
    const int frag0 = r16 * 8 + ((0 + g) ^ ((r16 >> 1) & 7));  // in 16-byte units
    const int frag1 = r16 * 8 + ((4 + g) ^ ((r16 >> 1) & 7));
    const int arow = WM * wm * 8;
    const int brow = WNC * wn * 8;
    auto read_a = [&](auto S, int s, int i) __attribute__((always_inline)) -> uint4 {
        return __builtin_bit_cast(uint4, Aof(S)[arow + (s ? frag1 : frag0) + 128 * i]);
    };

    // ---- weight tiles [TN n][64 k], same chunk layout -------------------------------
    auto read_b = [&](auto S, int s, int j) __attribute__((always_inline)) -> uint4 {
        return __builtin_bit_cast(uint4, Bof(S)[brow + (s ? frag1 : frag0) + 128 * j]);
    };
    // transfer (non-expanding kernel): rows n_base .., 8 per transfer, wave w moves
    // rows WR w .. WR w + WR - 1; rows past N read as zero.  Transfer u lands in rows
    // whose swizzle term is (4 (WR w / 8 + u) + l / 16) & 7: voff_w0 or voff_w1 by
    // the parity of WR w / 8 + u.
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(p.wbf + n_base * p.ldw, EXPAND ? 0 : ((p.N - n_base) < TN ? (p.N - n_base) : TN) * p.ldw * 2);
    const int wrow = WR * wave + (lane >> 3);  // + 8 u
    const int wpar = (WR / 8) * wave;
    const uint32_t voff_w0 = (uint32_t)(((int64_t)wrow * p.ldw + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
    const uint32_t voff_w1 = (uint32_t)(((int64_t)wrow * p.ldw + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
    const uint32_t wrow8_bytes = (uint32_t)(8 * p.ldw * 2);
    auto issue_w = [&](int64_t kt, auto S, int u) __attribute__((always_inline)) {
        dma16(rw, Bof(S) + (WR * wave + 8 * u) * 8, ((wpar + u) & 1) ? voff_w1 : voff_w0,
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
    f32x4 acc[MI][NJ];
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
        const int64_t kn = kt + 1 < k_hi ? kt + 1 : k_hi - 1;
        const int64_t kw = kt + 3 < k_hi ? kt + 3 : k_hi - 1;
#pragma unroll
        for (int grp = 0; grp < 2 * NJ; ++grp) {
            const int s = grp / NJ, j = grp % NJ;
            if (grp + 2 < 2 * NJ) bq[(grp + 2) & 3] = read_b(S{}, (grp + 2) / NJ, (grp + 2) % NJ);
            if (grp == 0) {
#pragma unroll
                for (int i = 0; i < MI; ++i) af[1][i] = read_a(S{}, 1, i);
            }
            if constexpr (EXPAND) {
                // the AR / 8 transfers first, then the weight-data loads (the
                // end-of-step wait counts on their being last); the three phases
                // of piece s spread over the slice's groups in order
                constexpr int nA = AR / 8;
                constexpr int gW = nA < 2 * NJ - 1 ? nA : 2 * NJ - 1;
                constexpr int j0 = NJ == 8 ? 1 : NJ == 4 ? 1 : 0;
                constexpr int j1 = NJ == 8 ? 4 : NJ == 4 ? 2 : NJ - 1;
                constexpr int j2 = NJ == 8 ? 6 : NJ == 4 ? 3 : NJ - 1;
                if (grp < nA) issue_a(kn, S1{}, grp);
                if (grp == gW) load_w(kw, wl);
                if (j == j0) expand_phase(wc, s, 0, st_w);
                if (j == j1) expand_phase(wc, s, 1, st_w);
                if (j == j2) expand_phase(wc, s, 2, st_w);
            } else if constexpr (TN == 256) {  // 16 groups: 4 + 4 transfers, alternating
                if (grp < 8) {
                    if (grp & 1) issue_a(kn, S1{}, grp >> 1);
                    else issue_w(kn, S1{}, grp >> 1);
                }
            } else {  // 256 x 128, 8 groups: 2 + 4 transfers
                if (grp < 2) issue_w(kn, S1{}, grp);
                else if (grp < 6) issue_a(kn, S1{}, grp - 2);
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
        if constexpr (!SQ) {  // rows this wave moved itself
#pragma unroll
            for (int i = 0; i < MI; ++i) af[0][i] = read_a(S1{}, 0, i);
        }
        __builtin_amdgcn_s_barrier();
        if constexpr (SQ) {  // rows other waves moved too
#pragma unroll
            for (int i = 0; i < MI; ++i) af[0][i] = read_a(S1{}, 0, i);
        }
        bq[0] = read_b(S1{}, 0, 0);
        bq[1] = read_b(S1{}, 1 / NJ, 1 % NJ);
        sched_fence();
    };

    // ---- prologue: A(k_lo) and weight tile k_lo in LDS; weight data of the next two steps loaded ----
    if constexpr (EXPAND) {
        load_w(k_lo, w0);
#pragma unroll
        for (int b = 0; b < AR / 8; ++b) issue_a(k_lo, IC<0>{}, b);
        load_w(k_lo + 1 < k_hi ? k_lo + 1 : k_lo, w1);
        load_w(k_lo + 2 < k_hi ? k_lo + 2 : k_hi - 1, w2);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ph = 0; ph < 3; ++ph) expand_phase(w0, c, ph, sB0);
    } else {
#pragma unroll
        for (int u = 0; u < WR / 8; ++u) issue_w(k_lo, IC<0>{}, u);
#pragma unroll
        for (int b = 0; b < AR / 8; ++b) issue_a(k_lo, IC<0>{}, b);
    }
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (!SQ) {
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = read_a(IC<0>{}, 0, i);
    }
    __syncthreads();
    if constexpr (SQ) {
#pragma unroll
        for (int i = 0; i < MI; ++i) af[0][i] = read_a(IC<0>{}, 0, i);
    }
    bq[0] = read_b(IC<0>{}, 0, 0);
    bq[1] = read_b(IC<0>{}, 1 / NJ, 1 % NJ);

    // ---- main k-loop: step k_lo peeled, then six steps per trip ----------------------
    step(k_lo, IC<0>{}, IC<1>{});
    int64_t kt = k_lo + 1;
    for (; kt + 6 <= k_hi; kt += 6) {
        step(kt + 0, IC<1>{}, IC<0>{});
        step(kt + 1, IC<2>{}, IC<0>{});
        step(kt + 2, IC<3>{}, IC<0>{});
        step(kt + 3, IC<4>{}, IC<0>{});
        step(kt + 4, IC<5>{}, IC<0>{});
        step(kt + 5, IC<0>{}, IC<0>{});
    }
    if (kt < k_hi) step(kt, IC<1>{}, IC<0>{});
    if (kt + 1 < k_hi) step(kt + 1, IC<2>{}, IC<0>{});
    if (kt + 2 < k_hi) step(kt + 2, IC<3>{}, IC<0>{});
    if (kt + 3 < k_hi) step(kt + 3, IC<4>{}, IC<0>{});
    if (kt + 4 < k_hi) step(kt + 4, IC<5>{}, IC<0>{});

    // ---- adapter term: Ke/64 extra k-steps, operands laid out in memory (last slice) ----
    if (slice == p.S - 1) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rea = make_rsrc(p.ext_a + m_base * p.Ke, rows_here * p.Ke * 2);
        const uint32_t voff_e0 = (uint32_t)(((int64_t)dma_row * p.Ke + 8 * ((lane & 7) ^ ((lane >> 4) & 7))) * 2);
        const uint32_t voff_e1 = (uint32_t)(((int64_t)dma_row * p.Ke + 8 * ((lane & 7) ^ (((lane >> 4) + 4) & 7))) * 2);
        const uint32_t row8_e = (uint32_t)(8 * p.Ke * 2);
        // weight-side operand rows n_base .. + TN - 1 (clamped to N-1): transfer u of
        // wave w covers rows WR w + 8 u .. + 7
        const __amdgpu_buffer_rsrc_t reb = make_rsrc(p.ext_b, p.N * p.Ke * 2);
        uint32_t voff_eb[WR / 8];
#pragma unroll
        for (int u = 0; u < WR / 8; ++u) {
            const int row = WR * wave + 8 * u + (lane >> 3);
            int64_t n = n_base + row;
            n = n < p.N ? n : p.N - 1;
            voff_eb[u] = (uint32_t)((n * p.Ke + 8 * ((lane & 7) ^ ((row >> 1) & 7))) * 2);
        }
        const int64_t nE = p.Ke / BK;
        for (int64_t e = 0; e < nE; ++e) {
#pragma unroll
            for (int b = 0; b < AR / 8; ++b)
                dma16(rea, sA0 + (AR * wave + 8 * b) * 8, ((apar + b) & 1) ? voff_e1 : voff_e0,
                      (uint32_t)b * row8_e + (uint32_t)e * (BK * 2));
#pragma unroll
            for (int u = 0; u < WR / 8; ++u) dma16(reb, sB0 + (WR * wave + 8 * u) * 8, voff_eb[u], (uint32_t)e * (BK * 2));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int i = 0; i < MI; ++i) af[0][i] = read_a(IC<0>{}, s, i);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const uint4 b = read_b(IC<0>{}, s, j);
#pragma unroll
                    for (int i = 0; i < MI; ++i) mfma16_acc(b, af[0][i], acc[i][j]);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }
    // the epilogue reads the accumulators with VALU instructions: let the
    // last MFMAs (inline asm, invisible to the hazard recognizer) drain
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

    // ---- epilogue: lane holds D[m = 16 i + r16][n = 16 j + 4 g .. + 3] ----------------
    // (bf16 output in 16-byte pieces, 64 contiguous bytes per row and tile pair:
    // with 8-byte pieces the stores took 3.5 us more of a 109 us launch)
    const __amdgpu_buffer_rsrc_t rout_y = make_rsrc(p.out, F32OUT ? 0 : p.M * p.N * 2);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int64_t m = m_base + WM * wm + 16 * i + r16;
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t n = n_base + WNC * wn + 16 * j + 4 * g;
            if ((F32OUT || NJ == 1) && n >= p.N) continue;
            if constexpr (F32OUT) {
                *reinterpret_cast<f32x4 *>(p.out_f32 + ((int64_t)slice * p.M + m) * p.N + n) = acc[i][j];
            } else if constexpr (NJ >= 2) {
                // tiles j, j + 1 (j even) leave as 16-byte pieces: lane g takes tile
                // j + g / 2, columns 8 (g % 2) .. + 7, gathered from lanes 2 (g % 2)
                // and 2 (g % 2) + 1 of the same row (four lanes write 64 contiguous bytes)
                if (j & 1) continue;
                const uint32_t p0x = pack_bf16x2(acc[i][j][0], acc[i][j][1]), p0y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                const uint32_t p1x = pack_bf16x2(acc[i][j + 1][0], acc[i][j + 1][1]),
                               p1y = pack_bf16x2(acc[i][j + 1][2], acc[i][j + 1][3]);
                const int srcA = (r16 + 16 * (2 * (g & 1))) * 4, srcB = (r16 + 16 * (2 * (g & 1) + 1)) * 4;
                const bool t1 = g >= 2;
                auto pull = [&](int src, uint32_t v0, uint32_t v1) __attribute__((always_inline)) -> uint32_t {
                    const uint32_t a0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v0);
                    const uint32_t a1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v1);
                    return t1 ? a1 : a0;
                };
                const uint4 o{pull(srcA, p0x, p1x), pull(srcA, p0y, p1y), pull(srcB, p0x, p1x), pull(srcB, p0y, p1y)};
                const int64_t n8 = n_base + WNC * wn + 16 * (j + (g >> 1)) + 8 * (g & 1);
                if (n8 < p.N)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rout_y,
                                                           (uint32_t)((m * p.N + n8) * 2), 0, kOutPolicy);
            } else {
                const uint2 o{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                *reinterpret_cast<uint2 *>(p.out + m * p.N + n) = o;
            }
        }
    }
    if (p.span) {  // measurement only: this workgroup's stores are out
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) span_end(p.span);
    }
}

// Transposed dequantized weight operand for the non-expanding dX GEMM: What^T
// [k x ldw] with zero columns d .. ldw-1, bf16, bit-identical to
// qlora_nf4_dequantize (the block scale is doubleDequant's, computed here from
// c2, c1 and the mean).  One workgroup per 64 W0 rows x 1024 columns; thread t
// expands an 8 x 32 block: rows 8 (t % 8) .., columns 32 (t / 8) .. (half of
// one NF4 block, so one scale per row).  Each code load is a 16-byte piece, so
// the 8 lanes of a row read 128 contiguous bytes; the block is transposed in
// registers (v_perm) and stored as 16-byte column pieces, so no LDS is
// involved and every store is a contiguous 128-byte row segment per 8 lanes.
// (The forward's What, laid out like the codes, is written by its own job in
// prep_kernel.)  Against 8 x 8 blocks (4-byte code pieces, 32-byte row
// segments per load, a scale lookup per 8 weights): 13.1 against 15.5 us for
// the dX preparation at 4096 x 4096, same bits; narrower blocks (8 x 4) and
// two tiles per workgroup with the next one's loads overlapping were slower.
// The dequantized weight copy is stored with device scope (sc1: written
// through the XCD's L2 into the memory-side cache the GEMM reads it from), so
// the end of the preparation launch has no dirty L2 lines of it to write back:
// 0.6-0.8 us less per launch at 4096 x 4096, the GEMM's reads unchanged.
constexpr int kCopyPolicy = 16;  // cache-policy bits of the copy's stores: sc1
__device__ __forceinline__ void dequant_tile_t(int64_t bid, const uint8_t *__restrict__ codes, int fmt, int bshift,
                                               const int8_t *__restrict__ c2, const float *__restrict__ c1,
                                               float mean, int64_t d, int64_t k, int64_t ldw, const Nf4Consts &tab,
                                               uint16_t *__restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t ct = (k + 1023) / 1024;
    const int64_t tk = bid % ct, td = bid / ct;
    const int ng = tid & 7, kg = tid >> 3;
    const int64_t n0 = td * 64 + 8 * ng;    // first of this thread's 8 W0 rows
    const int64_t k0 = tk * 1024 + 32 * kg;  // first of its 32 columns
    if (k0 >= k) return;                     // k % 64 == 0: whole 32-column groups
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, k * ldw * 2);
    float lvf = tab.level[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
    const int lv = __float_as_int(lvf);
    const int64_t kb = k / 64;
    uint4 cw[8];
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t n = n0 + e;
        cw[e] = n < d ? *reinterpret_cast<const uint4 *>(codes + n * (k / 2) + k0 / 2) : uint4{0, 0, 0, 0};
        sc[e] = n < d ? block_scale(fmt, c2, c1, mean, n * kb + k0 / 64, bshift) : 0.0f;
    }
    // v[e][q]: row e, columns 2 q, 2 q + 1 (bf16 pair)
    uint32_t v[8][16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t wv[4] = {cw[e].x, cw[e].y, cw[e].z, cw[e].w};
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint32_t x = pack_bf16x2(level(code_addr(wv[q >> 2], 2 * (q & 3)), lv) * sc[e],
                                           level(code_addr(wv[q >> 2], 2 * (q & 3) + 1), lv) * sc[e]);
            v[e][q] = n0 + e < d ? x : 0u;  // rows past d: zero columns of What^T
        }
    }
    // column c of the block: rows 0..7 packed as 4 bf16 pairs
    // (rows 2 e2, 2 e2 + 1) = low halves (c even) or high halves (c odd)
    // of v[2 e2][c / 2] and v[2 e2 + 1][c / 2]
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
            o[e2] = (c & 1) ? __builtin_amdgcn_perm(v[2 * e2 + 1][c >> 1], v[2 * e2][c >> 1], 0x07060302u)
                            : __builtin_amdgcn_perm(v[2 * e2 + 1][c >> 1], v[2 * e2][c >> 1], 0x05040100u);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, uint4{o[0], o[1], o[2], o[3]}), rout,
                                               (uint32_t)(((k0 + c) * ldw + n0) * 2), 0, kCopyPolicy);
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
    const float *Vpart;  // or V's S partial sums [S][r][M], added here in slice order
    int Vs;
    float *Vout;         // with Vpart: V [M x r] stored
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

constexpr int kWU = 2;  // 8-weight units per thread of the forward What copy

template <bool DX>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a, Nf4Consts tab) {
    int64_t b = blockIdx.x;
    if (b < a.g_shat) {
        const int64_t x = b * 256 + threadIdx.x;
        if (x < a.nb) a.shat[x] = block_scale(a.fmt, a.c2, a.c1, a.fmt != kNoDq ? *a.mean : 0.0f, x, a.bshift);
        return;
    }
    b -= a.g_shat;
    if (b < a.g_a && a.Vpart) {
        // ext_a from the partial sums of V: thread (c, row), rows fastest so that the
        // partial reads are contiguous.  c < r: V[row][c] = the S partials added in slice
        // order from +0 (rows_reduce_kernel's additions; all S loads issued first), stored,
        // and its hi / lo columns c and r + c of ext_a; r <= c < Ke - r: the zero column r + c
        const int64_t x = b * 256 + threadIdx.x;
        const int64_t row = x % a.M, c = x / a.M;
        if (c >= a.Ke - a.r) return;
        uint16_t *const dst = a.ext_a + row * a.Ke;
        if (c >= a.r) {
            dst[a.r + c] = 0;
            return;
        }
        constexpr int kMaxParts = 16;
        float pv[kMaxParts];
#pragma unroll
        for (int sl = 0; sl < kMaxParts; ++sl)
            pv[sl] = sl < a.Vs ? a.Vpart[((int64_t)sl * a.r + c) * a.M + row] : 0.0f;
        float sum = 0.0f;
#pragma unroll
        for (int sl = 0; sl < kMaxParts; ++sl)
            if (sl < a.Vs) sum += pv[sl];
        a.Vout[row * a.r + c] = sum;
        const float f = a.s * sum;
        const uint32_t hb = pack_bf16x2(f, 0.0f) & 0xFFFFu;
        dst[c] = (uint16_t)hb;
        dst[a.r + c] = (uint16_t)(pack_bf16x2(f - bf16_bits_to_f32(hb), 0.0f) & 0xFFFFu);
        return;
    }
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
            // What [d x k], row-major like the codes.  Wave w of workgroup b
            // writes the 512 kWU weights from 512 kWU (4 b + w): unit u of lane
            // l is the 8 weights at 512 u + 8 l (one code dword in, one 16-byte
            // piece out), so every load and store instruction of a wave covers
            // one contiguous span; all loads are issued before the first store,
            // and the workgroups run in several rounds, whose reads and writes
            // overlap.
            const int lane = threadIdx.x & 63;
            float lvf = tab.level[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) lvf = (lane & 15) == j ? tab.level[j] : lvf;
            const int lv = __float_as_int(lvf);
            const int64_t total = a.d * a.k;  // a multiple of 64
            const int64_t e0 = (b * 4 + (threadIdx.x >> 6)) * (512 * kWU) + 8 * lane;
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, total / 2);  // past the end: zero
            const __amdgpu_buffer_rsrc_t rw_out = make_rsrc(a.wbf, total * 2);
            uint32_t cw[kWU];
            float sc[kWU];
#pragma unroll
            for (int u = 0; u < kWU; ++u) {
                const int64_t e = e0 + 512 * u;
                cw[u] = load4(rc, (uint32_t)(e / 2), 0);
                const int64_t ec = e < total ? e : total - 64;  // a valid block for units past the end
                sc[u] = block_scale(a.fmt, a.c2, a.c1, mean, ec >> 6, a.bshift);
            }
            uint4 o[kWU];
#pragma unroll
            for (int u = 0; u < kWU; ++u) {
                uint32_t pr[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pr[q] = pack_bf16x2(level(code_addr(cw[u], 2 * q), lv) * sc[u],
                                        level(code_addr(cw[u], 2 * q + 1), lv) * sc[u]);
                o[u] = uint4{pr[0], pr[1], pr[2], pr[3]};
            }
#pragma unroll
            for (int u = 0; u < kWU; ++u) {
                const int64_t e = e0 + 512 * u;
                if (e < total)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[u]), rw_out, (uint32_t)(e * 2), 0,
                                                           kCopyPolicy);
            }
        }
        return;
    }
    b -= a.g_t;
    const bool second = b >= a.g_r0;
    cols_reduce(a.red[second ? 1 : 0], (b - (second ? a.g_r0 : 0)) * 256 + threadIdx.x);
}

// Tile shape of the non-expanding GEMM: 256 x 256, or the narrow 256 x 128
// (half the work per workgroup at a higher LDS cost per flop: the activation
// tile is moved and read for half the columns), measured at 0.66 of the wide
// tile's time (143 against 109 us for two rounds of narrow against one of wide
// tiles, M = d = k = 4096), so kNarrowCost = 0.7.  Rounds of 256 workgroups
// (one per CU) decide: narrow wins where the wide grid leaves CUs idle (M =
// 2048 against 4096 columns: 128 wide tiles).
constexpr double kNarrowCost = 0.7;
struct TileShape {
    int tm, tn;
};
int64_t tile_count(TileShape t, int64_t M, int64_t N) { return ((M + t.tm - 1) / t.tm) * ((N + t.tn - 1) / t.tn); }
TileShape pick_tile(int64_t M, int64_t N) {
    const TileShape wide{256, 256}, narrow{256, 128};
    const double rw = (double)((tile_count(wide, M, N) + 255) / 256);
    const double rn = (double)((tile_count(narrow, M, N) + 255) / 256) * kNarrowCost;
    return rn < rw ? narrow : wide;
}

// Slices of K for a grid of `tiles` output tiles over nK k-steps: with at most
// half a round of tiles (<= 128 workgroups for 256 CUs), enough slices to fill
// about one round, at most 8 and at least 4 k-steps (256 k) each; their fp32
// partial sums are added by ksplit_reduce_kernel.  One slice otherwise.
int ksplit_slices(int64_t tiles, int64_t nK) {
    if (tiles > 128) return 1;
    int64_t S = 256 / tiles;
    S = S < 8 ? S : 8;
    S = S < nK / 4 ? S : nK / 4;
    if (S < 2) return 1;
    const int64_t len = (nK + S - 1) / S;
    return (int)((nK + len - 1) / len);  // no empty slice
}

// out[e] = sum over s of part[s][e] in slice order, rounded once to bf16 (or
// stored in fp32 to out_f32); four consecutive elements per thread.
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(const float *__restrict__ part, int S, int64_t MN,
                                                            uint16_t *__restrict__ out, float *__restrict__ out_f32) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= MN) return;  // MN % 4 == 0
    f32x4 v = *reinterpret_cast<const f32x4 *>(part + e);
    for (int q = 1; q < S; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(part + (int64_t)q * MN + e);
        v = f32x4{v[0] + t[0], v[1] + t[1], v[2] + t[2], v[3] + t[3]};
    }
    if (out_f32) *reinterpret_cast<f32x4 *>(out_f32 + e) = v;
    else *reinterpret_cast<uint2 *>(out + e) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// Tiles and slices of K of one GEMM launch.
struct GemmGrid {
    TileShape ts;
    int64_t tiles;
    int S;
    int64_t ks_len;
};
GemmGrid gemm_grid(int64_t M, int64_t N, int64_t Kd, bool force_expand) {
    GemmGrid g;
    const bool expand = (M + BM - 1) / BM == 1 || force_expand;
    // the expanding kernel: the fewest 64-row blocks that hold M (one tile row)
    const int tm = force_expand || M > 256 ? BM : M > 128 ? 256 : M > 64 ? 128 : 64;
    g.ts = expand ? TileShape{tm, BN} : pick_tile(M, N);
    g.tiles = tile_count(g.ts, M, N);
    const int64_t nK = (Kd + BK - 1) / BK;
    g.S = ksplit_slices(g.tiles, nK);
    g.ks_len = (nK + g.S - 1) / g.S;
    return g;
}
size_t ksplit_bytes(const GemmGrid &g, int64_t M, int64_t N) {
    return g.S > 1 ? sizeof(float) * (size_t)g.S * (size_t)M * (size_t)N : 0;
}

// What a launch runs: the preparation and the GEMM (kFull); the GEMM kernel alone
// on a workspace that a full launch with the same arguments prepared (kCoreOnly);
// or, for measurement, the block scales and the expanding GEMM kernel whatever
// the number of row tiles, reusing the adapter operands a full launch prepared
// (kExpandCore).
enum LaunchWhat : int { kFull = 0, kCoreOnly = 1, kExpandCore = 2 };

// out_f32 (dX only): store the fp32 sums there instead of bf16 into out
hipError_t launch(bool dx, const Nf4Weights &w, const uint16_t *a, int64_t M, const float *V,
                  const uint16_t *ext_w, int r, float s, uint16_t *out, const GemmWs &ws,
                  const ColsReduceJob *red, hipStream_t st, int what = kFull, float *out_f32 = nullptr,
                  const float *Vpart = nullptr, int Vs = 0, float *Vout = nullptr) {
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
    p.out_f32 = out_f32;
    p.span = timing_take(dx ? kTimeDxGemm : kTimeFwdGemm);
    if (out_f32 && !dx) return hipErrorInvalidValue;
    // 32-bit buffer offsets: a 512-row slab of the activation operand and the
    // whole adapter operand must stay below 2 GiB
    if ((int64_t)BM * p.Kd * 2 >= (int64_t(1) << 31) || p.N * p.Ke * 2 >= (int64_t(1) << 31) ||
        (int64_t)BM * p.Ke * 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;

    const int64_t tiles_m = (M + BM - 1) / BM;
    const bool expand = tiles_m == 1 || what == kExpandCore;
    GemmGrid gg = gemm_grid(M, p.N, p.Kd, what == kExpandCore);
    if (ksplit_bytes(gg, M, p.N) > ws.kpart_bytes) {  // a workspace sized for the other kernel choice
        gg.S = 1;
        gg.ks_len = (p.Kd + BK - 1) / BK;
    }
    const TileShape ts = gg.ts;
    p.S = gg.S;
    p.ks_len = gg.ks_len;
    // split K: the fp32 kernels write one plane of partial sums per slice into the
    // workspace, which ksplit_reduce_kernel adds into out / out_f32
    const bool f32k = out_f32 || gg.S > 1;
    if (gg.S > 1) p.out_f32 = ws.kpart;
    if (what == kExpandCore) {
        PrepArgs q{};
        q.fmt = w.fmt;
        q.bshift = w.bshift;
        q.c2 = w.c2;
        q.c1 = w.c1;
        q.mean = w.mean;
        q.nb = w.d * w.k / 64;
        q.shat = ws.shat;
        q.red[0] = q.red[1] = ColsReduceJob{nullptr, 0, 1, 0, 0, 0.0f, nullptr};
        q.g_shat = (q.nb + 255) / 256;
        if (dx) hipLaunchKernelGGL(prep_kernel<true>, dim3((unsigned)q.g_shat), dim3(256), 0, st, q, nf4_consts());
        else hipLaunchKernelGGL(prep_kernel<false>, dim3((unsigned)q.g_shat), dim3(256), 0, st, q, nf4_consts());
    } else if (what == kFull) {
        PrepArgs q;
        q.fmt = w.fmt;
        q.bshift = w.bshift;
        q.c2 = w.c2;
        q.c1 = w.c1;
        q.mean = w.mean;
        q.nb = w.d * w.k / 64;
        q.shat = ws.shat;
        q.V = V;
        q.Vpart = Vpart;
        q.Vs = Vs;
        q.Vout = Vout;
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
        q.g_a = Vpart ? (M * (p.Ke - r) + 255) / 256 : (M * (p.Ke / 8) + 255) / 256;
        q.g_b = (p.N * (p.Ke / 8) + 255) / 256;
        // the bf16 copy of What (forward: 2048 kWU weights per workgroup) or What^T (dX: 64 x 1024 tiles)
        q.g_t = expand ? 0 : dx ? ((w.k + 1023) / 1024) * ((w.d + 63) / 64) : (w.d * w.k + 2048 * kWU - 1) / (2048 * kWU);
        q.g_r0 = (q.red[0].N * q.red[0].R + 255) / 256;
        const int64_t g_r1 = (q.red[1].N * q.red[1].R + 255) / 256;
        const dim3 pgrid((unsigned)(q.g_shat + q.g_a + q.g_b + q.g_t + q.g_r0 + g_r1));
        if (dx) hipLaunchKernelGGL(prep_kernel<true>, pgrid, dim3(256), 0, st, q, nf4_consts());
        else hipLaunchKernelGGL(prep_kernel<false>, pgrid, dim3(256), 0, st, q, nf4_consts());
    }
    const dim3 grid((unsigned)(gg.tiles * gg.S)), block(NTHREADS);
#define QNF4_GEMM(DXV, EXV, F32V, TNV, TMV) \
    hipLaunchKernelGGL((nf4_gemm_kernel<DXV, EXV, F32V, TNV, TMV>), grid, block, 0, st, p, nf4_consts())
#define QNF4_GEMM_SHAPES(DXV, F32V)                                 \
    do {                                                            \
        if (ts.tn == 256) QNF4_GEMM(DXV, false, F32V, 256, 256);    \
        else QNF4_GEMM(DXV, false, F32V, 128, 256);                 \
    } while (0)
#define QNF4_GEMM_EXPAND(DXV, F32V)                                  \
    do {                                                             \
        if (ts.tm == 64) QNF4_GEMM(DXV, true, F32V, 128, 64);        \
        else if (ts.tm == 128) QNF4_GEMM(DXV, true, F32V, 128, 128); \
        else if (ts.tm == 256) QNF4_GEMM(DXV, true, F32V, 128, 256); \
        else QNF4_GEMM(DXV, true, F32V, 128, 512);                   \
    } while (0)
    if (f32k) {
        if (expand) {
            if (dx) QNF4_GEMM_EXPAND(true, true);
            else QNF4_GEMM_EXPAND(false, true);
        } else {
            if (dx) QNF4_GEMM_SHAPES(true, true);
            else QNF4_GEMM_SHAPES(false, true);
        }
    } else if (expand) {
        if (dx) QNF4_GEMM_EXPAND(true, false);
        else QNF4_GEMM_EXPAND(false, false);
    } else if (dx) {
        QNF4_GEMM_SHAPES(true, false);
    } else {
        QNF4_GEMM_SHAPES(false, false);
    }
#undef QNF4_GEMM_EXPAND
#undef QNF4_GEMM_SHAPES
#undef QNF4_GEMM
    if (gg.S > 1) {
        const int64_t MN = M * p.N;
        hipLaunchKernelGGL(ksplit_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, st, ws.kpart, gg.S,
                           MN, out_f32 ? nullptr : out, out_f32);
    }
    return hipGetLastError();
}

}  // namespace

int64_t gemm_ext_cols(int r) { return (2 * (int64_t)r + BK - 1) / BK * BK; }

size_t gemm_ksplit_bytes(int64_t M, int64_t d, int64_t k) {
    const size_t fwd = ksplit_bytes(gemm_grid(M, d, k, false), M, d);
    const size_t dx = ksplit_bytes(gemm_grid(M, k, d, false), M, k);
    return fwd > dx ? fwd : dx;
}

int64_t gemm_wbf_elems(int64_t M, int64_t d, int64_t k) {
    return (M + BM - 1) / BM > 1 ? k * ((d + 63) / 64 * 64) : 0;
}

hipError_t launch_gemm_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const float *U,
                           const uint16_t *B, int r, float s, uint16_t *Y, const GemmWs &ws,
                           hipStream_t st, const float *Upart, int Us, float *Uout) {
    if (!U && (!Upart || Us < 1 || Us > 16 || !Uout)) return hipErrorInvalidValue;
    return launch(false, w, x, M, U, B, r, s, Y, ws, nullptr, st, kFull, nullptr, Upart, Us, Uout);
}

hipError_t launch_gemm_dx(const Nf4Weights &w, const uint16_t *dy, int64_t M, const float *G,
                          const uint16_t *A, int r, float s, uint16_t *dX, const GemmWs &ws,
                          const ColsReduceJob *red, hipStream_t st, float *dX_f32) {
    return launch(true, w, dy, M, G, A, r, s, dX, ws, red, st, kFull, dX_f32);
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
                            const GemmWs &ws, hipStream_t st, bool force_expand) {
    return launch(dx, w, a, M, nullptr, nullptr, r, 0.0f, out, ws, nullptr, st, force_expand ? kExpandCore : kCoreOnly);
}

}  // namespace qnf4
