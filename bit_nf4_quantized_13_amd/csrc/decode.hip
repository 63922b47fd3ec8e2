// Decode-shaped forward (M <= 16 tokens): Y = X What^T + s (X A^T) B^T in one
// kernel that streams the packed NF4 weights from HBM once.
//
// chkda.github.io "Why do we need LoRA and QLoRA?", "Double quantization and
// double dequantization": What = doubleDequant(c1, c2, W_NF4) in BF16 feeds the
// matrix multiplication.  With M <= 16 the product is bound by the bytes of the
// packed weights, so this kernel is organised around the cost of expanding a
// nibble, not around the matrix cores:
//
// * A 64-deep block of row n shares one scale s(n,b), so the product is taken
//   as sum_b s(n,b) * sum_{k in b} X[m][k] C[q(n,k)]: one MFMA pair per block
//   on the bf16 NF4 levels, then one fp32 FMA per result register.  The only
//   per-weight work left is the level lookup.  (This rounds the level, not the
//   scaled weight, to bf16: the same product with a different rounding, well
//   inside the tolerance of the bf16 What product.)
// * The lookup maps a code byte (two nibbles) to a packed pair of bf16 levels
//   through a 256-entry table in LDS, replicated once per lane so that every
//   lane reads its own bank: one v_perm (address) and one ds_read_b32 per two
//   weights.
// * Every global load is coalesced (consecutive lanes read consecutive
//   bytes: the address path of a CU handles such loads about three times
//   faster than loads in the MFMA operand layout, whose consecutive lanes sit
//   on different rows).  Codes: four lanes per row read a row's 64 bytes of a
//   pair of blocks; X and A: eight lanes per row read a block's 128 bytes.
//   Each wave then passes the data through a small LDS stage of its own,
//   padded so that the MFMA-layout reads are free of bank conflicts.
// * Work split: a workgroup (8 waves) owns up to TW <= 4 consecutive 16-row
//   tiles and one of S k-slices; the eight waves split the slice's blocks and
//   each runs all of the workgroup's tiles over its blocks, so an X fragment
//   is staged once per block per wave.  With enough tiles to occupy the chip
//   S = 1: a workgroup owns whole rows and writes Y itself.  With few tiles
//   S > 1: every workgroup stores its partial, and the last of the S
//   workgroups of a tile group (a counter in the workspace) adds the S
//   partials in slice order, the adapter term, and writes bf16 Y.  Cross-wave
//   sums run in a fixed order, so results do not depend on arrival order.
// * Streaming: a wave keeps the codes of its next blocks in a register ring
//   (RPC pairs) and the X / A of the next RXB blocks, refilled as each block
//   is consumed; the block loop is straight-line (blocks past the wave's
//   range read zero X and add nothing), so the compiler overlaps one block's
//   lookups and MFMAs with the next block's staging.
// * The LoRA down-projection U = X A^T (r <= 16) rides along: X is already
//   staged, so each block adds one MFMA pair on the A rows.
// * A weight stored without double quantization (one fp32 absmax per block)
//   takes the same path; each lane then loads the aligned 16-byte span that
//   holds its row's 8 block scales of an octet (three loads) instead of the
//   c2 bytes and the group's c1.
//
// MFMA v_mfma_f32_16x16x32_bf16, g = lane / 16: first operand lane (m, g)
// holds X[m][8 k], second operand lane (n, g) holds What[n][the same 8 k],
// result lane (n, g) register v is D[m = 4 g + v][n].  In block b, MFMA j
// (j = 0, 1) gives lane group g the k = 64 b + 16 g + 8 j .. + 7.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int DEC_WAVES = 8;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_MAX_TW = 4;                // tiles per workgroup
constexpr int DEC_MAX_S = 8;                 // k-slices
constexpr int DEC_MAX_GROUPS = 4096;         // counters reserved in the workspace
constexpr uint32_t DEC_TAG = 0x4E463444u;    // high word of an initialised counter
constexpr uint32_t DEC_OOB = 0x80000000u;    // buffer offset past every range used here
constexpr int DEC_US_LD = 132;               // row stride of U in LDS (r <= 128, 16-byte rows)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

struct DecodeArgs {
    const uint8_t *codes;  // W0 [d x k] packed NF4
    const int8_t *c2;
    const float *c1;
    const float *mean;
    int64_t d, k;
    const uint16_t *x;     // [M x k] bf16
    int M;
    const uint16_t *A;     // [r x k] bf16, read when U is null (r <= 16)
    const float *U;        // [M x r] fp32 computed beforehand, or null
    const uint16_t *B;     // [d x r] bf16
    int r;
    float s;
    uint16_t *y;           // [M x d] bf16
    float *u_save;         // [M x r] fp32 or null (fused U only)
    float *part;           // S > 1: partials [G S][TW + 1][64] f32x4: Y per tile, then U
    unsigned long long *ctr;  // S > 1: one counter per tile group
    int S, G;              // k-slices, tile groups (G S workgroups)
    // balanced splits, precomputed on the host (no wide division in the kernel):
    // group g has tiles [g tb + min(g, tr), +tb + (g < tr)), slice s has blocks
    // [s kbs + min(s, kr), +kbs + (s < kr))
    int tb, tr, kbs, kr;
    int bs;                // blocks of 64 << bs weights
    unsigned long long *span;  // null, or a measurement span (span_start / span_end)
};

// Device-coherent 16-byte store / load for partial sums handed from one
// workgroup to another, possibly on another XCD.  The hand-off is a release /
// acquire at device scope done with per-instruction scope bits instead of
// fences: the producer's partials are stored with device scope (sc1: written
// through the XCD's L2, which is not coherent with the other XCDs'), it waits
// for every store to be acknowledged at that scope (s_waitcnt vmcnt(0)) before
// its workgroup's arrival is counted by a device-scope atomic, and the
// consumer -- the workgroup that sees the last count -- reads the partials
// with device-scope loads (sc1: not served from its own L2), issued only after
// the atomic returned.  A device-scope release / acquire fence pair would
// give the same ordering by writing back and invalidating the whole L2 of
// both XCDs (about 4 us per call here); the scope bits confine it to the
// lines of the partials.
constexpr int DEC_SC1 = 16;
__device__ __forceinline__ void store16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, DEC_SC1);
}
__device__ __forceinline__ f32x4 load16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, DEC_SC1));
}

// B[row][j0 .. j0 + 7] as a bf16x8 MFMA operand (zero past r or when !ok).
// Straight-line code: every load is issued, out-of-range ones at an offset past
// the buffer (they read zero).
__device__ __forceinline__ uint4 load_bfrag(__amdgpu_buffer_rsrc_t rb, int row, int j0, int r, bool ok) {
    const bool live = ok && j0 < r;
    if (r % 8 == 0) return load16(rb, live ? (uint32_t)(((int64_t)row * r + j0) * 2) : DEC_OOB);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool in = live && j0 + e < r;
        h[e] = __builtin_amdgcn_raw_buffer_load_b16(rb, in ? (uint32_t)(((int64_t)row * r + j0 + e) * 2) : DEC_OOB,
                                                     0, 0);
    }
    return uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// TW tiles per workgroup; MV result registers that can hold m < M; XR row halves of X
// loaded (1: M <= 8); FU: U = X A^T computed here; F: the ScaleFormat of the block
// constants (double-quantized with int8 or FP8 c2, or the fp32 absmax of every block)
template <int TW, int MV, int XR, bool FU, int F>
__global__ __launch_bounds__(DEC_THREADS) void nf4_decode_kernel(DecodeArgs p, Nf4Consts tab) {
    constexpr bool DQ = F != kNoDq;
    constexpr int RPC = TW <= 2 ? 4 : 2;  // code pairs (two blocks each) in flight per wave
    constexpr int RXB = 2;                // X / A blocks in flight per wave
    constexpr int CP = 80;                // code stage row pitch: conflict-free 8-byte fragment reads
    constexpr int XP = 144;               // X / A stage row pitch: conflict-free 16-byte fragment reads
    constexpr int CSTAGE = 16 * CP;       // one tile's rows over a pair of blocks
    constexpr int XSTAGE = 16 * XP;       // one block of X or of A
    __shared__ __attribute__((aligned(16))) uint32_t tbl[256 * 64];  // pair table, one copy per lane
    __shared__ __attribute__((aligned(16))) unsigned char cst[DEC_WAVES][TW][CSTAGE];
    __shared__ __attribute__((aligned(16))) unsigned char xst[DEC_WAVES][2][XSTAGE];
    __shared__ int last_flag;
    // after the block loop the stages hold the cross-wave sums and U
    static_assert(sizeof(f32x4) * DEC_WAVES * TW * 64 <= sizeof(cst), "red alias");
    static_assert(sizeof(f32x4) * DEC_WAVES * 64 + sizeof(float) * 16 * DEC_US_LD <= sizeof(xst), "U alias");
    auto red = reinterpret_cast<f32x4 (*)[TW][64]>(&cst[0][0][0]);
    auto ured = reinterpret_cast<f32x4 (*)[64]>(&xst[0][0][0]);
    auto us = reinterpret_cast<float (*)[DEC_US_LD]>(&xst[0][0][0] + sizeof(f32x4) * DEC_WAVES * 64);

    // All offsets fit in 31 bits (d k <= 2^30, k <= 2^25): 32-bit index math.
    // Rows past d land past the end of their buffer and read zero.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    if (tid == 0) span_start(p.span);
    // the scalar arguments used before the block loop, requested together (one
    // wait for all of them instead of one per first use)
    asm volatile("" ::"s"(p.S), "s"(p.G), "s"(p.M), "s"(p.r), "s"(p.d), "s"(p.k), "s"(p.tb), "s"(p.tr),
                 "s"(p.kbs), "s"(p.kr), "s"(p.codes), "s"(p.c2), "s"(p.c1), "s"(p.mean), "s"(p.x), "s"(p.A));
    asm volatile("" ::"s"(p.B), "s"(p.U), "s"(p.part), "s"(tab.level[1]), "s"(tab.level[2]), "s"(tab.level[3]),
                 "s"(tab.level[4]), "s"(tab.level[5]), "s"(tab.level[6]), "s"(tab.level[7]), "s"(tab.level[8]),
                 "s"(tab.level[9]), "s"(tab.level[10]), "s"(tab.level[11]), "s"(tab.level[12]), "s"(tab.level[13]));
    asm volatile("" ::"s"(tab.level[14]), "s"(tab.level[15]), "s"(tab.level[0]));
    const int S = p.S, G = p.G, M = p.M, r = p.r;
    const int wg = blockIdx.x, sl = wg % S, grp = wg / S;
    const int d = (int)p.d, k = (int)p.k, kb = k / 64, hk = k / 2;
    // this group's tiles [t0, t0 + ntl), 1 <= ntl <= TW
    const int t0 = grp * p.tb + (grp < p.tr ? grp : p.tr);
    const int ntl = p.tb + (grp < p.tr ? 1 : 0);
    const int row_g = 16 * t0;
    // this wave's blocks [wb0, wb0 + nbw): the slice's blocks split eight ways (nbw may be 0)
    const int sb0 = sl * p.kbs + (sl < p.kr ? sl : p.kr);
    const int nsb = p.kbs + (sl < p.kr ? 1 : 0);
    const int wb0 = sb0 + nsb * wave / DEC_WAVES;
    const int nbw = nsb * (wave + 1) / DEC_WAVES - nsb * wave / DEC_WAVES;
    constexpr bool fuse_u = FU;

    const __amdgpu_buffer_rsrc_t rcode = make_rsrc(p.codes, (int64_t)d * hk);
    const int64_t nblk = ((int64_t)d * kb) >> p.bs;  // stored blocks
    const __amdgpu_buffer_rsrc_t rc2 = make_rsrc(p.c2, DQ ? nblk : 0);
    const __amdgpu_buffer_rsrc_t rc1 = make_rsrc(p.c1, (DQ ? (nblk + 255) / 256 : nblk) * 4);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (int64_t)M * k * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, fuse_u ? (int64_t)r * k * 2 : 0);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (int64_t)d * r * 2);
    const __amdgpu_buffer_rsrc_t rmean = make_rsrc(p.mean, DQ ? 4 : 0);
    const int64_t part_f4 = S > 1 ? (int64_t)G * S * (TW + 1) * 64 : 0;  // f32x4 slots
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part, part_f4 * 16);

    // wave w < ntl finishes tile w: its B fragments for the adapter term
    uint4 bfr = uint4{0, 0, 0, 0};
    if (wave < ntl) bfr = load_bfrag(rb, row_g + 16 * wave + n16, 8 * g, r, true);
    // a given U [M x r] (r > 16): prefetched, parked in LDS after the block loop
    constexpr int NUV = 16 * 128 / DEC_THREADS;
    float uvv[NUV];
    if (!fuse_u) {
        const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.U, (int64_t)M * r * 4);
#pragma unroll
        for (int u = 0; u < NUV; ++u) {
            const int e = tid + DEC_THREADS * u;
            uvv[u] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(ru, e < M * r ? (uint32_t)e * 4 : DEC_OOB, 0, 0));
        }
    }
    // the DQ mean through the vector memory path (a scalar load would make the
    // wave wait for it before issuing anything else)
    const float mean = DQ ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rmean, 0, 0, 0)) : 0.0f;

    // ---- coalesced loads into register rings -----------------------------------
    // Block b of the wave (0 <= b < nbw) is k-block wb0 + b.  Loads past the
    // wave's blocks or the group's tiles go to an offset past every buffer
    // (zero, no memory traffic), so every trip issues the same loads.
    // codes, pair q = blocks 2q, 2q+1 of tile t: lane 4 n + c holds bytes
    // 16 c .. 16 c + 15 of row n's 64 bytes (four lanes per row)
    uint4 cr[RPC][TW];
    const uint32_t code_lane = (uint32_t)((row_g + (lane >> 2)) * hk + 32 * wb0 + 16 * (lane & 3));
    const uint32_t tile_bytes = 16u * (uint32_t)hk;
    auto issue_codes = [&](int q, int j) __attribute__((always_inline)) {
        const bool ok = 2 * q < nbw;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const uint32_t off = ok && t < ntl ? code_lane + (uint32_t)t * tile_bytes + 64u * (uint32_t)q : DEC_OOB;
            cr[j][t] = load16(rcode, off);
        }
    };
    // X and A block b: lane l holds row 8 i + l / 8, bytes 16 (l % 8) .. + 15 of the
    // block's 128 (eight lanes per row); rows past M (X) or r (A) read zero.
    // With M <= 8 only X rows 0..7 are loaded: stage rows 8..15 keep stale
    // values, which reach only result rows m >= M (each MFMA result row depends
    // on its own X row alone) and those are never stored.
    uint4 xr[RXB][2], ar[RXB][2];
    const uint32_t xa_lane = (uint32_t)(((lane >> 3) * k + 64 * wb0 + 8 * (lane & 7)) * 2);
    auto issue_xa = [&](int b, int j) __attribute__((always_inline)) {
        const bool ok = b < nbw;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t off = ok ? xa_lane + (uint32_t)(16 * i * k) + 128u * (uint32_t)b : DEC_OOB;
            if (i < XR) xr[j][i] = load16(rx, off);
            if (fuse_u) ar[j][i] = load16(ra, off);
        }
    };
    // block constants of an octet (8 blocks from o): lane (n, g) takes row n of
    // tile g (g < ntl): its 8 c2 bytes from three aligned dwords, and the c1 of
    // the first and of the last block (8 blocks span at most two groups of 256).
    // Single-dword loads: each one is range-checked on its own.  Without double
    const int srow = row_g + 16 * g + n16;
    const bool srow_ok = g < ntl && srow < d;
    const uint32_t c2_lane = (uint32_t)(srow * kb + wb0);
    // quantization the lane loads the 16-byte aligned span of fp32 absmax
    // values that holds the octet's 8 (three 16-byte loads; d % 8 == 0 makes
    // every aligned 4-value group wholly inside or wholly past the buffer) and
    // picks its 8 by the offset inside the span.
    constexpr int NCW = DQ ? 3 : 1;
    constexpr int NCS = DQ ? 1 : 3;
    uint32_t c2w[NCW];
    float c1a, c1b;
    uint4 absv[NCS];
    // Blocks of 64 << bs weights: sub-block j (64 weights) takes block j >> bs, so
    // an octet spans at most 8 blocks from b0 = (c2_lane + o) >> bs; the same
    // windows from the aligned a0 = b0 & ~3 cover them.
    const int bs = p.bs;
    auto issue_c2 = [&](int o) __attribute__((always_inline)) {
        const uint32_t o8 = c2_lane + (uint32_t)o, b0 = o8 >> bs, a0 = b0 & ~3u;
        const bool ok = srow_ok && o < nbw;
        if constexpr (DQ) {
#pragma unroll
            for (int i = 0; i < NCW; ++i)
                c2w[i] = __builtin_amdgcn_raw_buffer_load_b32(rc2, ok ? a0 + 4u * i : DEC_OOB, 0, 0);
            c1a = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc1, ok ? (b0 >> 8) * 4 : DEC_OOB, 0, 0));
            c1b = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rc1, ok ? (((o8 + 7) >> bs) >> 8) * 4 : DEC_OOB, 0, 0));
        } else {
#pragma unroll
            for (int i = 0; i < NCS; ++i) absv[i] = load16(rc1, ok ? (a0 + 4u * i) * 4 : DEC_OOB);
        }
    };

    // The first block's loads go out before the table is built (the barrier
    // after it then waits only for a few issued loads per wave); the rest of
    // the ring follows: codes (from HBM, the longest wait), then X / A.  The
    // block loop refills one X / A block per block consumed.
    issue_codes(0, 0);
    issue_c2(0);
    issue_xa(0, 0);
    // pair table, while the first block's loads are under way: entry e = bf16(C[e & 15]) |
    // bf16(C[e >> 4]) << 16 at dword 64 e + lane
    {
        // the levels pass through scalar registers: left to itself the compiler
        // turns this select into an indexed load from the argument segment
        float lvf = tab.level[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            float cj;
            asm("s_mov_b32 %0, %1" : "=s"(cj) : "s"(tab.level[j]));
            lvf = n16 == j ? cj : lvf;
        }
        const int lv = __float_as_int(lvf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int flat = tid + DEC_THREADS * i;
            const int e = flat >> 4;
            const float lo = __int_as_float(__builtin_amdgcn_ds_bpermute((e & 15) << 2, lv));
            const float hi = __int_as_float(__builtin_amdgcn_ds_bpermute((e >> 4) << 2, lv));
            const uint32_t v = pack_bf16x2(lo, hi);
            reinterpret_cast<uint4 *>(tbl)[flat] = uint4{v, v, v, v};
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 1; j < RPC; ++j) issue_codes(j, j);
#pragma unroll
    for (int j = 1; j < RXB; ++j) issue_xa(j, j);

    const uint32_t lane4 = (uint32_t)lane * 4;
    const char *tbl_b = reinterpret_cast<const char *>(tbl);
    // byte i of a code dword -> LDS byte address (byte << 8) | (lane << 2)
    auto lut4 = [&](uint32_t cd) __attribute__((always_inline)) {
        uint4 o;
        o.x = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0400u));
        o.y = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0500u));
        o.z = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0600u));
        o.w = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0700u));
        return o;
    };
    // stage addresses of this lane: ring writes (coalesced layout) and MFMA
    // fragment reads.  Fragment k order inside a block: MFMA jj gives lane
    // group g the k = 16 g + 8 jj .. + 7, i.e. code bytes 8 g + 4 jj .. + 3.
    unsigned char *const cst_w = &cst[wave][0][0];
    unsigned char *const xst_w = &xst[wave][0][0];
    const int cst_wr = (lane >> 2) * CP + 16 * (lane & 3);
    const int cst_rd = n16 * CP + 8 * g;             // + 32 h for block h of the pair
    const int xst_wr = (lane >> 3) * XP + 16 * (lane & 7);  // + 8 XP i
    const int xst_rd = n16 * XP + 32 * g;            // + 16 jj

    f32x4 acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 uacc = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int o = 0; o < nbw; o += 8) {
        // block scales of the octet (zero for rows past d and tiles past ntl)
        float sc[8];
        if constexpr (!DQ) {
            const uint32_t f[12] = {absv[0].x, absv[0].y, absv[0].z, absv[0].w, absv[1].x, absv[1].y,
                                    absv[1].z, absv[1].w, absv[2].x, absv[2].y, absv[2].z, absv[2].w};
            if (bs == 0) {
                const uint32_t sh = (c2_lane + (uint32_t)o) & 3u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t v = sh == 0 ? f[e] : sh == 1 ? f[e + 1] : sh == 2 ? f[e + 2] : f[e + 3];
                    // blocks past nbw (another wave's, or the next row's) and rows past d add nothing
                    sc[e] = srow_ok && o + e < nbw ? __uint_as_float(v) : 0.0f;
                }
            } else {
                const uint32_t o8 = c2_lane + (uint32_t)o, a0 = (o8 >> bs) & ~3u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t off = ((o8 + (uint32_t)e) >> bs) - a0;  // 0 .. 6
                    uint32_t v = f[0];
#pragma unroll
                    for (int c = 1; c < 12; ++c) v = off == (uint32_t)c ? f[c] : v;
                    sc[e] = srow_ok && o + e < nbw ? __uint_as_float(v) : 0.0f;
                }
            }
        } else if (bs != 0) {
            const uint32_t o8 = c2_lane + (uint32_t)o, b0 = o8 >> bs, a0 = b0 & ~3u, ga = b0 >> 8;
            const uint64_t lo64 = (uint64_t)c2w[1] << 32 | c2w[0], hi64 = (uint64_t)c2w[2] << 32 | c2w[1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t idx = (o8 + (uint32_t)e) >> bs, off = idx - a0;  // 0 .. 6
                const uint32_t byte = (uint32_t)(off < 8 ? lo64 >> (8 * off) : hi64 >> (8 * (off - 4)));
                const float c2 = c2_value<0>(byte, F == kDqFp8);
                const bool ok = srow_ok && o + e < nbw;
                const float c1 = ok ? ((idx >> 8) == ga ? c1a : c1b) : 1.0f;
                sc[e] = dq_scale(c2, c1, mean) * (ok ? 1.0f : 0.0f);
            }
        } else {
            const uint32_t sh = 8 * ((c2_lane + (uint32_t)o) & 3u);
            const uint32_t lo = (uint32_t)(((uint64_t)c2w[1] << 32 | c2w[0]) >> sh);
            const uint32_t hi = (uint32_t)(((uint64_t)c2w[2] << 32 | c2w[1]) >> sh);
            const uint32_t ga = (c2_lane + (uint32_t)o) >> 8;
            constexpr bool fp8 = F == kDqFp8;
            const float c2v[8] = {c2_value<0>(lo, fp8), c2_value<1>(lo, fp8), c2_value<2>(lo, fp8),
                                  c2_value<3>(lo, fp8), c2_value<0>(hi, fp8), c2_value<1>(hi, fp8),
                                  c2_value<2>(hi, fp8), c2_value<3>(hi, fp8)};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float c2 = c2v[e];
                // blocks past nbw and rows past d get scale 0 from a finite
                // quotient (c1 = 1), so no NaN meets their zero products
                const bool ok = srow_ok && o + e < nbw;
                const float c1 = ok ? (((c2_lane + (uint32_t)(o + e)) >> 8) == ga ? c1a : c1b) : 1.0f;
                sc[e] = dq_scale(c2, c1, mean) * (ok ? 1.0f : 0.0f);  // exact: x * 1 = x
            }
        }
        issue_c2(o + 8);
        // Straight-line over the octet: blocks past nbw have zero X (their loads
        // read past the buffer) and so add nothing; tiles past ntl are computed
        // from zero codes and never stored.
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // pairs of the octet
            const int q = o / 2 + j;
#pragma unroll
            for (int t = 0; t < TW; ++t) *reinterpret_cast<uint4 *>(cst_w + t * CSTAGE + cst_wr) = cr[j % RPC][t];
            issue_codes(q + RPC, j % RPC);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = o + 2 * j + h;
                const int jx = (2 * j + h) % RXB;
                *reinterpret_cast<uint4 *>(xst_w + xst_wr) = xr[jx][0];
                if (XR == 2) *reinterpret_cast<uint4 *>(xst_w + xst_wr + 8 * XP) = xr[jx][1];
                if (fuse_u) {
                    *reinterpret_cast<uint4 *>(xst_w + XSTAGE + xst_wr) = ar[jx][0];
                    *reinterpret_cast<uint4 *>(xst_w + XSTAGE + xst_wr + 8 * XP) = ar[jx][1];
                }
                issue_xa(b + RXB, jx);
                const uint4 xf0 = *reinterpret_cast<const uint4 *>(xst_w + xst_rd);
                const uint4 xf1 = *reinterpret_cast<const uint4 *>(xst_w + xst_rd + 16);
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const uint2 cd = *reinterpret_cast<const uint2 *>(cst_w + t * CSTAGE + cst_rd + 32 * h);
                    const uint4 w0 = lut4(cd.x), w1 = lut4(cd.y);
                    f32x4 z = mfma16(xf0, w0, f32x4{0.f, 0.f, 0.f, 0.f});
                    z = mfma16(xf1, w1, z);
                    // the scale of (tile t, row n): computed by lane (n, t)
                    const float st =
                        __int_as_float(__builtin_amdgcn_ds_bpermute((n16 + 16 * t) * 4, __float_as_int(sc[2 * j + h])));
#pragma unroll
                    for (int v = 0; v < MV; ++v) acc[t][v] = __builtin_fmaf(st, z[v], acc[t][v]);
                }
                if (fuse_u) {
                    const uint4 af0 = *reinterpret_cast<const uint4 *>(xst_w + XSTAGE + xst_rd);
                    const uint4 af1 = *reinterpret_cast<const uint4 *>(xst_w + XSTAGE + xst_rd + 16);
                    uacc = mfma16(xf0, af0, uacc);
                    uacc = mfma16(xf1, af1, uacc);
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // bounds the scheduling window (register pressure)
        }
    }

    // ---- cross-wave sums (fixed order) --------------------------------------
    // the group counter: read here, used after the partials are out; a fresh
    // workspace gets it tagged
    unsigned long long ctr0 = 0;
    if (S > 1 && tid == 0) ctr0 = __hip_atomic_load(p.ctr + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // every wave is done with its stages
#pragma unroll
    for (int t = 0; t < TW; ++t) red[wave][t][lane] = acc[t];
    if (fuse_u) ured[wave][lane] = uacc;
    __syncthreads();
    // wave w < TW: tile w, the eight waves' sums in wave order
    f32x4 ysum = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < TW) {
#pragma unroll
        for (int q = 0; q < DEC_WAVES; ++q) ysum += red[q][wave][lane];
    }
    // with U fused, every wave that finishes a tile forms U itself
    f32x4 usum = f32x4{0.f, 0.f, 0.f, 0.f};
    if (fuse_u && wave < ntl) {
#pragma unroll
        for (int q = 0; q < DEC_WAVES; ++q) usum += ured[q][lane];
    }

    if (S > 1) {
        // publish this slice's partials (slots [wg][t][lane], then U at [wg][TW][lane]);
        // the last workgroup of the group to arrive adds all S in slice order
        if (wave < ntl) store16_sc1(rp, (uint32_t)((((int64_t)wg * (TW + 1) + wave) * 64 + lane) * 16), ysum);
        if (fuse_u && wave == 0) store16_sc1(rp, (uint32_t)((((int64_t)wg * (TW + 1) + TW) * 64 + lane) * 16), usum);
        __builtin_amdgcn_s_waitcnt(0);  // stores acknowledged before the count
        __syncthreads();
        if (tid == 0) {
            unsigned long long *c = p.ctr + grp;
            const unsigned long long tag0 = (unsigned long long)DEC_TAG << 32;
            if ((ctr0 >> 32) != DEC_TAG) {  // first use of this workspace: tag the counter
                unsigned long long expect = ctr0;
                __hip_atomic_compare_exchange_strong(c, &expect, tag0, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
            }
            const unsigned long long old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = (int)(old & 0xFFFFFFFFull) == S - 1;
            if (last) __hip_atomic_store(c, tag0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = last;
        }
        __syncthreads();
        if (!last_flag) {
            if (tid == 0) span_end(p.span);  // measurement only
            return;
        }
        f32x4 pv[DEC_MAX_S], uv[DEC_MAX_S];
#pragma unroll
        for (int q = 0; q < DEC_MAX_S; ++q) {
            const int64_t slot = (int64_t)(grp * S + q) * (TW + 1);
            pv[q] = q < S && wave < ntl ? load16_sc1(rp, (uint32_t)(((slot + wave) * 64 + lane) * 16))
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
            uv[q] = q < S && fuse_u && wave < ntl ? load16_sc1(rp, (uint32_t)(((slot + TW) * 64 + lane) * 16))
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 a = pv[0], u = uv[0];
#pragma unroll
        for (int q = 1; q < DEC_MAX_S; ++q)
            if (q < S) {
                a += pv[q];
                u += uv[q];
            }
        ysum = a;
        usum = u;
    }

    // ---- adapter term and bf16 store ------------------------------------------
    // U [m][j] in LDS, read back in the first-operand layout: a given U (any
    // r <= 128) in the shared array behind a barrier; a fused U (r <= 16) in
    // this wave's own small array (same-wave LDS accesses stay in order)
    constexpr int UWP = 20;  // row pitch of the per-wave U (r <= 16)
    static_assert(sizeof(f32x4) * DEC_WAVES * 64 + sizeof(float) * 16 * UWP * DEC_MAX_TW <= sizeof(xst), "U alias");
    float *const usw = reinterpret_cast<float *>(&xst[0][0][0] + sizeof(f32x4) * DEC_WAVES * 64) + wave * 16 * UWP;
    if (!fuse_u) {
#pragma unroll
        for (int u = 0; u < NUV; ++u) {
            const int e = tid + DEC_THREADS * u;
            if (e < M * r) us[e / r][e % r] = uvv[u];
        }
        __syncthreads();
    }
    if (wave >= ntl) return;
    if (fuse_u) {
        // lane (j, g) holds U[4 g + v][j]
#pragma unroll
        for (int v = 0; v < 4; ++v) usw[(4 * g + v) * UWP + n16] = usum[v];
        if (p.u_save && grp == 0 && wave == 0 && n16 < r) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (4 * g + v < M) p.u_save[(4 * g + v) * r + n16] = usum[v];
        }
    }
    // U B^T by MFMA over 32-wide slices of j: U split into bf16 hi + lo, lane
    // (m, g) holds U[m][32 it + 8 g .. + 7], lane (n, g) holds B[n][same j]
    const int row = row_g + 16 * wave + n16;
    f32x4 ad = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nj = (r + 31) / 32;
    for (int it = 0; it < nj; ++it) {
        const int j0 = 32 * it + 8 * g;
        uint4 uhi{0, 0, 0, 0}, ulo{0, 0, 0, 0};
        if (j0 < r) {
            const float *const ur = fuse_u ? usw + n16 * UWP + j0 : &us[n16][j0];
            const f32x4 u0 = *reinterpret_cast<const f32x4 *>(ur);
            const f32x4 u1 = *reinterpret_cast<const f32x4 *>(ur + 4);
            float uu[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) uu[e] = j0 + e < r ? uu[e] : 0.0f;
            uint32_t h2[4], l2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h2[e] = pack_bf16x2(uu[2 * e], uu[2 * e + 1]);
                l2[e] = pack_bf16x2(uu[2 * e] - bf16_bits_to_f32(h2[e] & 0xFFFFu),
                                    uu[2 * e + 1] - bf16_bits_to_f32(h2[e] >> 16));
            }
            uhi = uint4{h2[0], h2[1], h2[2], h2[3]};
            ulo = uint4{l2[0], l2[1], l2[2], l2[3]};
        }
        const uint4 bf = it == 0 ? bfr : load_bfrag(rb, row, j0, r, true);
        ad = mfma16(uhi, bf, ad);
        ad = mfma16(ulo, bf, ad);
    }
    // all loads are done: the stores below never wait on each other
    if (row >= d) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m >= M) continue;
        const float out = ysum[v] + p.s * ad[v];
        p.y[(int64_t)m * d + row] = (uint16_t)(pack_bf16x2(out, 0.0f) & 0xFFFFu);
    }
    if (p.span && n16 == 0) {  // measurement only: this lane's stores are out
        __builtin_amdgcn_s_waitcnt(0);
        span_end(p.span);
    }
}

struct DecodePlan {
    int S, G, TW, grid;
};

// Enough 16-row tiles to occupy the chip (>= 128): one k-slice, up to 256
// tile groups of up to four tiles (more groups only past 1024 tiles).
// Fewer tiles: one tile per group and up to eight k-slices, each wave of a
// slice keeping at least one block.
DecodePlan decode_plan(int64_t d, int64_t k) {
    const int64_t kb = k / 64, nt = (d + 15) / 16;
    DecodePlan pl;
    if (nt >= 128) {
        int64_t tw = (nt + 255) / 256;
        tw = tw > DEC_MAX_TW ? DEC_MAX_TW : tw;
        pl.TW = (int)tw;
        pl.G = (int)(nt > 256 * DEC_MAX_TW ? (nt + DEC_MAX_TW - 1) / DEC_MAX_TW : (nt < 256 ? nt : 256));
        pl.S = 1;
    } else {
        int64_t S = 256 / nt;
        const int64_t smax = kb / DEC_WAVES;
        S = S > smax ? smax : S;
        S = S > DEC_MAX_S ? DEC_MAX_S : (S < 1 ? 1 : S);
        pl.TW = 1;
        pl.G = (int)nt;
        pl.S = (int)S;
    }
    pl.grid = pl.G * pl.S;
    return pl;
}

template <int TW, bool FU, int F>
hipError_t launch_fu(const DecodeArgs &a, int grid, hipStream_t st) {
    if (a.M == 1) hipLaunchKernelGGL((nf4_decode_kernel<TW, 1, 1, FU, F>), dim3(grid), dim3(DEC_THREADS), 0, st, a, nf4_consts());
    else if (a.M <= 8) hipLaunchKernelGGL((nf4_decode_kernel<TW, 4, 1, FU, F>), dim3(grid), dim3(DEC_THREADS), 0, st, a, nf4_consts());
    else hipLaunchKernelGGL((nf4_decode_kernel<TW, 4, 2, FU, F>), dim3(grid), dim3(DEC_THREADS), 0, st, a, nf4_consts());
    return hipGetLastError();
}

template <int TW, int F>
hipError_t launch_f(const DecodeArgs &a, int grid, hipStream_t st) {
    return a.U ? launch_fu<TW, false, F>(a, grid, st) : launch_fu<TW, true, F>(a, grid, st);
}

template <int TW>
hipError_t launch_tw(const DecodeArgs &a, int fmt, int grid, hipStream_t st) {
    if (fmt == kDqInt8) return launch_f<TW, kDqInt8>(a, grid, st);
    if (fmt == kDqFp8) return launch_f<TW, kDqFp8>(a, grid, st);
    return launch_f<TW, kNoDq>(a, grid, st);
}

}  // namespace

size_t decode_counter_bytes() { return sizeof(unsigned long long) * DEC_MAX_GROUPS; }

size_t decode_part_bytes(int64_t M, int64_t d, int64_t k) {
    if (M < 1 || M > kDecodeChunkRows) return 0;  // per 16-row chunk: the same for every chunk
    const DecodePlan pl = decode_plan(d, k);
    if (pl.S == 1) return 0;
    return sizeof(f32x4) * (size_t)pl.grid * 64 * ((size_t)pl.TW + 1);
}

hipError_t launch_decode_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const uint16_t *A, const float *U,
                             const uint16_t *B, int r, float s, uint16_t *Y, float *U_save, float *part,
                             unsigned long long *ctr, hipStream_t st) {
    if (M < 1 || M > 16 || (!U && (!A || r > 16)) || w.k > (int64_t(1) << 25)) return hipErrorInvalidValue;
    if (!U && decode_dot_supported(M, w.d, w.k, r))
        return launch_decode_dot(w, x, M, A, B, r, s, Y, U_save, timing_take(kTimeDecode), st);
    const DecodePlan pl = decode_plan(w.d, w.k);
    if (pl.S > 1 && (!part || !ctr || pl.G > DEC_MAX_GROUPS)) return hipErrorInvalidValue;
    DecodeArgs a;
    a.codes = w.codes;
    a.c2 = w.c2;
    a.c1 = w.c1;
    a.mean = w.mean;
    a.d = w.d;
    a.k = w.k;
    a.x = x;
    a.M = (int)M;
    a.A = A;
    a.U = U;
    a.B = B;
    a.r = r;
    a.s = s;
    a.y = Y;
    a.u_save = U ? nullptr : U_save;
    a.part = part;
    a.ctr = ctr;
    a.S = pl.S;
    a.G = pl.G;
    const int64_t nt = (w.d + 15) / 16, kb = w.k / 64;
    a.tb = (int)(nt / pl.G);
    a.tr = (int)(nt % pl.G);
    a.kbs = (int)(kb / pl.S);
    a.kr = (int)(kb % pl.S);
    a.bs = w.bshift;
    a.span = timing_take(kTimeDecode);
    switch (pl.TW) {
        case 1: return launch_tw<1>(a, w.fmt, pl.grid, st);
        case 2: return launch_tw<2>(a, w.fmt, pl.grid, st);
        case 3: return launch_tw<3>(a, w.fmt, pl.grid, st);
        default: return launch_tw<4>(a, w.fmt, pl.grid, st);
    }
}

}  // namespace qnf4
