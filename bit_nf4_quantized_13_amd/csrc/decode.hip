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
// * Codes are read with 8-byte loads, four lanes per row and 32 bytes (one
//   block) per row per load; one ds_bpermute per code dword moves them into the
//   MFMA operand layout.
// * Work split: a workgroup (8 waves) takes T tiles of 16 rows and one of S
//   k-slices; its waves split the slice P ways and the tiles 8/P ways.  X and A
//   fragments of a wave's k-range stay in registers for all of its tiles.
//   Partial sums are reduced across waves in LDS in a fixed order; with S > 1
//   every workgroup stores its partial, and the last of the S workgroups of a
//   tile group (a counter in the workspace) adds the S partials in slice order,
//   the adapter term, and writes bf16 Y.  Results do not depend on arrival order.
// * The LoRA down-projection U = X A^T (r <= 16) rides along: X is already in
//   registers, so each k-range adds one MFMA pair per block on the A rows.
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
constexpr int DEC_KB = 4;                    // 64-deep blocks per wave per chunk
constexpr int DEC_MAX_TW = 8;                // tiles per wave
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
    float *part;           // partials [grid][T + 1][64] f32x4: Y per tile, then U
    unsigned long long *ctr;  // one per tile group
    int S, T, P, nbw;      // k-slices, tiles per group, waves per tile subset, blocks per wave
    int grid_;             // workgroups
};

// Device-coherent 16-byte store / load (sc1: not cached non-coherently in the
// per-XCD L2), for partial sums handed from one workgroup to another.
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

template <int TW, int MV>  // TW tiles per wave; MV result registers that can hold m < M
__global__ __launch_bounds__(DEC_THREADS) void nf4_decode_kernel(DecodeArgs p, Nf4Consts tab) {
    __shared__ __attribute__((aligned(16))) uint32_t tbl[256 * 64];  // pair table, one copy per lane
    __shared__ f32x4 red[DEC_WAVES][TW][64];
    __shared__ f32x4 ured[DEC_WAVES][64];
    __shared__ __attribute__((aligned(16))) float us[16][DEC_US_LD];  // U [m][j] for the adapter term
    __shared__ int last_flag;

    // All offsets fit in 31 bits (d k <= 2^30, k <= 2^25): 32-bit index math.
    // Rows past d land past the end of their buffer and read zero.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int S = p.S, P = p.P, T = p.T, M = p.M, r = p.r;
    const int wg = blockIdx.x, sl = wg % S, grp = wg / S;
    const int kpart = wave % P, tsub = wave / P;
    const int d = (int)p.d, k = (int)p.k, kb = k / 64, hk = k / 2;
    const int wblk0 = (sl * P + kpart) * p.nbw;                  // this wave's blocks [wblk0, wblk1)
    const int wblk1 = wblk0 + p.nbw < kb ? wblk0 + p.nbw : kb;
    const int row_g = grp * T * 16;                               // first row of the tile group
    const int row_w = row_g + tsub * TW * 16;                     // first row of this wave's tiles
    const bool fuse_u = p.U == nullptr;
    const bool u_wave = fuse_u && tsub == 0;

    const __amdgpu_buffer_rsrc_t rcode = make_rsrc(p.codes, (int64_t)d * hk);
    const __amdgpu_buffer_rsrc_t rc2 = make_rsrc(p.c2, (int64_t)d * kb);
    const __amdgpu_buffer_rsrc_t rc1 = make_rsrc(p.c1, (((int64_t)d * kb + 255) / 256) * 4);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (int64_t)M * k * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, fuse_u ? (int64_t)r * k * 2 : 0);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (int64_t)d * r * 2);
    const __amdgpu_buffer_rsrc_t rmean = make_rsrc(p.mean, 4);
    const int64_t part_f4 = p.S > 1 ? (int64_t)p.grid_ * (T + 1) * 64 : 0;  // f32x4 slots
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part, part_f4 * 16);

    // thread (tile tt of the group, lane): tt = wave, wave + 8; B fragments for the adapter
    constexpr int NTT = (2 * DEC_MAX_TW + DEC_WAVES - 1) / DEC_WAVES;
    uint4 bfr[NTT];
#pragma unroll
    for (int h = 0; h < NTT; ++h) {
        const int tt = wave + DEC_WAVES * h;
        bfr[h] = load_bfrag(rb, row_g + 16 * tt + n16, 8 * g, r, tt < T);
    }

    // a given U [M x r] (r > 16): prefetched, parked in LDS with the table
    constexpr int NUV = 16 * 128 / DEC_THREADS;
    float uvv[NUV];
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.U, fuse_u ? 0 : (int64_t)M * r * 4);
#pragma unroll
    for (int u = 0; u < NUV; ++u) {
        const int e = tid + DEC_THREADS * u;
        uvv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ru, e < M * r ? (uint32_t)e * 4 : DEC_OOB, 0, 0));
    }

    f32x4 acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 uacc = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint32_t lane4 = (uint32_t)lane * 4;
    const int code_src = (4 * n16 + g) * 4;  // lane holding dwords 2 g, 2 g + 1 of row n16
    const char *tbl_b = reinterpret_cast<const char *>(tbl);
    // byte i of a code dword -> LDS byte address (byte << 8) | (lane << 2)
    auto lut4 = [&](uint32_t cd) {
        uint4 o;
        o.x = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0400u));
        o.y = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0500u));
        o.z = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0600u));
        o.w = *reinterpret_cast<const uint32_t *>(tbl_b + __builtin_amdgcn_perm(cd, lane4, 0x0C0C0700u));
        return o;
    };

    constexpr int NI = TW * DEC_KB;          // (tile, block) items per chunk, tile-major
    constexpr int NQ = (TW + 3) / 4;         // tiles whose block constants this lane loads
    constexpr int D = NI;                    // code loads in flight per wave: all of the chunk's
    const uint32_t tstride = 16u * (uint32_t)hk;  // bytes of codes per 16-row tile
    const int nchunks = (p.nbw + DEC_KB - 1) / DEC_KB;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int cb = wblk0 + ch * DEC_KB;
        const int nval = wblk1 - cb;  // blocks of this chunk in range (uniform; may be <= 0)
        // codes of item i: lane 4 n + q reads bytes 8 q .. 8 q + 7 of row n's block
        const uint32_t code0 = (uint32_t)((row_w + (lane >> 2)) * hk + 32 * cb + 8 * (lane & 3));
        auto load_code = [&](int i) {
            const int t = i / DEC_KB, b = i % DEC_KB;
            const uint32_t off = b < nval ? code0 + (uint32_t)t * tstride + 32u * b : DEC_OOB;
            return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rcode, off, 0, 0));
        };
        // X (and A) fragments of the chunk's blocks
        const uint32_t x0 = (uint32_t)((n16 * k + 64 * cb + 16 * g) * 2);
        uint4 xf[DEC_KB][2], af[DEC_KB][2];
#pragma unroll
        for (int b = 0; b < DEC_KB; ++b) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t off = b < nval ? x0 + 128u * b + 16u * j : DEC_OOB;
                xf[b][j] = load16(rx, off);
                af[b][j] = u_wave ? load16(ra, off) : uint4{0, 0, 0, 0};
            }
        }
        // block constants: lane (n, g) loads tiles t = g + 4 u of row n: the chunk's
        // four c2 bytes as one dword and their one c1 (four blocks at a multiple of
        // four never straddle a 256-block group)
        const bool c2vec = (kb % 4 == 0) && (cb % 4 == 0);  // uniform
        uint32_t c2w[NQ];
        float c1q[NQ][DEC_KB];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int row = row_w + 16 * (g + 4 * u) + n16;
            const uint32_t jb = (uint32_t)(row * kb + cb);
            const bool tile_ok = g + 4 * u < TW && nval > 0;
            if (c2vec) {
                c2w[u] = __builtin_amdgcn_raw_buffer_load_b32(rc2, tile_ok ? jb : DEC_OOB, 0, 0);
                const float c1 = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rc1, tile_ok ? (jb >> 8) * 4 : DEC_OOB, 0, 0));
#pragma unroll
                for (int b = 0; b < DEC_KB; ++b) c1q[u][b] = c1;
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int b = 0; b < DEC_KB; ++b) {
                    const bool ok = tile_ok && b < nval;
                    w |= __builtin_amdgcn_raw_buffer_load_b8(rc2, ok ? jb + b : DEC_OOB, 0, 0) << (8 * b);
                    c1q[u][b] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rc1, ok ? ((jb + b) >> 8) * 4 : DEC_OOB, 0, 0));
                }
                c2w[u] = w;
            }
        }
        // the DQ mean through the vector memory path (a scalar load would make the
        // wave wait for it before issuing anything else)
        const float mean = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rmean, 0, 0, 0));
        uint2 cw[D];
#pragma unroll
        for (int i = 0; i < D; ++i) cw[i] = load_code(i);
        if (ch == 0) {
            // pair table: entry e = bf16(C[e & 15]) | bf16(C[e >> 4]) << 16 at dword 64 e + lane
            float lvf = tab.level[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) lvf = n16 == j ? tab.level[j] : lvf;
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
            if (!fuse_u) {
#pragma unroll
                for (int u = 0; u < NUV; ++u) {
                    const int e = tid + DEC_THREADS * u;
                    if (e < M * r) us[e / r][e % r] = uvv[u];
                }
            }
            __syncthreads();
        }
        if (u_wave) {  // U partial while the codes are in flight
#pragma unroll
            for (int b = 0; b < DEC_KB; ++b) {
                uacc = mfma16(xf[b][0], af[b][0], uacc);
                uacc = mfma16(xf[b][1], af[b][1], uacc);
            }
        }
        // scales of the loaded constants (zero for blocks out of range and rows past d)
        float sq[NQ][DEC_KB];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const bool row_ok = row_w + 16 * (g + 4 * u) + n16 < d;
#pragma unroll
            for (int b = 0; b < DEC_KB; ++b) {
                const int8_t c2 = (int8_t)((c2w[u] >> (8 * b)) & 0xFFu);
                sq[u][b] = row_ok && b < nval ? dq_scale(c2, c1q[u][b], mean) : 0.0f;
            }
        }

        // four-stage software pipeline over the items, so that the LDS round
        // trips of one item overlap the MFMAs of the previous ones:
        //   A(i): code dwords into MFMA layout (ds_bpermute)
        //   B(i): NF4 pair lookups (v_perm + ds_read_b32) and the item's scale
        //   C(i): MFMA pair on the block
        //   E(i): scaled accumulation into the tile's sum
        uint32_t cd[2][2];
        uint4 wv[2][2];
        float scv[4];
        f32x4 tmp[2];
#pragma unroll
        for (int it = 0; it < NI + 3; ++it) {
            __builtin_amdgcn_sched_barrier(0);  // keep the stages of one step together
            if (it >= 3) {  // E(it - 3)
                const int i = it - 3, t = i / DEC_KB;
#pragma unroll
                for (int v = 0; v < MV; ++v) acc[t][v] = __builtin_fmaf(scv[i % 4], tmp[i % 2][v], acc[t][v]);
            }
            if (it >= 2 && it - 2 < NI) {  // C(it - 2)
                const int i = it - 2, b = i % DEC_KB;
                f32x4 z = mfma16(xf[b][0], wv[i % 2][0], f32x4{0.f, 0.f, 0.f, 0.f});
                tmp[i % 2] = mfma16(xf[b][1], wv[i % 2][1], z);
            }
            if (it >= 1 && it - 1 < NI) {  // B(it - 1)
                const int i = it - 1, t = i / DEC_KB, b = i % DEC_KB;
                wv[i % 2][0] = lut4(cd[i % 2][0]);
                wv[i % 2][1] = lut4(cd[i % 2][1]);
                scv[i % 4] = __int_as_float(
                    __builtin_amdgcn_ds_bpermute((n16 + 16 * (t % 4)) * 4, __float_as_int(sq[t / 4][b])));
            }
            if (it < NI) {  // A(it)
                const int i = it;
                const uint2 c = cw[i % D];
                if (i + D < NI) cw[i % D] = load_code(i + D);
                cd[i % 2][0] = (uint32_t)__builtin_amdgcn_ds_bpermute(code_src, (int)c.x);
                cd[i % 2][1] = (uint32_t)__builtin_amdgcn_ds_bpermute(code_src, (int)c.y);
            }
        }
    }

    // ---- cross-wave sums (fixed order) --------------------------------------
    // the group counter: read here (after the last load the waves wait on), used
    // after the partials are out; a fresh workspace gets it tagged
    unsigned long long ctr0 = 0;
    if (S > 1 && tid == 0) ctr0 = __hip_atomic_load(p.ctr + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int t = 0; t < TW; ++t) red[wave][t][lane] = acc[t];
    if (u_wave) ured[kpart][lane] = uacc;
    __syncthreads();
    f32x4 ysum[NTT];
#pragma unroll
    for (int h = 0; h < NTT; ++h) {
        const int tt = wave + DEC_WAVES * h;
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tt < T) {
            const int ts = tt / TW, t = tt % TW;
            for (int q = 0; q < P; ++q) a += red[ts * P + q][t][lane];
        }
        ysum[h] = a;
    }
    f32x4 usum = f32x4{0.f, 0.f, 0.f, 0.f};
    if (fuse_u && wave == 0)
        for (int q = 0; q < P; ++q) usum += ured[q][lane];

    if (S > 1) {
        // publish this slice's partials (slots [wg][tt][lane], then U at [wg][T][lane]);
        // the last workgroup of the group to arrive adds all S in slice order
#pragma unroll
        for (int h = 0; h < NTT; ++h) {
            const int tt = wave + DEC_WAVES * h;
            if (tt < T) store16_sc1(rp, (uint32_t)((((int64_t)wg * (T + 1) + tt) * 64 + lane) * 16), ysum[h]);
        }
        if (fuse_u && wave == 0) store16_sc1(rp, (uint32_t)((((int64_t)wg * (T + 1) + T) * 64 + lane) * 16), usum);
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
        if (!last_flag) return;
        f32x4 pv[NTT][8];
#pragma unroll
        for (int h = 0; h < NTT; ++h) {
            const int tt = wave + DEC_WAVES * h;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                pv[h][q] = q < S && tt < T
                               ? load16_sc1(rp, (uint32_t)((((int64_t)(grp * S + q) * (T + 1) + tt) * 64 + lane) * 16))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 uv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            uv[q] = fuse_u && wave == 0 && q < S
                        ? load16_sc1(rp, (uint32_t)((((int64_t)(grp * S + q) * (T + 1) + T) * 64 + lane) * 16))
                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < NTT; ++h) {
            f32x4 a = pv[h][0];
#pragma unroll
            for (int q = 1; q < 8; ++q)
                if (q < S) a += pv[h][q];
            ysum[h] = a;
        }
        f32x4 a = uv[0];
#pragma unroll
        for (int q = 1; q < 8; ++q)
            if (q < S) a += uv[q];
        usum = a;
    }

    // ---- adapter term and bf16 store ------------------------------------------
    if (fuse_u && wave == 0) {
        // lane (j, g) holds U[4 g + v][j]
#pragma unroll
        for (int v = 0; v < 4; ++v) us[4 * g + v][n16] = usum[v];
        if (p.u_save && grp == 0 && n16 < r) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (4 * g + v < M) p.u_save[(4 * g + v) * r + n16] = usum[v];
        }
    }
    __syncthreads();
    // U B^T by MFMA over 32-wide slices of j: U split into bf16 hi + lo, lane
    // (m, g) holds U[m][32 it + 8 g .. + 7], lane (n, g) holds B[n][same j]
    f32x4 ad[NTT];
#pragma unroll
    for (int h = 0; h < NTT; ++h) ad[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nj = (r + 31) / 32;
    for (int it = 0; it < nj; ++it) {
        const int j0 = 32 * it + 8 * g;
        uint4 uhi{0, 0, 0, 0}, ulo{0, 0, 0, 0};
        if (j0 < r) {
            const f32x4 u0 = *reinterpret_cast<const f32x4 *>(&us[n16][j0]);
            const f32x4 u1 = *reinterpret_cast<const f32x4 *>(&us[n16][j0 + 4]);
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
#pragma unroll
        for (int h = 0; h < NTT; ++h) {
            const int tt = wave + DEC_WAVES * h;
            if (tt >= T) continue;
            const uint4 bf = it == 0 ? bfr[h] : load_bfrag(rb, row_g + 16 * tt + n16, j0, r, true);
            ad[h] = mfma16(uhi, bf, ad[h]);
            ad[h] = mfma16(ulo, bf, ad[h]);
        }
    }
    // all loads are done: the stores below never wait on each other
#pragma unroll
    for (int h = 0; h < NTT; ++h) {
        const int tt = wave + DEC_WAVES * h;
        const int row = row_g + 16 * tt + n16;
        if (tt >= T || row >= d) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * g + v;
            if (m >= M) continue;
            const float out = ysum[h][v] + p.s * ad[h][v];
            p.y[(int64_t)m * d + row] = (uint16_t)(pack_bf16x2(out, 0.0f) & 0xFFFFu);
        }
    }
}

struct DecodePlan {
    int S, T, TW, P, nbw, groups, grid;
};

DecodePlan decode_plan(int64_t d, int64_t k) {
    const int64_t kb = k / 64, ntiles = (d + 15) / 16;
    DecodePlan pl;
    pl.P = 4;  // two tile subsets of four k-ranges each
    const int ts = DEC_WAVES / pl.P;
    int64_t S = (kb + pl.P * DEC_KB - 1) / (pl.P * DEC_KB);  // one chunk per wave
    if (S > 8) S = 8;
    pl.S = (int)S;
    pl.nbw = (int)((kb + S * pl.P - 1) / (S * pl.P));
    // about one workgroup per compute unit
    const int64_t t_need = (ntiles * S + 255) / 256;
    int64_t tw = (t_need + ts - 1) / ts;
    tw = tw < 1 ? 1 : (tw > DEC_MAX_TW ? DEC_MAX_TW : tw);
    pl.TW = (int)tw;
    pl.T = ts * pl.TW;
    pl.groups = (int)((ntiles + pl.T - 1) / pl.T);
    if (pl.S > 1 && pl.groups > DEC_MAX_GROUPS) {  // too many counters: one slice
        pl.S = 1;
        pl.nbw = (int)((kb + pl.P - 1) / pl.P);
    }
    pl.grid = pl.groups * pl.S;
    return pl;
}

template <int TW>
hipError_t launch_tw(const DecodeArgs &a, int mv, int grid, hipStream_t st) {
    if (mv == 1) hipLaunchKernelGGL((nf4_decode_kernel<TW, 1>), dim3(grid), dim3(DEC_THREADS), 0, st, a, nf4_consts());
    else hipLaunchKernelGGL((nf4_decode_kernel<TW, 4>), dim3(grid), dim3(DEC_THREADS), 0, st, a, nf4_consts());
    return hipGetLastError();
}

}  // namespace

size_t decode_counter_bytes() { return sizeof(unsigned long long) * DEC_MAX_GROUPS; }

size_t decode_part_bytes(int64_t M, int64_t d, int64_t k) {
    if (M < 1 || M > 16) return 0;
    const DecodePlan pl = decode_plan(d, k);
    if (pl.S == 1) return 0;
    return sizeof(f32x4) * (size_t)pl.grid * 64 * ((size_t)pl.T + 1);
}

hipError_t launch_decode_fwd(const Nf4Weights &w, const uint16_t *x, int64_t M, const uint16_t *A, const float *U,
                             const uint16_t *B, int r, float s, uint16_t *Y, float *U_save, float *part,
                             unsigned long long *ctr, hipStream_t st) {
    if (M < 1 || M > 16 || (!U && (!A || r > 16)) || w.k > (int64_t(1) << 25)) return hipErrorInvalidValue;
    const DecodePlan pl = decode_plan(w.d, w.k);
    if (pl.S > 1 && (!part || !ctr)) return hipErrorInvalidValue;
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
    a.grid_ = pl.grid;
    a.ctr = ctr;
    a.S = pl.S;
    a.T = pl.T;
    a.P = pl.P;
    a.nbw = pl.nbw;
    const int mv = M == 1 ? 1 : 4;
    switch (pl.TW) {
        case 1: return launch_tw<1>(a, mv, pl.grid, st);
        case 2: return launch_tw<2>(a, mv, pl.grid, st);
        case 3: return launch_tw<3>(a, mv, pl.grid, st);
        case 4: return launch_tw<4>(a, mv, pl.grid, st);
        case 5: return launch_tw<5>(a, mv, pl.grid, st);
        case 6: return launch_tw<6>(a, mv, pl.grid, st);
        case 7: return launch_tw<7>(a, mv, pl.grid, st);
        default: return launch_tw<8>(a, mv, pl.grid, st);
    }
}

}  // namespace qnf4
