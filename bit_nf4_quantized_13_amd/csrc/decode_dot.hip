// Decode-shaped forward for M <= 2 tokens on packed bf16 dot products:
// Y = X What^T + s (X A^T) B^T, What = doubleDequant(c1, c2, W_NF4) (chkda.github.io
// "Why do we need LoRA and QLoRA?", "Double quantization and double
// dequantization"), one kernel that streams the packed weights once.
//
// With one or two token rows a 16-row matrix-core tile would be almost empty,
// so this kernel works on the vector ALU instead:
//
// * 128 lanes share a weight row (k <= 4096); lane c owns the k-chunk c (32
//   weights), so its slice of X (32 k per token row) is loaded once into
//   registers and reused for every row the workgroup visits.  A wave
//   instruction then reads 1 KiB of contiguous code bytes (64 lanes x 16 B).
// * A code byte maps to the packed bf16 pair of its two levels through a
//   256-entry table in LDS, replicated once per lane (every lane reads its own
//   bank); one v_dot2 per byte and token row multiplies the pair with the
//   matching X pair in fp32.  The chunk's 32 products are summed first and the
//   block scale of the chunk is applied to that sum, so the level, not the
//   scaled weight, is what gets rounded to bf16 (the same product with a
//   different rounding, inside the tolerance of the bf16 What product).
// * A workgroup (16 waves) takes up to eight rounds of eight rows; the code
//   loads of the first rounds (all eight for one token row) are issued before
//   the table is built, so the workgroup's share of the weight is in flight
//   from the start.
// * Lane sums are reduced over each 16-lane row by DPP in a fixed pattern, and
//   the 8 row sums of an output (4 rows x 2 waves) are added in a fixed order
//   through LDS: results do not depend on timing.
// * U = X A^T (r <= 16) is computed by every workgroup on the same lanes: slot
//   s takes ranks s and s + 8.  The adapter term s U B^T is an fp32 dot of
//   length r per output.
#include "launch.hpp"

namespace qnf4 {
namespace {

constexpr int DD_THREADS = 1024;            // 16 waves
constexpr int DD_SLOTS = DD_THREADS / 128;  // rows per round (128 lanes per row)
constexpr int DD_RMAX = 8;                  // rounds per workgroup
constexpr uint32_t DD_OOB = 0x80000000u;    // buffer offset past every range used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dd_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 dd_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The packed codes are read once per call: loaded with the non-temporal hint
// (nt), which measured 13.0 against 14.1 us for 14336 x 4096 at M = 1 (the
// matrix-core decode kernel, whose X and A traffic shares the caches, got
// slower with it and keeps plain loads).
__device__ __forceinline__ uint4 dd_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ uint32_t u4_word(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
// Sum over the 16 lanes of a DPP row; lane 0 of the row holds it afterwards
// (the other lanes hold the same sum in another association order).
__device__ __forceinline__ float dd_row_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
    return v;
}

struct DotArgs {
    const uint8_t *codes;  // W0 [d x k] packed NF4
    const int8_t *c2;
    const float *c1;
    const float *mean;
    int d, k, bs;          // blocks of 64 << bs weights
    const uint16_t *x;     // [M x k] bf16
    int M;
    const uint16_t *A;     // [r x k] bf16
    const uint16_t *B;     // [d x r] bf16
    int r;
    float s;
    uint16_t *y;           // [M x d] bf16
    float *u_save;         // [M x r] or null
    // workgroup g has the 8-row units [g ub + min(g, ur), + ub + (g < ur)), at most DD_RMAX
    int ub, ur;
    unsigned long long *span;  // null, or a measurement span (span_start / span_end)
};

// MV token rows held in registers (M <= MV), NCH k-chunks per lane (launched with
// NCH = 1: k <= 4096 over 128 lanes), F: the ScaleFormat of the block constants.
// PD rounds of loads are in flight (8 for one token row, 4 for two).
template <int MV, int NCH, int F>
__global__ __launch_bounds__(DD_THREADS) void nf4_decode_dot_kernel(DotArgs p, Nf4Consts tab) {
    constexpr bool DQ = F != kNoDq;
    constexpr int PD = MV * NCH >= 4 ? 2 : 8 / (MV * NCH);
    __shared__ __attribute__((aligned(16))) uint32_t tbl[256 * 64];  // pair table, one copy per lane
    __shared__ float ypart[DD_RMAX][DD_SLOTS][8][MV];                  // row sums: 2 waves x 4 DPP rows
    __shared__ float upart[2][DD_SLOTS][8][MV];
    __shared__ float us[MV][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6, slot = tid >> 7, c = tid & 127;
    const int part = 4 * (wave & 1) + (lane >> 4);  // which of the 8 partial sums of a row this DPP row gives
    if (tid == 0) span_start(p.span);
    const int d = p.d, k = p.k, kb = k >> 6, hk = k >> 1, kc = k >> 5, M = p.M, r = p.r;
    const int g = blockIdx.x;
    const int u0 = g * p.ub + (g < p.ur ? g : p.ur);
    const int nu = p.ub + (g < p.ur ? 1 : 0);
    const int row0 = 8 * u0;

    // Offsets stay below 2^31 (d k / 2 code bytes, M k and r k bf16 values).
    const __amdgpu_buffer_rsrc_t rcode = dd_rsrc(p.codes, (int64_t)d * hk);
    const int64_t nblk = ((int64_t)d * kb) >> p.bs;
    const __amdgpu_buffer_rsrc_t rc2 = dd_rsrc(p.c2, DQ ? nblk : 0);
    const __amdgpu_buffer_rsrc_t rc1 = dd_rsrc(p.c1, (DQ ? (nblk + 255) / 256 : nblk) * 4);
    const __amdgpu_buffer_rsrc_t rmean = dd_rsrc(p.mean, DQ ? 4 : 0);
    const __amdgpu_buffer_rsrc_t rx = dd_rsrc(p.x, (int64_t)M * k * 2);
    const __amdgpu_buffer_rsrc_t ra = dd_rsrc(p.A, (int64_t)r * k * 2);

    // ---- loads: X and A first (they gate U), then PD rounds of codes --------
    // X slice: xv[q][m][w] = X[m][32 ch + 8 w .. + 7], ch = c + 128 q (rows past M
    // and chunks past k read zero)
    uint4 xv[NCH][MV][4];
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int ch = c + 128 * q;
#pragma unroll
        for (int m = 0; m < MV; ++m)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                xv[q][m][w] = dd_load16(rx, ch < kc ? (uint32_t)((m * k + 32 * ch) * 2 + 16 * w) : DD_OOB);
    }
    // A rows slot and slot + 8, the same k as the X slice
    uint4 av[2][NCH][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = slot + 8 * jj;
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const int ch = c + 128 * q;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                av[jj][q][w] = dd_load16(ra, j < r && ch < kc ? (uint32_t)((j * k + 32 * ch) * 2 + 16 * w) : DD_OOB);
        }
    }
    const float mean = DQ ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rmean, 0, 0, 0)) : 0.0f;
    // round i, slot s: row row0 + 8 i + s; its code chunk and block constants (the
    // chunk lies in 64-weight sub-block row kb + ch / 2 of stored block (that >> bs)).
    // Rounds past the workgroup's rows or rows past d read zero.
    uint4 cw[DD_RMAX][NCH];
    uint32_t c2b[DD_RMAX][NCH];
    float c1v[DD_RMAX][NCH];
    auto issue_round = [&](int i) __attribute__((always_inline)) {
        const int row = row0 + 8 * i + slot;
        const bool rok = i < nu && row < d;
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const int ch = c + 128 * q;
            const bool ok = rok && ch < kc;
            cw[i][q] = dd_load16_stream(rcode, ok ? (uint32_t)(row * hk + 16 * ch) : DD_OOB);
            const uint32_t blk = (uint32_t)(row * kb + (ch >> 1)) >> p.bs;
            if constexpr (DQ) {
                c2b[i][q] = __builtin_amdgcn_raw_buffer_load_b8(rc2, ok ? blk : DD_OOB, 0, 0);
                c1v[i][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc1, ok ? (blk >> 8) * 4 : DD_OOB, 0, 0));
            } else {
                c2b[i][q] = 0;
                c1v[i][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc1, ok ? blk * 4 : DD_OOB, 0, 0));
            }
        }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) issue_round(i);

    // ---- pair table: entry e = bf16(C[e & 15]) | bf16(C[e >> 4]) << 16 at dword 64 e + lane
    {
        // the levels pass through scalar registers (a plain select would become an
        // indexed load from the argument segment)
        float lvf = tab.level[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            float cj;
            asm("s_mov_b32 %0, %1" : "=s"(cj) : "s"(tab.level[j]));
            lvf = (lane & 15) == j ? cj : lvf;
        }
        const int lv = __float_as_int(lvf);
#pragma unroll
        for (int i = 0; i < 256 * 64 / 4 / DD_THREADS; ++i) {
            const int flat = tid + DD_THREADS * i;
            const int e = flat >> 4;
            const float lo = __int_as_float(__builtin_amdgcn_ds_bpermute((e & 15) << 2, lv));
            const float hi = __int_as_float(__builtin_amdgcn_ds_bpermute((e >> 4) << 2, lv));
            const uint32_t v = pack_bf16x2(lo, hi);
            reinterpret_cast<uint4 *>(tbl)[flat] = uint4{v, v, v, v};
        }
    }

    // ---- U = X A^T on the same lanes (slot s: ranks s and s + 8) ------------
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        float up[MV];
#pragma unroll
        for (int m = 0; m < MV; ++m) up[m] = 0.0f;
#pragma unroll
        for (int q = 0; q < NCH; ++q)
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int m = 0; m < MV; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) up[m] = dot2(u4_word(av[jj][q][w], e), u4_word(xv[q][m][w], e), up[m]);
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const float v = dd_row_sum(up[m]);
            if ((lane & 15) == 0) upart[jj][slot][part][m] = v;
        }
    }
    __syncthreads();  // the table is complete

    // ---- the rounds: lookups, dot products, block scales, row sums ----------
    const uint32_t lane4 = (uint32_t)lane * 4;
    const char *tbl_b = reinterpret_cast<const char *>(tbl);
#pragma unroll
    for (int i = 0; i < DD_RMAX; ++i) {
        if (i >= nu) break;
        if (i + PD < DD_RMAX) issue_round(i + PD);
        float yr[MV];
#pragma unroll
        for (int m = 0; m < MV; ++m) yr[m] = 0.0f;
        const int row = row0 + 8 * i + slot;
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            float pr[MV];
#pragma unroll
            for (int m = 0; m < MV; ++m) pr[m] = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t cd = u4_word(cw[i][q], w);  // code bytes 4 w .. 4 w + 3 of the chunk
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    // byte b -> LDS byte address (byte << 8) | (lane << 2); its two weights
                    // k = 32 ch + 8 w + 2 b, + 1 meet X dword b of xv[q][m][w]
                    const uint32_t addr = __builtin_amdgcn_perm(cd, lane4, 0x0C0C0400u + 0x100u * b);
                    const uint32_t wp = *reinterpret_cast<const uint32_t *>(tbl_b + addr);
#pragma unroll
                    for (int m = 0; m < MV; ++m) pr[m] = dot2(wp, u4_word(xv[q][m][w], b), pr[m]);
                }
            }
            const int ch = c + 128 * q;
            const bool ok = row < d && ch < kc;
            float sc;
            if constexpr (DQ) {
                // a finite quotient (c1 = 1) and scale 0 where the chunk is outside the weight
                const float c1 = ok ? c1v[i][q] : 1.0f;
                sc = dq_scale(c2_value<0>(c2b[i][q], F == kDqFp8), c1, mean) * (ok ? 1.0f : 0.0f);
            } else {
                sc = ok ? c1v[i][q] : 0.0f;
            }
#pragma unroll
            for (int m = 0; m < MV; ++m) yr[m] = __builtin_fmaf(sc, pr[m], yr[m]);
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const float v = dd_row_sum(yr[m]);
            if ((lane & 15) == 0) ypart[i][slot][part][m] = v;
        }
    }
    __syncthreads();

    // ---- U in LDS (the 8 partial sums of each entry in order) ----------------
    if (tid < 16 * MV) {
        const int m = tid >> 4, j = tid & 15;
        float u = 0.0f;
        if (m < M && j < r) {
#pragma unroll
            for (int e = 0; e < 8; ++e) u += upart[j >> 3][j & 7][e][m];
            if (p.u_save && g == 0) p.u_save[m * r + j] = u;
        }
        us[m][j] = u;
    }
    __syncthreads();

    // ---- outputs: the 8 row sums in order, the adapter term, bf16 -----------
    if (tid < 8 * DD_RMAX * MV) {
        const int rl = tid / MV, m = tid % MV;
        const int i = rl >> 3, row = row0 + rl;
        if (i < nu && row < d && m < M) {
            float ys = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ys += ypart[i][rl & 7][e][m];
            float ad = 0.0f;
            for (int j = 0; j < r; ++j) ad = __builtin_fmaf(us[m][j], bf16_bits_to_f32(p.B[(int64_t)row * r + j]), ad);
            p.y[(int64_t)m * d + row] = (uint16_t)(pack_bf16x2(ys + p.s * ad, 0.0f) & 0xFFFFu);
        }
    }
    if (p.span) {  // measurement only: every store of the workgroup is out
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) span_end(p.span);
    }
}

template <int MV, int NCH>
hipError_t launch_dd(const DotArgs &a, int fmt, int grid, hipStream_t st) {
    if (fmt == kDqInt8)
        hipLaunchKernelGGL((nf4_decode_dot_kernel<MV, NCH, kDqInt8>), dim3(grid), dim3(DD_THREADS), 0, st, a, nf4_consts());
    else if (fmt == kDqFp8)
        hipLaunchKernelGGL((nf4_decode_dot_kernel<MV, NCH, kDqFp8>), dim3(grid), dim3(DD_THREADS), 0, st, a, nf4_consts());
    else
        hipLaunchKernelGGL((nf4_decode_dot_kernel<MV, NCH, kNoDq>), dim3(grid), dim3(DD_THREADS), 0, st, a, nf4_consts());
    return hipGetLastError();
}

}  // namespace

// Chosen where it beats the matrix-core kernel (measured): one or two token
// rows and at least 32 rows per workgroup over 256 workgroups (below that the
// table, U and the A rows are paid for too few rows).
bool decode_dot_supported(int64_t M, int64_t d, int64_t k, int r) {
    return M >= 1 && M <= 2 && r >= 1 && r <= 16 && k <= 4096 && d >= 8192 && d * k <= (int64_t(1) << 31) - 2 * k;
}

hipError_t launch_decode_dot(const Nf4Weights &w, const uint16_t *x, int64_t M, const uint16_t *A, const uint16_t *B,
                             int r, float s, uint16_t *Y, float *U_save, unsigned long long *span, hipStream_t st) {
    if (!decode_dot_supported(M, w.d, w.k, r) || !A) return hipErrorInvalidValue;
    DotArgs a;
    a.codes = w.codes;
    a.c2 = w.c2;
    a.c1 = w.c1;
    a.mean = w.mean;
    a.d = (int)w.d;
    a.k = (int)w.k;
    a.bs = w.bshift;
    a.x = x;
    a.M = (int)M;
    a.A = A;
    a.B = B;
    a.r = r;
    a.s = s;
    a.y = Y;
    a.u_save = U_save;
    a.span = span;
    // 8-row units over the workgroups: at least one round of 256 workgroups when
    // there are enough units, at most DD_RMAX units each
    const int64_t units = (w.d + 7) / 8;
    int64_t G = units < 256 ? units : 256;
    if (units > 256 * DD_RMAX) G = (units + DD_RMAX - 1) / DD_RMAX;
    a.ub = (int)(units / G);
    a.ur = (int)(units % G);
    const int grid = (int)G;
    return M == 1 ? launch_dd<1, 1>(a, w.fmt, grid, st) : launch_dd<2, 1>(a, w.fmt, grid, st);
}

}  // namespace qnf4
