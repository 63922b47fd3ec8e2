// The C ABI (include/qlora_nf4.h): argument validation, workspace layout and
// the launch sequence of each call.  No allocation, no synchronisation, no
// global mutable state; every check runs before the first launch.
#include "qlora_nf4.h"

#include <cmath>
#include <cstring>
#include <mutex>

#include "launch.hpp"

using namespace qnf4;

namespace {

constexpr int64_t kMaxWeights = int64_t(1) << 30;  // 2^24 NF4 blocks: 65536 DQ groups
constexpr int64_t kDecodeMaxK = int64_t(1) << 25;  // 32-bit buffer offsets of X and A rows
constexpr int64_t kMaxDim = int64_t(1) << 20;      // d, k of a linear call: 32-bit offsets in GEMM tiles
constexpr int64_t kMaxPlanes = int64_t(1) << 29;   // M * r16: U and G as transposed bf16 hi / lo planes

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape and format checks shared by every call that takes a weight.
int check_weight(const qlora_nf4_weight *w, bool need_data) {
    if (!w) return QLORA_EINVAL;
    if (w->d <= 0 || w->k <= 0) return QLORA_EINVAL;
    if (w->block != 64 && w->block != 128 && w->block != 256) return QLORA_ENOTSUP;
    if (w->dq_block != QLORA_NF4_DQ_BLOCK && w->dq_block != QLORA_NF4_NO_DQ) return QLORA_ENOTSUP;
    if (w->c2_format != QLORA_C2_INT8 && w->c2_format != QLORA_C2_FP8_E4M3) return QLORA_ENOTSUP;
    if (w->k % w->block != 0) return QLORA_EINVAL;
    if (w->d > kMaxWeights / w->k) return QLORA_ENOTSUP;
    if (need_data) {
        const bool dq = w->dq_block != QLORA_NF4_NO_DQ;
        if (!w->codes || !w->absmax_scale) return QLORA_EINVAL;
        if (dq && (!w->absmax_q || !w->absmax_mean)) return QLORA_EINVAL;
        if (!aligned(w->codes, 16) || !aligned(w->absmax_scale, 4) || (dq && !aligned(w->absmax_mean, 4)))
            return QLORA_EALIGN;
    }
    return QLORA_OK;
}

// The kernels' view of a checked weight.
Nf4Weights nf4_view(const qlora_nf4_weight *w) {
    const bool dq = w->dq_block != QLORA_NF4_NO_DQ;
    const int fmt = !dq ? kNoDq : w->c2_format == QLORA_C2_FP8_E4M3 ? kDqFp8 : kDqInt8;
    const int bshift = w->block == 256 ? 2 : w->block == 128 ? 1 : 0;
    return Nf4Weights{w->codes, dq ? w->absmax_q : nullptr, w->absmax_scale, dq ? w->absmax_mean : nullptr,
                      w->d, w->k, fmt, bshift};
}

int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_EHIP; }

// ---- workspace layouts ------------------------------------------------------
struct QuantWs {
    size_t absmax, group_sum, total;
};
QuantWs quant_ws(int64_t d, int64_t k, int block) {
    const int64_t nb = d * k / block;
    const int64_t g = (nb + QLORA_NF4_DQ_BLOCK - 1) / QLORA_NF4_DQ_BLOCK;
    QuantWs q;
    q.absmax = 0;
    q.group_sum = round_up(sizeof(float) * nb, 256);
    q.total = q.group_sum + round_up(sizeof(double) * g, 256);
    return q;
}

struct LinWs {
    size_t ctr, dpart, shat, ext_a, ext_b, wbf, kpart, kpart_bytes, u, bt, g, vt, part, total;
};
// The decode counters sit first, at the same offset for every shape, so that no
// other call's data ever lands on them.
LinWs lin_ws(int64_t M, int64_t d, int64_t k, int r) {
    LinWs l;
    size_t off = 0;
    l.ctr = off;
    off += round_up(decode_counter_bytes(), 256);
    l.dpart = off;
    off += round_up(decode_part_bytes(M, d, k), 256);
    l.shat = off;
    off += round_up(sizeof(float) * (d * k / QLORA_NF4_BLOCK), 256);
    const int64_t ke = gemm_ext_cols(r);
    l.ext_a = off;
    off += round_up(sizeof(uint16_t) * M * ke, 256);
    l.ext_b = off;
    off += round_up(sizeof(uint16_t) * (d > k ? d : k) * ke, 256);
    l.wbf = off;
    off += round_up(sizeof(uint16_t) * gemm_wbf_elems(M, d, k), 256);
    l.kpart = off;  // the GEMMs' split-K partial sums
    l.kpart_bytes = gemm_ksplit_bytes(M, d, k);
    off += round_up(l.kpart_bytes, 256);
    l.u = off;
    off += round_up(sizeof(float) * M * r, 256);
    l.bt = off;
    off += round_up(sizeof(uint16_t) * d * r, 256);
    l.g = off;
    off += round_up(sizeof(float) * M * r, 256);
    l.vt = off;  // transposed hi / lo planes of U and of G
    off += round_up(sizeof(uint16_t) * 2 * 2 * cols_rank_pad(r) * M, 256);
    l.part = off;  // the column reductions' partials, or (before them) the wide-rank row products
    size_t part_bytes = sizeof(float) * cols_splits(M) * (size_t)r * (round_up(d, 64) + k);
    const size_t rows_k = rows_split_part_bytes(M, k, r), rows_d = rows_split_part_bytes(M, d, r);
    part_bytes = part_bytes > rows_k ? part_bytes : rows_k;
    part_bytes = part_bytes > rows_d ? part_bytes : rows_d;
    off += round_up(part_bytes, 256);
    l.total = off;
    return l;
}

GemmWs gemm_ws(char *base, const LinWs &l) {
    return GemmWs{reinterpret_cast<float *>(base + l.shat), reinterpret_cast<uint16_t *>(base + l.ext_a),
                  reinterpret_cast<uint16_t *>(base + l.ext_b), reinterpret_cast<uint16_t *>(base + l.wbf),
                  reinterpret_cast<float *>(base + l.kpart), l.kpart_bytes};
}

// Dropout parameters: the keep threshold floor(p 2^32) (exact in fp64; below 2^32
// for p < 1) and c = fp32(1 / fp32(1 - p)).
bool dropout_params(float p, uint32_t *thr, float *c) {
    if (!(p >= 0.0f && p < 1.0f)) return false;  // also rejects NaN
    *thr = (uint32_t)std::floor((double)p * 4294967296.0);
    *c = 1.0f / (1.0f - p);
    return true;
}

// Shapes the linear calls support.  The kernels address each operand (or
// each tile of one) through buffer resources with 32-bit byte offsets:
// d, k <= 2^20; M k (X, dX), M d (Y, dY) and d k (W0) <= 2^30 elements; and
// M r16 <= 2^29 (r16 = r rounded up to 16) for the bf16 planes of U and G.
bool linear_shape_ok(int64_t M, int64_t d, int64_t k, int32_t r) {
    if (d > kMaxDim || k > kMaxDim || d > kMaxWeights / k) return false;
    if (M > kMaxWeights / k || M > kMaxWeights / d) return false;
    return M <= kMaxPlanes / cols_rank_pad(r);
}

// ---- the static scratch of qlora_linear_fwd_noalloc ----------------------------
// Device memory of the allocation-free forward: the decode kernel's counters,
// its partial sums and, for r > 16, U.  One array per GPU (a __device__ object
// exists on every device the library runs on), held until the process ends.
// In host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call there).
int scratch_of_current_device(void **addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_EHIP;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return QLORA_OK;
}

// Device memory the decode-shaped forward (M <= 16) needs beside its inputs and
// outputs: counters, partial sums and (r > 16) U.
struct DecodeWs {
    size_t ctr, dpart, u, total;
};
DecodeWs decode_ws(int64_t M, int64_t d, int64_t k, int r) {
    DecodeWs l;
    l.ctr = 0;
    l.dpart = round_up(decode_counter_bytes(), 256);
    l.u = l.dpart + round_up(decode_part_bytes(M, d, k), 256);
    l.total = l.u + round_up(sizeof(float) * M * r, 256);
    return l;
}

// The decode-shaped forward: one kernel (U = X A^T fused for r <= 16), or U by
// the skinny kernel first (into U_save, else u_buf) for r > 16.
hipError_t decode_forward(const Nf4Weights &nw, const qlora_bf16 *x, int64_t M, const qlora_bf16 *A,
                          const qlora_bf16 *B, int32_t r, float scale, qlora_bf16 *Y, float *U_save,
                          unsigned long long *ctr, float *dpart, float *u_buf, hipStream_t s) {
    if (r <= 16) return launch_decode_fwd(nw, x, M, A, nullptr, B, r, scale, Y, U_save, dpart, ctr, s);
    float *U = U_save ? U_save : u_buf;
    hipError_t e = launch_rows_skinny(x, A, M, nw.k, r, U, nullptr, nullptr, s);  // M <= 16: no partials
    if (e == hipSuccess) e = launch_decode_fwd(nw, x, M, nullptr, U, B, r, scale, Y, nullptr, dpart, ctr, s);
    return e;
}

int check_linear(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M, const qlora_bf16 *A,
                 const qlora_bf16 *B, int32_t r, float alpha) {
    int st = check_weight(w, true);
    if (st != QLORA_OK) return st;
    if (!x || !A || !B) return QLORA_EINVAL;
    if (M <= 0 || r <= 0) return QLORA_EINVAL;
    if (!std::isfinite(alpha)) return QLORA_EINVAL;
    if (r > QLORA_MAX_RANK) return QLORA_ENOTSUP;
    if (w->d % 8 != 0) return QLORA_ENOTSUP;  // bf16 rows of [M x d] must be 16-byte aligned
    if (!linear_shape_ok(M, w->d, w->k, r)) return QLORA_ENOTSUP;
    if (!aligned(x, 16) || !aligned(A, 16) || !aligned(B, 2)) return QLORA_EALIGN;
    return QLORA_OK;
}

}  // namespace

// ---- the measurement hook (qlora_time_next_kernel) ----------------------------
namespace {
std::mutex g_time_mu;
unsigned long long *g_time_span[kTimedKernels];
}  // namespace

unsigned long long *qnf4::timing_take(int kernel) {
    std::lock_guard<std::mutex> lock(g_time_mu);
    unsigned long long *sp = g_time_span[kernel];
    g_time_span[kernel] = nullptr;
    return sp;
}

extern "C" {

int qlora_abi_version(void) { return QLORA_ABI_VERSION; }

const char *qlora_status_str(int status) {
    switch (status) {
        case QLORA_OK: return "QLORA_OK: success";
        case QLORA_EINVAL: return "QLORA_EINVAL: invalid argument (null pointer, size <= 0, k % block != 0, non-finite alpha)";
        case QLORA_ENOTSUP: return "QLORA_ENOTSUP: unsupported configuration (block not 64, 128 or 256, dq_block not 256 or 0, unknown c2_format, r > 128, d % 8 != 0, tensor too large)";
        case QLORA_EALIGN: return "QLORA_EALIGN: misaligned pointer (16-byte alignment required)";
        case QLORA_EWORKSPACE: return "QLORA_EWORKSPACE: workspace missing or too small";
        case QLORA_EHIP: return "QLORA_EHIP: HIP launch or runtime error";
        case QLORA_ESCRATCH: return "QLORA_ESCRATCH: the allocation-free call takes M <= 16 and sizes whose scratch fits the library's static 8 MiB";
        default: return "unknown qlora status";
    }
}

int qlora_nf4_codebook(float out[16]) {
    if (!out) return QLORA_EINVAL;
    std::memcpy(out, nf4_consts().level, sizeof(float) * 16);
    return QLORA_OK;
}

int qlora_nf4_thresholds(float out[15]) {
    if (!out) return QLORA_EINVAL;
    std::memcpy(out, nf4_consts().thresh, sizeof(float) * 15);
    return QLORA_OK;
}

size_t qlora_nf4_quantize_workspace(int64_t d, int64_t k, int32_t block, int32_t dq_block) {
    qlora_nf4_weight w{};
    w.d = d;
    w.k = k;
    w.block = block;
    w.dq_block = dq_block;
    if (check_weight(&w, false) != QLORA_OK) return 0;
    return quant_ws(d, k, block).total;
}

int qlora_nf4_quantize(const float *W0, const qlora_nf4_weight *w, void *ws, size_t ws_bytes,
                       void *stream) {
    int st = check_weight(w, true);
    if (st != QLORA_OK) return st;
    if (!W0) return QLORA_EINVAL;
    if (!aligned(W0, 16)) return QLORA_EALIGN;
    const QuantWs q = quant_ws(w->d, w->k, w->block);
    if (!ws || ws_bytes < q.total) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    char *base = static_cast<char *>(ws);
    const bool dq = w->dq_block != QLORA_NF4_NO_DQ;
    return hip_status(launch_quantize(W0, w->d * w->k, w->block, w->codes, dq ? w->absmax_q : nullptr, w->absmax_scale,
                                      dq ? w->absmax_mean : nullptr, reinterpret_cast<float *>(base + q.absmax),
                                      reinterpret_cast<double *>(base + q.group_sum), nf4_view(w).fmt,
                                      static_cast<hipStream_t>(stream)));
}

int qlora_nf4_dequantize(const qlora_nf4_weight *w, qlora_bf16 *W_out, void *stream) {
    int st = check_weight(w, true);
    if (st != QLORA_OK) return st;
    if (!W_out) return QLORA_EINVAL;
    if (!aligned(W_out, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    const Nf4Weights nw = nf4_view(w);
    return hip_status(launch_dequantize(nw.codes, nw.c2, nw.c1, nw.mean, nw.fmt, nw.bshift, w->d * w->k, W_out,
                                        static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_workspace(int64_t M, int64_t d, int64_t k, int32_t r) {
    if (M <= 0 || d <= 0 || k <= 0 || r <= 0 || r > QLORA_MAX_RANK) return 0;
    if (k % QLORA_NF4_BLOCK != 0 || !linear_shape_ok(M, d, k, r)) return 0;
    return lin_ws(M, d, k, r).total;
}

int qlora_linear_fwd(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M,
                     const qlora_bf16 *A, const qlora_bf16 *B, int32_t r, float alpha,
                     qlora_bf16 *Y, float *U_save, void *ws, size_t ws_bytes, void *stream) {
    int st = check_linear(w, x, M, A, B, r, alpha);
    if (st != QLORA_OK) return st;
    if (!Y) return QLORA_EINVAL;
    if (!aligned(Y, 16) || (U_save && !aligned(U_save, 4))) return QLORA_EALIGN;
    const LinWs l = lin_ws(M, w->d, w->k, r);
    if (!ws || ws_bytes < l.total) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    char *base = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = alpha / static_cast<float>(r);
    float *U = U_save ? U_save : reinterpret_cast<float *>(base + l.u);
    const Nf4Weights nw = nf4_view(w);
    float *dpart = reinterpret_cast<float *>(base + l.dpart);
    unsigned long long *ctr = reinterpret_cast<unsigned long long *>(base + l.ctr);
    hipError_t e = hipSuccess;
    if (M <= kDecodeChunkRows && w->k <= kDecodeMaxK) {
        // HBM-bound: one pass over the codes per 16-row chunk of X; U = X A^T in the
        // same kernel for r <= 16
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += 16) {
            const int64_t mc = M - m0 < 16 ? M - m0 : 16;
            e = decode_forward(nw, x + m0 * w->k, mc, A, B, r, scale, Y + m0 * w->d, U_save ? U_save + m0 * r : nullptr,
                               ctr, dpart, U + m0 * r, s);
        }
    } else {
        float *part = reinterpret_cast<float *>(base + l.part);
        if (rows_split_partials_used(M, r)) {  // U's partials, added by the GEMM's preparation launch
            int S = 0;
            e = launch_rows_split_partials(x, A, M, w->k, r, part, &S, s);
            if (e == hipSuccess) e = launch_gemm_fwd(nw, x, M, nullptr, B, r, scale, Y, gemm_ws(base, l), s, part, S, U);
        } else {
            e = launch_rows_skinny(x, A, M, w->k, r, U, nullptr, part, s);
            if (e == hipSuccess) e = launch_gemm_fwd(nw, x, M, U, B, r, scale, Y, gemm_ws(base, l), s);
        }
    }
    return hip_status(e);
}

int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *Y, float *U_save,
                             void *stream) {
    int st = check_linear(w, x, M, A, B, r, alpha);
    if (st != QLORA_OK) return st;
    if (!Y) return QLORA_EINVAL;
    if (!aligned(Y, 16) || (U_save && !aligned(U_save, 4))) return QLORA_EALIGN;
    if (M > 16 || w->k > kDecodeMaxK) return QLORA_ESCRATCH;
    const DecodeWs l = decode_ws(M, w->d, w->k, r);
    if (l.total > kNoAllocScratchBytes) return QLORA_ESCRATCH;
    void *addr = nullptr;
    st = scratch_of_current_device(&addr);
    if (st != QLORA_OK) return st;
    (void)hipGetLastError();
    char *base = static_cast<char *>(addr);
    const float scale = alpha / static_cast<float>(r);
    return hip_status(decode_forward(nf4_view(w), x, M, A, B, r, scale, Y, U_save,
                                     reinterpret_cast<unsigned long long *>(base + l.ctr),
                                     reinterpret_cast<float *>(base + l.dpart), reinterpret_cast<float *>(base + l.u),
                                     static_cast<hipStream_t>(stream)));
}

int qlora_linear_bwd(const qlora_nf4_weight *w, const qlora_bf16 *x, const qlora_bf16 *dY,
                     const qlora_bf16 *A, const qlora_bf16 *B, const float *U, int64_t M,
                     int32_t r, float alpha, qlora_bf16 *dX, float *dA, float *dB, void *ws,
                     size_t ws_bytes, void *stream) {
    int st = check_linear(w, x, M, A, B, r, alpha);
    if (st != QLORA_OK) return st;
    if (!dY || !dA || !dB) return QLORA_EINVAL;
    if (!aligned(dY, 16) || (dX && !aligned(dX, 16)) || !aligned(dA, 4) || !aligned(dB, 4) ||
        (U && !aligned(U, 4)))
        return QLORA_EALIGN;
    const LinWs l = lin_ws(M, w->d, w->k, r);
    if (!ws || ws_bytes < l.total) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    char *base = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = alpha / static_cast<float>(r);
    const int64_t d = w->d, k = w->k;
    float *Uw = reinterpret_cast<float *>(base + l.u);
    uint16_t *Bt = reinterpret_cast<uint16_t *>(base + l.bt);
    float *G = reinterpret_cast<float *>(base + l.g);
    float *part = reinterpret_cast<float *>(base + l.part);
    const Nf4Weights nw = nf4_view(w);

    uint16_t *vt_u = reinterpret_cast<uint16_t *>(base + l.vt);
    uint16_t *vt_g = vt_u + 2 * cols_rank_pad(r) * M;
    hipError_t e = hipSuccess;
    const float *Uin = U;
    if (!Uin) {  // recompute U = X A^T, with its transposed planes
        e = launch_rows_skinny(x, A, M, k, r, Uw, vt_u, part, s);
        Uin = Uw;
    }
    if (rows_bt_supported(M, r, B)) {                                           // G = dY B (and U's planes)
        if (e == hipSuccess) e = launch_rows_bt(dY, B, M, d, r, G, vt_g, U, vt_u, s);
    } else {
        if (e == hipSuccess) e = launch_bwd_prep(B, d, r, Bt, U, M, vt_u, s);    // B^T [r x d] (and U's planes)
        if (e == hipSuccess) e = launch_rows_skinny(dY, Bt, M, d, r, G, vt_g, part, s);  // G = dY B
    }
    ColsReduceJob red[2];
    float *part_b = part;                                                       // dB = s U^T dY (as [d x r])
    float *part_a = part + (size_t)cols_splits(M) * r * round_up(d, 64);        // dA = s G^T X
    if (e == hipSuccess)
        e = launch_cols_pair(dY, vt_u, d, scale, part_b, dB, 0, x, vt_g, k, scale, part_a, dA, 1, M, r, red, s);
    if (e == hipSuccess && dX)                                                  // dX = dY What + s G A
        e = launch_gemm_dx(nw, dY, M, G, A, r, scale, dX, gemm_ws(base, l), red, s);
    else if (e == hipSuccess)
        e = launch_cols_reduce(red, s);
    return hip_status(e);
}

int qlora_adapter_merge(const qlora_nf4_weight *w, const qlora_bf16 *A, const qlora_bf16 *B, int32_t r,
                        float alpha, qlora_bf16 *W_out, void *stream) {
    int st = check_weight(w, true);
    if (st != QLORA_OK) return st;
    if (!A || !B || !W_out || r <= 0 || !std::isfinite(alpha)) return QLORA_EINVAL;
    if (r > QLORA_MAX_RANK) return QLORA_ENOTSUP;
    if (!aligned(A, 16) || !aligned(B, 2) || !aligned(W_out, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    const Nf4Weights nw = nf4_view(w);
    const float scale = alpha / static_cast<float>(r);
    return hip_status(launch_adapter_merge(&nw, nullptr, w->d, w->k, A, B, r, (double)scale, W_out,
                                           static_cast<hipStream_t>(stream)));
}

int qlora_adapter_unmerge(const qlora_bf16 *W_in, int64_t d, int64_t k, const qlora_bf16 *A, const qlora_bf16 *B,
                          int32_t r, float alpha, qlora_bf16 *W_out, void *stream) {
    if (!W_in || !A || !B || !W_out || d <= 0 || k <= 0 || r <= 0 || !std::isfinite(alpha)) return QLORA_EINVAL;
    if (k % 8 != 0) return QLORA_EINVAL;
    if (r > QLORA_MAX_RANK || d > kMaxWeights / k) return QLORA_ENOTSUP;
    if (!aligned(W_in, 16) || !aligned(A, 16) || !aligned(B, 2) || !aligned(W_out, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    const float scale = alpha / static_cast<float>(r);
    return hip_status(launch_adapter_merge(nullptr, W_in, d, k, A, B, r, -(double)scale, W_out,
                                           static_cast<hipStream_t>(stream)));
}

int qlora_lora_dropout(const qlora_bf16 *x, int64_t M, int64_t k, float p, uint64_t seed, qlora_bf16 *xd,
                       void *stream) {
    uint32_t thr;
    float c;
    if (!x || !xd || M <= 0 || k <= 0 || k % 8 != 0 || !dropout_params(p, &thr, &c)) return QLORA_EINVAL;
    if (M > kMaxWeights / k) return QLORA_ENOTSUP;
    if (!aligned(x, 16) || !aligned(xd, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    return hip_status(launch_lora_dropout(x, M, k, thr, c, seed, xd, static_cast<hipStream_t>(stream)));
}

// A linear workspace, then Xd [M x k] bf16, then the dX GEMM's fp32 sums [M x k].
size_t qlora_linear_dropout_workspace(int64_t M, int64_t d, int64_t k, int32_t r) {
    const size_t base = qlora_linear_workspace(M, d, k, r);
    if (base == 0) return 0;
    return base + round_up(sizeof(uint16_t) * M * k, 256) + round_up(sizeof(float) * M * k, 256);
}

int qlora_linear_fwd_dropout(const qlora_nf4_weight *w, const qlora_bf16 *x, int64_t M, const qlora_bf16 *A,
                             const qlora_bf16 *B, int32_t r, float alpha, float p, uint64_t seed, qlora_bf16 *Y,
                             float *U_save, void *ws, size_t ws_bytes, void *stream) {
    int st = check_linear(w, x, M, A, B, r, alpha);
    if (st != QLORA_OK) return st;
    uint32_t thr;
    float c;
    if (!Y || !dropout_params(p, &thr, &c)) return QLORA_EINVAL;
    if (!aligned(Y, 16) || (U_save && !aligned(U_save, 4))) return QLORA_EALIGN;
    const LinWs l = lin_ws(M, w->d, w->k, r);
    if (!ws || ws_bytes < qlora_linear_dropout_workspace(M, w->d, w->k, r)) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    char *base = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = alpha / static_cast<float>(r);
    uint16_t *xd = reinterpret_cast<uint16_t *>(base + l.total);
    float *U = U_save ? U_save : reinterpret_cast<float *>(base + l.u);
    const Nf4Weights nw = nf4_view(w);
    hipError_t e = launch_lora_dropout(x, M, w->k, thr, c, seed, xd, s);
    if (e == hipSuccess)  // U = Xd A^T
        e = launch_rows_skinny(xd, A, M, w->k, r, U, nullptr, reinterpret_cast<float *>(base + l.part), s);
    if (e == hipSuccess) {
        if (M <= 16 && w->k <= kDecodeMaxK)
            e = launch_decode_fwd(nw, x, M, nullptr, U, B, r, scale, Y, nullptr, reinterpret_cast<float *>(base + l.dpart),
                                  reinterpret_cast<unsigned long long *>(base + l.ctr), s);
        else
            e = launch_gemm_fwd(nw, x, M, U, B, r, scale, Y, gemm_ws(base, l), s);
    }
    return hip_status(e);
}

int qlora_linear_bwd_dropout(const qlora_nf4_weight *w, const qlora_bf16 *x, const qlora_bf16 *dY,
                             const qlora_bf16 *A, const qlora_bf16 *B, const float *U, int64_t M, int32_t r,
                             float alpha, float p, uint64_t seed, qlora_bf16 *dX, float *dA, float *dB, void *ws,
                             size_t ws_bytes, void *stream) {
    int st = check_linear(w, x, M, A, B, r, alpha);
    if (st != QLORA_OK) return st;
    uint32_t thr;
    float c;
    if (!dY || !dA || !dB || !dropout_params(p, &thr, &c)) return QLORA_EINVAL;
    if (!aligned(dY, 16) || (dX && !aligned(dX, 16)) || !aligned(dA, 4) || !aligned(dB, 4) ||
        (U && !aligned(U, 4)))
        return QLORA_EALIGN;
    const LinWs l = lin_ws(M, w->d, w->k, r);
    if (!ws || ws_bytes < qlora_linear_dropout_workspace(M, w->d, w->k, r)) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    char *base = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = alpha / static_cast<float>(r);
    const int64_t d = w->d, k = w->k;
    uint16_t *xd = reinterpret_cast<uint16_t *>(base + l.total);
    float *Uw = reinterpret_cast<float *>(base + l.u);
    uint16_t *Bt = reinterpret_cast<uint16_t *>(base + l.bt);
    float *G = reinterpret_cast<float *>(base + l.g);
    float *part = reinterpret_cast<float *>(base + l.part);
    const Nf4Weights nw = nf4_view(w);
    uint16_t *vt_u = reinterpret_cast<uint16_t *>(base + l.vt);
    uint16_t *vt_g = vt_u + 2 * cols_rank_pad(r) * M;
    hipError_t e = launch_lora_dropout(x, M, k, thr, c, seed, xd, s);           // the forward's Xd again
    if (e == hipSuccess && !U) e = launch_rows_skinny(xd, A, M, k, r, Uw, vt_u, part, s);
    if (rows_bt_supported(M, r, B)) {                                            // G = dY B (and U's planes)
        if (e == hipSuccess) e = launch_rows_bt(dY, B, M, d, r, G, vt_g, U, vt_u, s);
    } else {
        if (e == hipSuccess) e = launch_bwd_prep(B, d, r, Bt, U, M, vt_u, s);
        if (e == hipSuccess) e = launch_rows_skinny(dY, Bt, M, d, r, G, vt_g, part, s);   // G = dY B
    }
    ColsReduceJob red[2];
    float *part_b = part;                                                       // dB = s U^T dY
    float *part_a = part + (size_t)cols_splits(M) * r * round_up(d, 64);        // dA = s G^T Xd
    if (e == hipSuccess)
        e = launch_cols_pair(dY, vt_u, d, scale, part_b, dB, 0, xd, vt_g, k, scale, part_a, dA, 1, M, r, red, s);
    if (e == hipSuccess && dX) {
        // the base term dY What in fp32 (the GEMM's adapter columns get scale 0), then the masked
        // adapter term added to it and the sum rounded once to bf16
        float *dx_f32 = reinterpret_cast<float *>(base + l.total + round_up(sizeof(uint16_t) * M * k, 256));
        e = launch_gemm_dx(nw, dY, M, G, A, r, 0.0f, dX, gemm_ws(base, l), red, s, dx_f32);
        if (e == hipSuccess) e = launch_dropout_dx_add(dx_f32, dX, M, k, G, r, A, scale * c, thr, seed, s);
    } else if (e == hipSuccess) {
        e = launch_cols_reduce(red, s);
    }
    return hip_status(e);
}

int qlora_linear_gemm_only(const qlora_nf4_weight *w, int32_t backward, int32_t expand, const qlora_bf16 *a,
                           int64_t M, int32_t r, qlora_bf16 *out, void *ws, size_t ws_bytes, void *stream) {
    int st = check_weight(w, true);
    if (st != QLORA_OK) return st;
    if (!a || !out || M <= 0 || r <= 0) return QLORA_EINVAL;
    if (r > QLORA_MAX_RANK || w->d % 8 != 0) return QLORA_ENOTSUP;
    if (!linear_shape_ok(M, w->d, w->k, r)) return QLORA_ENOTSUP;
    if (!aligned(a, 16) || !aligned(out, 16)) return QLORA_EALIGN;
    if (!backward && M <= kDecodeChunkRows && w->k <= kDecodeMaxK)
        return QLORA_EINVAL;  // the decode path has no separate GEMM
    const LinWs l = lin_ws(M, w->d, w->k, r);
    if (!ws || ws_bytes < l.total) return QLORA_EWORKSPACE;
    if (!aligned(ws, 16)) return QLORA_EALIGN;
    (void)hipGetLastError();
    const Nf4Weights nw = nf4_view(w);
    return hip_status(launch_gemm_core(backward != 0, nw, a, M, r, out, gemm_ws(static_cast<char *>(ws), l),
                                       static_cast<hipStream_t>(stream), expand != 0));
}

int qlora_time_next_kernel(int32_t kernel, uint64_t *span) {
    if (kernel < 0 || kernel >= kTimedKernels) return QLORA_EINVAL;
    if (span && !aligned(span, 8)) return QLORA_EALIGN;
    std::lock_guard<std::mutex> lock(g_time_mu);
    g_time_span[kernel] = reinterpret_cast<unsigned long long *>(span);
    return QLORA_OK;
}

int qlora_wall_clock_khz(int32_t *khz) {
    if (!khz) return QLORA_EINVAL;
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QLORA_EHIP;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return QLORA_EHIP;
    *khz = v;
    return QLORA_OK;
}

}  // extern "C"
