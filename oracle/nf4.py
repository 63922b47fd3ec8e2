"""NF4 codebook, blockwise NF4 quantization and double quantization -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Everything here follows chkda.github.io "Why do we need LoRA and QLoRA?":

  codebook           "NF4: Choose the codebook to fit the distribution" (the
                     16 printed levels) and "Building the NF4 codebook" (the
                     quantile construction; a sketch that needs a tail cutoff
                     and an exact zero -- see READINGS below).
  quantize_blocks    "Quantizing and dequantizing with the codebook": per block
                     of 64, scale = max |w|, code = index of the nearest level
                     of w/scale, ties to the smaller index, all-zero block ->
                     the exact-zero level.
  int8_absmax_*      "First, how does k-bit quantization work?": c = 127/absmax
                     (stored in fp32), q = round(c*X), Xhat = q / c; an
                     all-zero input stores zeros and a nonzero scale.
  quantize_single    the same page's bits-per-weight accounting ("before" double
  dequantize_single  quantization): one fp32 absmax per block, stored as is,
                     W[i] = BF16(C[W[i]] * absmax[i//64]).
  e4m3_*, fp8_*      the same section's c2_FP8 label, as a second c2 format
                     (reading R16).
  double_quantize    "Double quantization and double dequantization": the block
  double_dequantize  scales are quantized to 8 bits in groups of 256 with one
                     fp32 second-level scale per group, after subtracting a
                     mean; doubleDequant recovers scales[j] = dequant(c2[j],
                     c1[j // 256]) + mean and W[i] = BF16(C[W[i]] * scales[i//64]).

READINGS (where the pages are silent or loose; each is listed in the design
notes):
  R1 codebook: positive levels Q(p - i (p - 1/2)/8), i = 0..7, negative levels
     -Q(p - i (p - 1/2)/7), i = 0..6, plus an exact 0, sorted and divided by
     the largest magnitude, with Q the standard-normal inverse CDF and
     p = P_MAX = 0.967705, then rounded to fp32.  The literal i/(n+1) sketch
     does not give the printed table; this construction gives all 16 printed
     4-decimal values only for p in about [0.9677024, 0.9677082] (and the
     5-decimal 0.16093 of the worked example); 0.967705 is its centre.
  R2 flattening: W0 [d x k] row-major, so block b holds elements 64b..64b+63.
  R3 nearest level: x = fl32(w / scale) (correctly rounded fp32 division),
     code = #{j : x > m_j} with m_j the exact midpoint of C[j], C[j+1]; this is
     argmin |x - C[j]| with ties to the smaller j.
  R4 packing: byte t = code[2t] | code[2t+1] << 4 (even element in the low
     nibble).
  R5 the mean: one fp32 mean per tensor = fp32(T / nb) where T is a
     stride-halving float64 tree: per group of 256 scales (pairs (i, i+h) for
     h = 128..1, missing entries +0.0), then the same tree over the group sums
     padded with +0.0 to a power of two.
  R6 second level: the Int8 absmax rule applied per group to (scale - mean):
     c1 = fl32(127 / a_g) with a_g = max |fl32(s - mean)|, c2 = clamp(rint_even(
     fl32(c1 * fl32(s - mean))), -127, 127) as int8 (the pages' label "FP8" is
     read as the only 8-bit quantizer they define).  a_g = 0 or a non-finite c1
     -> c1 = 127 and c2 = 0 for the group.
  R7 dequantized scale: fl32(fl32(c2 / c1) + mean) with IEEE division.
  R8 BF16(.) is one round-to-nearest-even of the fp32 product.
  R16 c2 in FP8: the pages write doubleDequant(c1_FP32, c2_FP8, W_NF4); as a
     second format c2 is stored as OCP FP8 e4m3 (1 sign, 4 exponent bits with
     bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
     largest finite 448).  The absmax rule of R6 with 448 in place of 127:
     c1 = fl32(448 / a_g), c2 = the e4m3 value nearest fl32(c1 (s - mean))
     (clamped to +-448), ties to the even code; a_g = 0 or a non-finite c1 ->
     c1 = 448, c2 = +0.  Its value enters R7 exactly.
"""
from __future__ import annotations

from fractions import Fraction
from statistics import NormalDist

import numpy as np

P_MAX = 0.967705          # reading R1
BLOCK = 64                # chkda "Quantizing and dequantizing with the codebook"
DQ_BLOCK = 256            # chkda "Double quantization and double dequantization"
INT8_Q = 127              # chkda "First, how does k-bit quantization work?"
FP8_MAX = 448.0           # largest finite OCP e4m3 value (reading R16)
C2_FORMATS = ("int8", "fp8")


# ----------------------------------------------------------------------------
# codebook
# ----------------------------------------------------------------------------
def nf4_codebook_f64(p_max: float = P_MAX) -> np.ndarray:
    """The 16 NF4 levels in float64, before rounding to fp32 (reading R1).

    Equally spaced probabilities between P_MAX and 1/2 become standard-normal
    quantiles (chkda "Building the NF4 codebook"); 8 positive and 7 negative
    values plus an exact zero ("NF4: Choose the codebook ..."), normalised to
    [-1, 1].
    """
    q = NormalDist().inv_cdf
    positive = [q(p_max - i * (p_max - 0.5) / 8) for i in range(8)]
    negative = [-q(p_max - i * (p_max - 0.5) / 7) for i in range(7)]
    levels = sorted(negative + [0.0] + positive)
    top = max(abs(v) for v in levels)
    return np.array([v / top for v in levels], dtype=np.float64)


def nf4_codebook() -> np.ndarray:
    """The fp32 codebook C[0..15] (float32 array)."""
    return nf4_codebook_f64().astype(np.float32)


def nf4_midpoints() -> np.ndarray:
    """Exact float64 midpoints m_j = (C[j] + C[j+1]) / 2, j = 0..14.

    The sum of two fp32 values of magnitude <= 1 is exact in float64, and the
    halving is exact, so these are the true decision boundaries (reading R3).
    """
    c = nf4_codebook().astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


# ----------------------------------------------------------------------------
# bf16 rounding (reading R8)
# ----------------------------------------------------------------------------
def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    Defined on finite inputs (overflow rounds to +-inf as IEEE requires).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_nearest_bits_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 once: the nearest bf16 value, ties to the
    one with an even last mantissa bit; returns uint16 bits.

    Written from that definition: the two bf16 neighbours of |x| (8 significant
    bits, so the float64 pattern truncated to its top 8 significant bits and
    the next value up) are compared by their exact distances to |x|.  Defined
    for zero and for magnitudes in the bf16 normal range [2^-126, 2^128).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    mag = np.abs(x)
    assert np.all((mag == 0) | ((mag >= 2.0 ** -126) & (mag < 2.0 ** 128))), "outside the bf16 normal range"
    u = mag.view(np.uint64)
    step = np.uint64(1) << np.uint64(45)                  # 52 - 7 fraction bits dropped
    lo_b = u & ~(step - np.uint64(1))
    hi_b = lo_b + step                                    # a carry moves into the exponent, as it should
    lo, hi = lo_b.view(np.float64), hi_b.view(np.float64)
    d_lo, d_hi = mag - lo, hi - mag                       # both exact (same binade or Sterbenz)
    lo_even = (lo_b & step) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    r = np.where(pick_hi, hi, lo)
    r = np.where(mag == 0, 0.0, r)
    bits32 = r.astype(np.float32).view(np.uint32)         # r is a bf16 value: exact in fp32
    sign = (np.signbit(x).astype(np.uint32) << np.uint32(15))
    return ((bits32 >> np.uint32(16)) | sign).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# blockwise NF4 quantization (chkda "Quantizing and dequantizing ...")
# ----------------------------------------------------------------------------
def _blocks(w: np.ndarray, block: int) -> tuple[np.ndarray, int]:
    """Flatten (reading R2) and pad the ragged tail block with zeros."""
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = flat.size
    nb = -(-n // block)
    padded = np.zeros(nb * block, dtype=np.float32)
    padded[:n] = flat
    return padded.reshape(nb, block), n


def block_absmax(w: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """max |w| of every block of the flattened weights (exact in fp32), the
    per-block scale of the absmax rule; a ragged tail block is padded with zeros."""
    blocks, _ = _blocks(w, block)
    return np.abs(blocks).max(axis=1).astype(np.float32)


def quantize_blocks(w: np.ndarray, block: int = BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """NF4-quantize the flattened weights block by block.

    Returns (codes uint8[N] in 0..15, scale float32[nb]).  Per block the scale
    is max |w| (exact in fp32); a zero scale gives every element the
    exact-zero code; otherwise x = fl32(w / scale) and code = #{j: x > m_j}.
    Padding entries of a ragged last block are zeros and do not change its
    absmax.
    """
    blocks, n = _blocks(w, block)
    scale = block_absmax(w, block)
    zero_code = int(np.argmin(np.abs(nf4_codebook())))           # the exact 0 (index 7)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)              # fp32 IEEE division
    mids = nf4_midpoints()
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    x64 = x.astype(np.float64)
    for m in mids:
        codes += (x64 > m).astype(np.uint8)
    codes[scale == 0, :] = zero_code
    return codes.reshape(-1)[:n], scale


def nearest_level_bruteforce(x: float) -> int:
    """argmin_j |x - C[j]| in exact rational arithmetic, ties to the smaller j.

    Independent of the midpoint formulation; used to pin quantize_blocks.
    """
    cb = [Fraction(float(c)) for c in nf4_codebook()]
    fx = Fraction(float(x))
    best, best_d = 0, abs(fx - cb[0])
    for j in range(1, 16):
        d = abs(fx - cb[j])
        if d < best_d:
            best, best_d = j, d
    return best


def dequantize_blocks(codes: np.ndarray, scale: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Single-level NF4 dequantization: scale * C[code] in fp32 (no DQ)."""
    cb = nf4_codebook()
    codes = np.asarray(codes).reshape(-1)
    blk = np.arange(codes.size) // block
    return (cb[codes] * np.asarray(scale, dtype=np.float32)[blk]).astype(np.float32)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, even element in the low nibble (reading R4)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, np.uint8)])
    return (c[0::2] | (c[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & np.uint8(0x0F)
    out[1::2] = p >> np.uint8(4)
    return out[:n]


# ----------------------------------------------------------------------------
# Int8 absmax (chkda "First, how does k-bit quantization work?")
# ----------------------------------------------------------------------------
def int8_absmax_quantize(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Symmetric Int8: c = fl32(127 / absmax), q = clamp(rint_even(fl32(c*x))).

    An all-zero input (or an absmax so small that c is not finite) stores
    zeros and the nonzero scale 127 (reading R6).  Code -128 is never used.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    with np.errstate(divide="ignore", over="ignore"):
        c = np.float32(INT8_Q) / a if a != 0 else np.float32(np.inf)
    if a == 0 or not np.isfinite(c):
        return np.zeros(x.shape, dtype=np.int8), np.float32(INT8_Q)
    prod = (c * x).astype(np.float32)                             # fp32 multiply
    q = np.clip(np.rint(prod), -INT8_Q, INT8_Q).astype(np.int8)   # rint: ties to even
    return q, np.float32(c)


def int8_dequantize(q: np.ndarray, c: np.float32) -> np.ndarray:
    """Xhat = q / c, one IEEE fp32 division per element."""
    return (np.asarray(q).astype(np.float32) / np.float32(c)).astype(np.float32)


# ----------------------------------------------------------------------------
# OCP FP8 e4m3 (reading R16)
# ----------------------------------------------------------------------------
def e4m3_values() -> np.ndarray:
    """The value of each of the 256 e4m3 codes (float64; NaN for S.1111.111).

    Code = sign << 7 | E << 3 | m: E = 0 gives (m / 8) 2^-6, else (1 + m/8) 2^(E - 7).
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code of each fp32 value, ties to the even code; magnitudes
    above 448 become 448 first.  The sign bit is the sign of x (-0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x).astype(np.float64), FP8_MAX)
    vals = e4m3_values()[:127]                      # codes 0 .. 126: 0 .. 448, increasing
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (code | (np.signbit(x).astype(np.uint8) << np.uint8(7))).astype(np.uint8)


def fp8_absmax_quantize(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """The absmax rule with FP8's 448: c = fl32(448 / absmax), q = e4m3(fl32(c x)).

    An all-zero input (or a non-finite c) stores +0 codes and c = 448 (R16).
    Returns (uint8 e4m3 codes, c).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    with np.errstate(divide="ignore", over="ignore"):
        c = np.float32(FP8_MAX) / a if a != 0 else np.float32(np.inf)
    if a == 0 or not np.isfinite(c):
        return np.zeros(x.shape, dtype=np.uint8), np.float32(FP8_MAX)
    return e4m3_encode((c * x).astype(np.float32)), np.float32(c)


def c2_values(c2: np.ndarray, c2_format: str = "int8") -> np.ndarray:
    """The fp32 value of stored c2 bytes (int8, or e4m3 bit patterns)."""
    c2 = np.asarray(c2)
    if c2_format == "fp8":
        return e4m3_values()[c2.view(np.uint8).astype(np.int64)].astype(np.float32)
    return c2.astype(np.float32)


# ----------------------------------------------------------------------------
# double quantization (chkda "Double quantization and double dequantization")
# ----------------------------------------------------------------------------
def tree_sum_f64(values: np.ndarray) -> np.float64:
    """Stride-halving float64 tree: a[i] += a[i + h] for h = n/2, ..., 1.

    ``values`` is padded with +0.0 to a power of two first (reading R5).
    """
    v = np.asarray(values, dtype=np.float64).reshape(-1)
    n = 1
    while n < v.size:
        n *= 2
    a = np.zeros(n, dtype=np.float64)
    a[: v.size] = v
    while a.size > 1:
        h = a.size // 2
        a = a[:h] + a[h:]
    return a[0]


def scales_mean(scale: np.ndarray, dq_block: int = DQ_BLOCK) -> np.float32:
    """fp32(T / nb) with T the two-level stride-halving tree (reading R5)."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    nb = s.size
    g = -(-nb // dq_block)
    padded = np.zeros(g * dq_block, dtype=np.float64)
    padded[:nb] = s
    partial = np.array([tree_sum_f64(padded[i * dq_block:(i + 1) * dq_block]) for i in range(g)])
    total = tree_sum_f64(partial)
    return np.float32(total / np.float64(nb))


def double_quantize(scale: np.ndarray, dq_block: int = DQ_BLOCK, c2_format: str = "int8"):
    """Quantize the block scales: returns (c2 [nb], c1 float32[G], mean float32).

    Each group of ``dq_block`` centred scales (fl32(s - mean)) is absmax
    quantized with its own fp32 second-level scale c1: Int8 (reading R6, c2
    int8) or FP8 e4m3 (reading R16, c2 uint8 bit patterns).
    """
    assert c2_format in C2_FORMATS
    s = np.asarray(scale, dtype=np.float32).reshape(-1)
    nb = s.size
    mean = scales_mean(s, dq_block)
    centred = (s - mean).astype(np.float32)
    g = -(-nb // dq_block)
    fp8 = c2_format == "fp8"
    c2 = np.zeros(nb, dtype=np.uint8 if fp8 else np.int8)
    c1 = np.zeros(g, dtype=np.float32)
    quant = fp8_absmax_quantize if fp8 else int8_absmax_quantize
    for i in range(g):
        q, c = quant(centred[i * dq_block:(i + 1) * dq_block])
        c2[i * dq_block:(i + 1) * dq_block] = q
        c1[i] = c
    return c2, c1, mean


def double_dequantize_scales(c2: np.ndarray, c1: np.ndarray, mean, dq_block: int = DQ_BLOCK,
                             c2_format: str = "int8") -> np.ndarray:
    """scales[j] = dequant(c2[j], c1[j // dq_block]) + mean, all in fp32 (R7)."""
    c2 = np.asarray(c2).reshape(-1)
    group = np.arange(c2.size) // dq_block
    q = (c2_values(c2, c2_format) / np.asarray(c1, dtype=np.float32)[group]).astype(np.float32)
    return (q + np.float32(mean)).astype(np.float32)


def double_dequantize(packed: np.ndarray, c2: np.ndarray, c1: np.ndarray, mean, n: int,
                      block: int = BLOCK, dq_block: int = DQ_BLOCK, c2_format: str = "int8") -> np.ndarray:
    """doubleDequant: W[i] = BF16(C[W[i]] * scales[i // block]); uint16 bits [n]."""
    codes = unpack_codes(packed, n)
    shat = double_dequantize_scales(c2, c1, mean, dq_block, c2_format)
    blk = np.arange(n) // block
    prod = (nf4_codebook()[codes] * shat[blk]).astype(np.float32)  # one fp32 multiply
    return bf16_rne_bits(prod)


# ----------------------------------------------------------------------------
# the whole storage format
# ----------------------------------------------------------------------------
def quantize(w0: np.ndarray, block: int = BLOCK, dq_block: int = DQ_BLOCK, c2_format: str = "int8") -> dict:
    """NF4 + double quantization of W0 [d x k] (fp32).

    Returns a dict with packed codes (uint8[N/2]), codes (uint8[N]), the exact
    block scales (float32[nb]), c2 ([nb]: int8, or uint8 e4m3 bit patterns),
    c1 (float32[G]), mean (float32) and the c2 format.
    """
    codes, scale = quantize_blocks(w0, block)
    c2, c1, mean = double_quantize(scale, dq_block, c2_format)
    return {"codes": codes, "packed": pack_codes(codes), "absmax": scale,
            "c2": c2, "c1": c1, "mean": np.float32(mean), "n": int(np.asarray(w0).size),
            "c2_format": c2_format}


def dequantize(q: dict, shape=None, block: int = BLOCK, dq_block: int = DQ_BLOCK) -> np.ndarray:
    """bf16 bits of the double-dequantized weights, optionally reshaped."""
    bits = double_dequantize(q["packed"], q["c2"], q["c1"], q["mean"], q["n"], block, dq_block,
                             q.get("c2_format", "int8"))
    return bits.reshape(shape) if shape is not None else bits


def quantize_single(w0: np.ndarray, block: int = BLOCK) -> dict:
    """NF4 without double quantization: the block absmax itself is stored (fp32).

    chkda "Double quantization and double dequantization", its bits-per-weight
    accounting: before double quantization one fp32 scale serves each block of
    64 weights.  Returns packed codes, codes, the fp32 absmax per block and n.
    """
    codes, scale = quantize_blocks(w0, block)
    return {"codes": codes, "packed": pack_codes(codes), "absmax": scale,
            "n": int(np.asarray(w0).size)}


def dequantize_single(q: dict, shape=None, block: int = BLOCK) -> np.ndarray:
    """bf16 bits of W[i] = BF16(C[code[i]] * absmax[i // block]) (R8), no DQ."""
    codes = unpack_codes(q["packed"], q["n"])
    bits = bf16_rne_bits(dequantize_blocks(codes, q["absmax"], block))
    return bits.reshape(shape) if shape is not None else bits


def storage_bits_per_weight(n: int, block: int = BLOCK, dq_block: int = DQ_BLOCK) -> dict:
    """Bits per weight of the stored format, split as the pages count it.

    chkda "Double quantization ...": before DQ one fp32 scale per block (32/64
    bits per weight); after DQ one 8-bit scale per block plus one fp32 scale
    per group of ``dq_block`` blocks.  The single fp32 mean is reported apart.
    """
    nb = -(-n // block)
    g = -(-nb // dq_block)
    return {"codes": 4.0, "scales_before": 32.0 * nb / n,
            "scales_after": (8.0 * nb + 32.0 * g) / n, "mean": 32.0 / n}
