"""Pins for the CPU oracle: what the pages and mathematics fix, not the oracle itself.

Every expected value below is printed on the pages (fixtures under
tests/golden/, each with its citation), a closed form, an invariant, a
textbook/library routine, or a brute force on tiny inputs.  Runs without a GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import nf4, qlora
from tests.conftest import golden_kv, read_golden
from workloads import bf16_bits_as_f32, make_layer, random_weights


def printed_levels():
    return np.array([float(v) for v in read_golden("nf4_levels_printed.txt")])


# ----------------------------------------------------------------------------
# codebook -- chkda "NF4: Choose the codebook to fit the distribution"
# ----------------------------------------------------------------------------
def test_codebook_reproduces_printed_levels():
    c = nf4.nf4_codebook().astype(np.float64)
    printed = printed_levels()
    assert printed.size == 16
    # every level rounds to the printed 4-decimal value
    assert np.all(np.abs(c - printed) < 5e-5), np.abs(c - printed).max()


def test_codebook_structure():
    c = nf4.nf4_codebook()
    assert c.dtype == np.float32 and c.size == 16
    assert c.view(np.uint32)[7] == 0                 # exact +0.0
    assert c[0] == np.float32(-1.0) and c[15] == np.float32(1.0)
    assert np.all(np.diff(c) > 0)                    # strictly increasing
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8


def test_codebook_level9_worked_example_five_decimals():
    kv = golden_kv("worked_examples.txt")
    c9 = float(nf4.nf4_codebook()[int(kv["nf4.code"][0])])
    assert abs(c9 - float(kv["nf4.level_5dp"][0])) < 5e-6


@pytest.mark.parametrize("p_max", [0.9677, 0.96770833, 0.9677000, 0.9678])
def test_codebook_reading_window_excludes_nearby_constants(p_max):
    """The printed table pins p_max to a narrow window (reading R1): nearby
    round constants fail at least one printed level or the 5-decimal C[9]."""
    c = nf4.nf4_codebook_f64(p_max)
    printed = printed_levels()
    ok4 = all(round(a, 4) == b for a, b in zip(c, printed))
    ok5 = round(c[9], 5) == 0.16093
    assert not (ok4 and ok5)


def test_midpoints_are_exact():
    c = nf4.nf4_codebook()
    m = nf4.nf4_midpoints()
    for j in range(15):
        from fractions import Fraction
        assert Fraction(m[j]) == (Fraction(float(c[j])) + Fraction(float(c[j + 1]))) / 2


# ----------------------------------------------------------------------------
# nearest-level quantizer -- chkda "Quantizing and dequantizing with the codebook"
# ----------------------------------------------------------------------------
def _codes_with_unit_scale(x: np.ndarray) -> np.ndarray:
    """Quantize values of [-1, 1] in blocks whose absmax is exactly 1."""
    x = np.asarray(x, dtype=np.float32)
    n = x.size
    nblk = -(-n // 63)
    blocks = np.zeros((nblk, 64), dtype=np.float32)
    blocks[:, 0] = 1.0
    flat = blocks[:, 1:].reshape(-1)
    flat[:n] = x
    blocks[:, 1:] = flat.reshape(nblk, 63)
    codes, scale = nf4.quantize_blocks(blocks)
    assert np.all(scale == 1.0)
    return codes.reshape(nblk, 64)[:, 1:].reshape(-1)[:n]


def test_quantizer_matches_exact_bruteforce_random():
    rng = np.random.default_rng(1)
    x = rng.uniform(-1, 1, 3000).astype(np.float32)
    got = _codes_with_unit_scale(x)
    want = np.array([nf4.nearest_level_bruteforce(v) for v in x])
    assert np.array_equal(got, want)


def test_quantizer_adversarial_points():
    """Exact midpoints (ties -> smaller index), their fp32 neighbours, +-0,
    tiny and subnormal values, the levels themselves and +-1."""
    c = nf4.nf4_codebook()
    m = nf4.nf4_midpoints()
    pts = [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-38, -1e-38]
    pts += list(c)
    for mj in m:
        f = np.float32(mj)
        pts += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    x = np.array(pts, dtype=np.float32)
    got = _codes_with_unit_scale(x)
    want = np.array([nf4.nearest_level_bruteforce(v) for v in x])
    assert np.array_equal(got, want)


def test_ties_go_to_smaller_index():
    c = nf4.nf4_codebook()
    m = nf4.nf4_midpoints()
    ties = [j for j in range(15) if float(np.float32(m[j])) == m[j]]
    assert len(ties) >= 1
    got = _codes_with_unit_scale(np.array([m[j] for j in ties], dtype=np.float32))
    assert list(got) == ties


def test_all_zero_block_gets_exact_zero_code():
    codes, scale = nf4.quantize_blocks(np.zeros(128, np.float32))
    assert np.all(scale == 0) and np.all(codes == 7)
    assert nf4.nf4_codebook()[7] == 0


def test_worked_example_nf4():
    kv = golden_kv("worked_examples.txt")
    s = np.float32(float(kv["nf4.scale"][0]))
    w = np.float32(float(kv["nf4.weight"][0]))
    block = np.zeros(64, np.float32)
    block[0], block[1] = s, w
    codes, scale = nf4.quantize_blocks(block)
    assert scale[0] == s
    assert codes[1] == int(kv["nf4.code"][0]) == int(kv["nf4.code_binary"][0], 2)
    assert codes[0] == 15 and np.all(codes[2:] == 7)
    assert abs(float(w / s) - float(kv["nf4.normalised"][0])) < 1e-7
    rec = nf4.dequantize_blocks(codes, scale)[1]
    # the page multiplies the 5-decimal level by the scale, so the printed
    # 0.32186 carries the level's rounding error (<= 5e-6) times the scale
    assert abs(float(rec) - float(kv["nf4.reconstructed_5dp"][0])) <= float(s) * 5e-6
    # nibble order (reading R4): code 15 low, code 9 high -> 0x9F; zeros -> 0x77
    packed = nf4.pack_codes(codes)
    assert packed[0] == 0x9F and np.all(packed[1:] == 0x77) and packed.size == 32
    assert np.array_equal(nf4.unpack_codes(packed, 64), codes)


def test_round_trip_bound_half_gap():
    w = random_weights(3, (64, 64 * 40), std=1.0)
    codes, scale = nf4.quantize_blocks(w)
    c = nf4.nf4_codebook().astype(np.float64)
    gaps = np.diff(c)
    blk = np.arange(w.size) // 64
    x = (w.reshape(-1) / scale[blk]).astype(np.float32).astype(np.float64)
    err = np.abs(x - c[codes])
    # the error is at most half of the gap of the interval x falls in
    idx = np.clip(np.searchsorted(c, x) - 1, 0, 14)
    assert np.all(err <= gaps[idx] / 2 + 1e-12)
    assert err.max() <= (c[1] - c[0]) / 2 + 1e-12 and (c[1] - c[0]) / 2 < 0.1520


def test_ragged_tail_block():
    w = random_weights(4, (1, 64 * 3 + 10))
    codes, scale = nf4.quantize_blocks(w)
    assert codes.size == w.size and scale.size == 4
    assert scale[3] == np.abs(w.reshape(-1)[192:]).max()


# ----------------------------------------------------------------------------
# Int8 absmax -- chkda "First, how does k-bit quantization work?"
# ----------------------------------------------------------------------------
def test_worked_example_int8():
    kv = golden_kv("worked_examples.txt")
    x = np.array([float(v) for v in kv["int8.x"]], np.float32)
    q, c = nf4.int8_absmax_quantize(x)
    assert c == np.float32(float(kv["int8.c"][0]))
    assert list(q) == [int(v) for v in kv["int8.q"]]
    xhat = nf4.int8_dequantize(q, c)
    assert [round(float(v), 4) for v in xhat] == [float(v) for v in kv["int8.xhat_4dp"]]
    assert xhat[1] == np.float32(38) / np.float32(127)


def test_int8_range_and_zero_input():
    rng = np.random.default_rng(2)
    for _ in range(50):
        x = rng.standard_normal(256).astype(np.float32)
        q, c = nf4.int8_absmax_quantize(x)
        assert q.min() >= -127 and q.max() <= 127
        assert np.abs(q).max() == 127
    q, c = nf4.int8_absmax_quantize(np.zeros(16, np.float32))
    assert np.all(q == 0) and c != 0


# ----------------------------------------------------------------------------
# double quantization -- chkda "Double quantization and double dequantization"
# ----------------------------------------------------------------------------
def test_bits_per_weight():
    kv = golden_kv("worked_examples.txt")
    for n in (4096 * 4096, 11008 * 4096, 22016 * 8192, 256 * 512):
        b = nf4.storage_bits_per_weight(n)
        assert b["scales_before"] == float(kv["dq.before"][0])
        assert b["scales_after"] == float(kv["dq.after"][0])
        assert b["scales_before"] - b["scales_after"] == float(kv["dq.saved"][0])
        assert round(b["codes"] + b["scales_after"], 3) == 4.127


def test_tree_sum_pairs_stride_halving():
    # stride-halving pairs (0,2),(1,3) then (0,1): (1e16 - 1e16) + (1 + 1) = 2;
    # a sequential sum gives 1 and an adjacent-pair tree gives 0 in float64.
    v = np.array([1e16, 1.0, -1e16, 1.0])
    assert nf4.tree_sum_f64(v) == 2.0
    assert ((v[0] + v[1]) + v[2]) + v[3] == 1.0
    assert (v[0] + v[1]) + (v[2] + v[3]) == 0.0


def test_tree_sum_exact_and_padded():
    v = np.arange(1, 1001, dtype=np.float64)
    assert nf4.tree_sum_f64(v) == 500500.0
    assert nf4.tree_sum_f64(np.array([3.5])) == 3.5


def test_mean_close_to_exact_sum():
    s = np.abs(random_weights(5, (1000 * 64,))).reshape(-1, 64).max(axis=1)
    mean = nf4.scales_mean(s)
    exact = math.fsum(float(v) for v in s) / s.size
    assert abs(float(mean) - exact) <= np.spacing(np.float32(exact))


def test_double_quant_worked_int8_example():
    """Scales whose mean is 0 reduce double quantization to the printed Int8
    example on (s - mean) = [-1, 0.3, 1, -0.3]."""
    s = np.array([-1.0, 0.3, 1.0, -0.3], np.float32)
    c2, c1, mean = nf4.double_quantize(s)
    assert mean == 0 and c1[0] == 127
    assert list(c2) == [-127, 38, 127, -38]
    shat = nf4.double_dequantize_scales(c2, c1, mean)
    assert [round(float(v), 4) for v in shat] == [-1.0, 0.2992, 1.0, -0.2992]


def test_double_quant_round_trip_bound_and_ragged_groups():
    w = random_weights(6, (37, 64 * 300))          # nb = 11100: ragged last group
    codes, s = nf4.quantize_blocks(w)
    c2, c1, mean = nf4.double_quantize(s)
    assert c1.size == -(-s.size // 256)
    shat = nf4.double_dequantize_scales(c2, c1, mean)
    centred = (s - mean).astype(np.float32)
    for g in range(c1.size):
        sl = slice(g * 256, (g + 1) * 256)
        a_g = np.abs(centred[sl]).max()
        err = np.abs(shat[sl].astype(np.float64) - s[sl])
        assert np.all(err <= a_g / 254 * (1 + 1e-6) + 4 * np.spacing(s[sl]))
    assert np.all(np.abs(c2.astype(int)) <= 127)


def test_zero_group_and_zero_tensor():
    c2, c1, mean = nf4.double_quantize(np.zeros(300, np.float32))
    assert mean == 0 and np.all(c2 == 0) and np.all(c1 == 127)
    q = nf4.quantize(np.zeros((4, 64), np.float32))
    bits = nf4.dequantize(q)
    assert np.all((bits & 0x7FFF) == 0)           # +-0 exactly


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3)
    # exact ties: low 16 bits 0x8000, both parities of the kept bit
    hi = rng.integers(0x3000, 0x4F00, 4000, dtype=np.uint32) | (rng.integers(0, 2, 4000, dtype=np.uint32) << 15)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)   # both parities of the kept bit
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, -3e-39], np.float32)])
    assert np.all(np.isfinite(x))
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.bf16_rne_bits(x), want)


def test_double_dequant_error_bound():
    w = random_weights(8, (64, 64 * 64))
    q = nf4.quantize(w)
    what = nf4.bf16_bits_to_f32(nf4.dequantize(q)).astype(np.float64)
    shat = nf4.double_dequantize_scales(q["c2"], q["c1"], q["mean"]).astype(np.float64)
    blk = np.arange(w.size) // 64
    c = nf4.nf4_codebook().astype(np.float64)[q["codes"]]
    s = q["absmax"].astype(np.float64)[blk]
    bound = 0.1520 * s + np.abs(s - shat[blk]) + 2.0 ** -8 * np.abs(c * shat[blk]) + 1e-12
    assert np.all(np.abs(w.reshape(-1) - what) <= bound)


# ----------------------------------------------------------------------------
# c2 in FP8 (OCP e4m3) -- chkda "Double quantization and double
# dequantization" labels c2 as FP8 (reading R16)
# ----------------------------------------------------------------------------
def test_e4m3_closed_form_values():
    v = nf4.e4m3_values()
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9        # subnormals m 2^-9
    assert v[0x08] == 2.0 ** -6                                      # smallest normal
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0 == nf4.FP8_MAX and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:127]) > 0)                              # codes 0..126 increasing
    assert np.array_equal(v[0x80:0xFF], -v[:127])


def test_e4m3_against_torch_float8_e4m3fn():
    # torch's CPU float8_e4m3fn is an independent implementation of the same
    # OCP format: decoding of all 256 codes, and round-to-nearest-even encoding
    # of in-range values (torch does not saturate above 448, the oracle clamps)
    v = nf4.e4m3_values()
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    rng = np.random.default_rng(25)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-14, 6.5, 100000))).astype(np.float32)
    vals = v[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)           # exact ties
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e4)),
                        vals.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0])])
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nf4.e4m3_encode(x), want)
    assert np.all(nf4.e4m3_encode(np.float32([460.0, 1e6, -1e6])) == [0x7E, 0x7E, 0xFE])


def test_fp8_double_quant_largest_maps_to_448_and_error_bound():
    w = random_weights(26, (64, 64 * 64))
    q = nf4.quantize(w, c2_format="fp8")
    assert q["c2"].dtype == np.uint8
    s = q["absmax"].astype(np.float64)
    x = (q["absmax"] - q["mean"]).astype(np.float32)
    vals = nf4.c2_values(q["c2"], "fp8").astype(np.float64)
    for g in range(q["c1"].size):
        sl = slice(256 * g, 256 * (g + 1))
        a = np.abs(x[sl]).max()
        assert q["c1"][g] == np.float32(448.0) / np.float32(a)        # the absmax rule with 448
        assert np.abs(vals[sl]).max() == 448.0                        # the largest maps to 448
    shat = nf4.double_dequantize_scales(q["c2"], q["c1"], q["mean"], c2_format="fp8").astype(np.float64)
    c1 = q["c1"].astype(np.float64)[np.arange(s.size) // 256]
    eps = 2.0 ** -23
    # 3 mantissa bits: half an ulp is 2^-4 relative (2^-10 absolute below 2^-6)
    bound = (2.0 ** -4 * np.abs(x) * (1 + 4 * eps) + 2.0 ** -10 / c1
             + 4 * eps * (np.abs(s) + np.abs(float(q["mean"]))))
    assert np.all(np.abs(shat - s) <= bound)
    # the Int8 format on the same scales has a uniform step 1/c1: FP8 is finer near the mean
    q8 = nf4.quantize(w)
    e8 = np.abs(nf4.double_dequantize_scales(q8["c2"], q8["c1"], q8["mean"]).astype(np.float64) - s)
    small = np.abs(x) < np.abs(x).max() / 16
    assert np.abs(shat - s)[small].mean() < e8[small].mean()


def test_fp8_zero_group_and_dequant_path():
    c2, c1, mean = nf4.double_quantize(np.full(300, 0.5, np.float32), c2_format="fp8")
    assert np.all(c2 == 0) and np.all(c1 == np.float32(448)) and mean == np.float32(0.5)
    w = random_weights(27, (8, 64 * 40))
    q = nf4.quantize(w, c2_format="fp8")
    bits = nf4.dequantize(q)
    # the same doubleDequant with the c2 values written out as fp32 by hand
    sh = ((nf4.e4m3_values()[q["c2"].astype(np.int64)].astype(np.float32)
           / q["c1"][np.arange(q["c2"].size) // 256]).astype(np.float32) + q["mean"]).astype(np.float32)
    prod = (nf4.nf4_codebook()[q["codes"]] * sh[np.arange(w.size) // 64]).astype(np.float32)
    assert np.array_equal(bits, nf4.bf16_rne_bits(prod))


# ----------------------------------------------------------------------------
# adapter dropout (reading R17): Philox4x32-10 and the dropout layer
# ----------------------------------------------------------------------------
def _philox_scalar(ctr, key, width):
    """Philox4xW-10 on Python ints, for W = 32 (the dropout generator) and
    W = 64 (numpy's Philox): one counter at a time, written from the round
    definition independently of the vectorized oracle."""
    mask = (1 << width) - 1
    mult = {32: (0xD2511F53, 0xCD9E8D57), 64: (0xD2E7470EE14C6C93, 0xCA5A826395121157)}[width]
    weyl = {32: (0x9E3779B9, 0xBB67AE85), 64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)}[width]
    c, k = list(ctr), list(key)
    for rnd in range(10):
        if rnd:
            k = [(k[0] + weyl[0]) & mask, (k[1] + weyl[1]) & mask]
        p0, p1 = mult[0] * c[0], mult[1] * c[2]
        c = [(p1 >> width) ^ c[1] ^ k[0], p1 & mask, (p0 >> width) ^ c[3] ^ k[1], p0 & mask]
    return c


def test_philox4x32_known_answers():
    for name, *words in (line.split() for line in read_golden("philox_kat.txt")):
        v = [int(w, 16) for w in words]
        got = qlora.philox4x32_10(np.array([v[:4]], np.uint64), (v[4], v[5]))[0]
        assert [int(g) for g in got] == v[6:], name
        assert _philox_scalar(v[:4], v[4:6], 32) == v[6:], name


def test_philox_rounds_match_numpy_philox4x64():
    # numpy's Philox bit generator is Philox4x64-10; it advances its counter
    # before each block, so its block j comes from counter + j + 1
    for key, ctr0 in (((0, 0), 0), ((0x0123456789ABCDEF, 42), 7), ((2**64 - 1, 5), 2**64 - 3)):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                              counter=np.array([ctr0, 0, 0, 0], dtype=np.uint64))
        raw = [int(v) for v in bg.random_raw(12)]
        for j in range(3):
            c = ctr0 + j + 1
            ctr = [c & (2**64 - 1), c >> 64, 0, 0]
            assert _philox_scalar(ctr, list(key), 64) == raw[4 * j:4 * j + 4]


def test_philox4x32_vectorized_equals_scalar():
    rng = np.random.default_rng(28)
    ctr = rng.integers(0, 2**32, (64, 4), dtype=np.uint64)
    key = (int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32)))
    got = qlora.philox4x32_10(ctr, key)
    for i in range(64):
        assert [int(g) for g in got[i]] == _philox_scalar([int(c) for c in ctr[i]], list(key), 32)


def test_dropout_mask_layout_rate_and_edges():
    m, k, seed = 48, 1024, 0x1234_5678_9ABC
    keep = qlora.dropout_keep_mask(m, k, 0.05, seed)
    # element i uses word i % 4 of the block for counter i // 4 (low, high words)
    for i in (0, 1, 2, 3, 4, 7, 8, 4097, m * k - 1):
        blk = i // 4
        w = _philox_scalar([blk & 0xFFFFFFFF, blk >> 32, 0, 0], [seed & 0xFFFFFFFF, seed >> 32], 32)[i % 4]
        assert keep.reshape(-1)[i] == (w >= qlora.dropout_threshold(0.05))
    for p in (0.05, 0.3, 0.5):
        frac = 1.0 - qlora.dropout_keep_mask(m, k, p, seed + 1).mean()
        assert abs(frac - p) < 5 * np.sqrt(p * (1 - p) / (m * k))
    assert qlora.dropout_keep_mask(m, k, 0.0, seed).all()
    assert qlora.dropout_threshold(0.5) == 2**31 and qlora.dropout_threshold(0.0) == 0
    # the threshold is floor(p 2^32) of the fp32 p, exactly, in rationals
    from fractions import Fraction
    for p in (0.05, 0.1, 0.3, 1e-9, 0.999999):
        exact = Fraction(float(np.float32(p))) * 2**32
        assert qlora.dropout_threshold(p) == exact.numerator // exact.denominator
    assert qlora.dropout_threshold(0.05) == 214748368          # fp32(0.05) = 0.0500000007...
    assert qlora.dropout_scale(0.5) == np.float32(2.0) and qlora.dropout_scale(0.0) == np.float32(1.0)
    assert not np.array_equal(keep, qlora.dropout_keep_mask(m, k, 0.05, seed + 1))


def test_lora_dropout_values():
    x = make_layer(29, 0, 8, 512, 32, 4).x
    xd, keep = qlora.lora_dropout_bits(x, 0.0, 5)
    assert keep.all() and np.array_equal(xd, x)                    # p = 0: the identity
    xd, keep = qlora.lora_dropout_bits(x, 0.1, 5)
    assert np.all(xd[~keep] == 0)
    xs, ref = bf16_bits_as_f32(xd)[keep].astype(np.float64), bf16_bits_as_f32(x)[keep].astype(np.float64) / 0.9
    assert np.all(np.abs(xs - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)  # one bf16 rounding of x / (1 - p)


def test_dropout_backward_central_finite_differences():
    rng = np.random.default_rng(30)
    m, d, k, r, alpha, p = 5, 6, 8, 3, 12.0, 0.25
    w = rng.standard_normal((d, k))
    a, b, x, dy = (rng.standard_normal(sh) for sh in ((r, k), (d, r), (m, k), (m, d)))
    keep = qlora.dropout_keep_mask(m, k, p, 77)
    c = float(qlora.dropout_scale(p))

    def loss(x_, a_, b_):
        y, _ = qlora.forward_dropout(w, x_, c * keep * x_, a_, b_, alpha)
        return float(np.sum(y * dy))
    dx, da, db = qlora.backward_dropout(w, c * keep * x, keep, dy, a, b, alpha, p)
    h = 1e-6
    for arr, grad, f in ((x, dx, lambda t: loss(t, a, b)), (a, da, lambda t: loss(x, t, b)),
                         (b, db, lambda t: loss(x, a, t))):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            e = np.zeros_like(arr)
            e[idx] = h
            num[idx] = (f(arr + e) - f(arr - e)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-6)
    y0, u0 = qlora.forward_dropout(w, x, x, a, b, alpha)               # p = 0 reduces to the plain layer
    y1, u1 = qlora.forward(w, x, a, b, alpha)
    assert np.allclose(y0, y1, rtol=1e-13, atol=1e-12) and np.allclose(u0, u1, rtol=1e-13, atol=1e-12)


# ----------------------------------------------------------------------------
# the format without double quantization -- chkda "Double quantization and
# double dequantization", the bits-per-weight accounting ("before")
# ----------------------------------------------------------------------------
def test_single_level_worked_example():
    kv = golden_kv("worked_examples.txt")
    s = np.float32(float(kv["nf4.scale"][0]))
    block = np.zeros(64, np.float32)
    block[0], block[1] = s, np.float32(float(kv["nf4.weight"][0]))
    q = nf4.quantize_single(block)
    assert q["absmax"].dtype == np.float32 and q["absmax"][0] == s
    what = nf4.bf16_bits_to_f32(nf4.dequantize_single(q)).astype(np.float64)
    assert what[0] == float(s) and np.all(what[2:] == 0)
    # the printed 0.32186 (5-decimal level times the scale), plus bf16's half ulp
    assert abs(what[1] - float(kv["nf4.reconstructed_5dp"][0])) <= float(s) * 5e-6 + 2.0 ** -9 * 0.33


def test_single_level_storage_is_four_and_a_half_bits():
    kv = golden_kv("worked_examples.txt")
    for shape in ((256, 512), (64, 4096)):
        q = nf4.quantize_single(random_weights(21, shape))
        n = q["n"]
        bits = 8.0 * (q["packed"].nbytes + q["absmax"].nbytes) / n
        assert bits == float(kv["dq.total_before"][0])
        assert q["absmax"].nbytes * 8.0 / n == float(kv["dq.before"][0])
    b = nf4.storage_bits_per_weight(4096 * 4096)
    assert round(b["codes"] + b["scales_after"], 3) == float(kv["dq.total_after_approx"][0])


def test_single_level_error_bound():
    w = random_weights(22, (64, 64 * 64))
    q = nf4.quantize_single(w)
    what = nf4.bf16_bits_to_f32(nf4.dequantize_single(q)).astype(np.float64)
    s = q["absmax"].astype(np.float64)[np.arange(w.size) // 64]
    c = nf4.nf4_codebook().astype(np.float64)[q["codes"]]
    # half the widest codebook gap of the level, then one bf16 rounding
    bound = 0.1520 * s + 2.0 ** -8 * np.abs(c * s) + 1e-12
    assert np.all(np.abs(w.reshape(-1) - what) <= bound)
    # and per element: the nearest level, found by exact brute force
    rng = np.random.default_rng(23)
    for i in rng.integers(0, w.size, 200):
        x = np.float32(np.float32(w.reshape(-1)[i]) / np.float32(s[i]))
        assert q["codes"][i] == nf4.nearest_level_bruteforce(float(x))


@pytest.mark.parametrize("block", [128, 256])
def test_larger_blocks_nearest_level_and_reduction_to_64(block):
    # each element: the exact brute-force nearest level of w / absmax(its block)
    w = random_weights(31, (8, 2 * block * 4))
    q = nf4.quantize_single(w, block)
    s = q["absmax"][np.arange(w.size) // block]
    assert np.all(s == np.abs(w.reshape(-1, block)).max(axis=1).repeat(block))
    rng = np.random.default_rng(32)
    for i in rng.integers(0, w.size, 200):
        x = np.float32(np.float32(w.reshape(-1)[i]) / np.float32(s[i]))
        assert q["codes"][i] == nf4.nearest_level_bruteforce(float(x))
    # a tensor whose 64-weight pieces all share their block's absmax quantizes the
    # same with blocks of 64 and of `block` (no double quantization)
    v = np.clip(random_weights(33, (4, 4 * block)), -0.5, 0.5).reshape(-1, 64)
    v[:, 3] = np.repeat(np.linspace(0.6, 0.9, v.shape[0] // (block // 64)), block // 64).astype(np.float32)
    v = v.reshape(4, 4 * block)
    q64, qb = nf4.quantize_single(v, 64), nf4.quantize_single(v, block)
    assert np.array_equal(q64["packed"], qb["packed"])
    assert np.array_equal(nf4.dequantize_single(q64, v.shape, 64), nf4.dequantize_single(qb, v.shape, block))
    bits = nf4.storage_bits_per_weight(4096 * 4096, block)
    assert bits["scales_before"] == 32.0 / block and bits["scales_after"] == 8.0 / block + 32.0 / (256 * block)


def test_single_level_equals_double_quant_when_dq_is_exact():
    # every block has absmax 0.75: the mean is 0.75 exactly, the centred scales
    # are 0, so c2 = 0, c1 = 127 and the recovered scale is exactly 0.75 --
    # both formats must then give the same bf16 weights
    w = random_weights(24, (48, 64 * 48), std=0.1)
    blk = w.reshape(-1, 64)
    blk[:] = np.clip(blk, -0.7, 0.7)
    blk[:, 5] = np.where(np.arange(blk.shape[0]) % 2 == 0, 0.75, -0.75)
    dq = nf4.quantize(w)
    assert np.all(dq["c2"] == 0) and dq["mean"] == np.float32(0.75)
    single = nf4.quantize_single(w)
    assert np.array_equal(nf4.dequantize(dq), nf4.dequantize_single(single))
    assert np.array_equal(dq["packed"], single["packed"])


# ----------------------------------------------------------------------------
# the linear layer -- chkda "How does it work?", "Merging LoRA weights ...";
# fromzero2ai "Why Does This Save Memory?"
# ----------------------------------------------------------------------------
def test_parameter_count():
    kv = golden_kv("worked_examples.txt")
    d, k, r = (int(kv[f"params.{n}"][0]) for n in "dkr")
    n = qlora.trainable_parameters(d, k, r)
    assert n == int(kv["params.count"][0])
    assert d * k == int(kv["params.full"][0]) and d * k // n == int(kv["params.ratio"][0])
    a = np.zeros((r, k)); b = np.zeros((d, r))
    assert a.size + b.size == n


def _tiny_layer(seed=0, m=5, d=6, k=7, r=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((d, k)), rng.standard_normal((m, k)), rng.standard_normal((r, k)),
            rng.standard_normal((d, r)), rng.standard_normal((m, d)))


def test_b_zero_and_alpha_zero_leave_base_output():
    w, x, a, b, _ = _tiny_layer()
    base = x @ w.T
    y0, _ = qlora.forward(w, x, a, np.zeros_like(b), 16.0)
    y1, _ = qlora.forward(w, x, a, b, 0.0)
    assert np.array_equal(y0, base) and np.array_equal(y1, base)
    _, da, _ = qlora.backward(w, x, np.ones((x.shape[0], w.shape[0])), a, np.zeros_like(b), 16.0)
    assert np.all(da == 0)


def test_merge_equivalence():
    w, x, a, b, _ = _tiny_layer(1, m=9, d=16, k=12, r=4)
    y, _ = qlora.forward(w, x, a, b, 8.0)
    ym = x @ qlora.merged_weight(w, a, b, 8.0).T
    assert np.allclose(y, ym, rtol=1e-12, atol=1e-12)


def test_forward_reduces_to_matmul_of_merged_weight_rank_one():
    # r = 1, alpha = 1: Y = X (W + b a)^T, computed as an explicit sum of outer products
    w, x, a, b, _ = _tiny_layer(2, m=3, d=4, k=5, r=1)
    y, u = qlora.forward(w, x, a, b, 1.0)
    for i in range(3):
        for o in range(4):
            want = sum(x[i, j] * (w[o, j] + b[o, 0] * a[0, j]) for j in range(5))
            assert abs(y[i, o] - want) < 1e-12
    assert np.allclose(u[:, 0], [sum(x[i, j] * a[0, j] for j in range(5)) for i in range(3)])


def test_backward_central_finite_differences():
    w, x, a, b, dy = _tiny_layer(3)
    alpha = 6.0
    dx, da, db = qlora.backward(w, x, dy, a, b, alpha)

    def loss(xx, aa, bb):
        y, _ = qlora.forward(w, xx, aa, bb, alpha)
        return float(np.sum(dy * y))

    h = 1e-6
    for arr, grad, which in ((x, dx, 0), (a, da, 1), (b, db, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            mm = arr.copy(); mm[idx] -= h
            args_p = [x, a, b]; args_m = [x, a, b]
            args_p[which] = p; args_m[which] = mm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(num, grad, rtol=1e-6, atol=1e-7), which


def test_workload_inputs_are_bf16_and_seeded():
    l1 = make_layer(0, 0, 8, 64, 4, 2)
    l2 = make_layer(0, 0, 8, 64, 4, 2)
    assert np.array_equal(l1.w0, l2.w0) and np.array_equal(l1.x, l2.x)
    assert l1.x.dtype == np.uint16 and l1.w0.dtype == np.float32
    xf = bf16_bits_as_f32(l1.x)
    assert np.all(np.isfinite(xf))


def test_adapter_grads_central_finite_differences():
    """The dX-free adapter gradients, pinned like backward(): central finite
    differences of sum(dY * Y) in fp64."""
    w, x, a, b, dy = _tiny_layer(4)
    alpha = 10.0
    da, db = qlora.adapter_grads(x, dy, a, b, alpha)

    def loss(aa, bb):
        y, _ = qlora.forward(w, x, aa, bb, alpha)
        return float(np.sum(dy * y))

    h = 1e-6
    for arr, grad, which in ((a, da, 0), (b, db, 1)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            mm = arr.copy(); mm[idx] -= h
            args_p = (p, b) if which == 0 else (a, p)
            args_m = (mm, b) if which == 0 else (a, mm)
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7)


def _bf16_vals(rng, shape, scale):
    return nf4.bf16_bits_to_f32(nf4.bf16_rne_bits((rng.standard_normal(shape) * scale).astype(np.float32)))


def _bf16_nearest_exact(v):
    """The bf16 nearest the rational v (ties to even), as (value, distance of v
    from the nearest rounding boundary relative to |v|): written from the
    definition on Fractions, independent of the oracle's float64 rounding."""
    from fractions import Fraction
    if v == 0:
        return Fraction(0), Fraction(1)
    mag = abs(v)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    while Fraction(2) ** e > mag:
        e -= 1
    while Fraction(2) ** (e + 1) <= mag:
        e += 1
    ulp = Fraction(2) ** (e - 7)                       # 8 significant bits
    q = mag / ulp
    fl = q.numerator // q.denominator
    frac = q - fl
    up = frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1)
    val = (fl + (1 if up else 0)) * ulp
    boundary_gap = abs(frac - Fraction(1, 2)) * ulp / mag
    return (val if v > 0 else -val), boundary_gap


def _bits_value(bits):
    from fractions import Fraction
    return Fraction(float(nf4.bf16_bits_to_f32(np.array([bits], np.uint16))[0]))


def test_bf16_nearest_f64_is_the_nearest_value():
    from fractions import Fraction
    rng = np.random.default_rng(10)
    vals = list(rng.standard_normal(3000) * 0.03) + list(rng.standard_normal(500) * 1e5)
    # exact ties (a bf16 value plus half its ulp) and their neighbours one fp64 ulp away
    for m in range(128, 256, 7):
        for e in (-20, -3, 0, 9):
            t = (m + 0.5) * 2.0 ** (e - 7)
            vals += [t, -t, np.nextafter(t, 0.0), np.nextafter(t, np.inf)]
    vals += [0.0, -0.0, 2.0 ** -126, 1.0, 255.5 * 2.0 ** -7]
    bits = nf4.bf16_nearest_bits_f64(np.array(vals, np.float64))
    for v, b in zip(vals, bits):
        want, _ = _bf16_nearest_exact(Fraction(v))
        assert _bits_value(b) == want, v
        assert (int(b) >> 15) == int(np.signbit(v))
    # on fp32 inputs it is the fp32 -> bf16 round to nearest even
    f = (rng.standard_normal(4000) * 0.1).astype(np.float32)
    assert np.array_equal(nf4.bf16_nearest_bits_f64(f.astype(np.float64)), nf4.bf16_rne_bits(f))


def test_merged_bf16_rank_one_by_brute_force():
    """r = 1: every element by hand in exact rationals, rounded once to bf16
    (ties to even); the oracle's vectorised fp64 form must agree bit for bit,
    ties included: here its fp64 value is the exact one (checked), so it meets
    the same ties."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    d, k, alpha = 5, 7, 3.0
    base = nf4.bf16_rne_bits((rng.standard_normal((d, k)) * 0.02).astype(np.float32))
    a, b = _bf16_vals(rng, (1, k), 1.0), _bf16_vals(rng, (d, 1), 0.01)
    got = qlora.merged_weight_bf16(base, a, b, alpha)
    s = Fraction(float(np.float32(np.float32(alpha) / np.float32(1))))
    basef = nf4.bf16_bits_to_f32(base)
    for n in range(d):
        for c in range(k):
            exact = Fraction(float(basef[n, c])) + s * Fraction(float(b[n, 0])) * Fraction(float(a[0, c]))
            m = float(basef[n, c]) + float(s) * (float(b[n, 0]) * float(a[0, c]))
            assert Fraction(m) == exact
            want, _ = _bf16_nearest_exact(exact)
            assert _bits_value(got[n, c]) == want


def test_merged_bf16_is_one_rounding_of_the_exact_merge():
    """chkda "Merging LoRA weights for inference": W0 + (alpha/r) B A.  For
    r > 1 and a scale alpha/r that is not a power of two, merge and unmerge
    against the exact rational value of base + s sum_j B[n][j] A[j][k]
    (s = the fp32 alpha/r), rounded once to the nearest bf16: bit-equal
    wherever the exact value is not within 2^-40 (relative) of a rounding
    boundary."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    d, k, r, alpha = 12, 24, 5, 7.0
    base = nf4.bf16_rne_bits((rng.standard_normal((d, k)) * 0.02).astype(np.float32))
    a, b = _bf16_vals(rng, (r, k), 1.0 / np.sqrt(r)), _bf16_vals(rng, (d, r), 0.01)
    s = Fraction(float(np.float32(np.float32(alpha) / np.float32(r))))
    assert s != Fraction(7, 5)                              # the fp32 scale, not the real 7/5
    basef = nf4.bf16_bits_to_f32(base)
    for sign in (1, -1):
        got = qlora.merged_weight_bf16(base, a, b, alpha, sign=float(sign))
        skipped = 0
        for n in range(d):
            for c in range(k):
                acc = sum(Fraction(float(b[n, j])) * Fraction(float(a[j, c])) for j in range(r))
                exact = Fraction(float(basef[n, c])) + sign * s * acc
                want, gap = _bf16_nearest_exact(exact)
                if gap <= 2.0 ** -40:
                    skipped += 1
                    continue
                assert _bits_value(got[n, c]) == want, (sign, n, c)
        assert skipped <= 2


def test_merged_bf16_is_the_rounded_exact_merge():
    """Against the plain fp64 merge (BLAS product): within half a bf16 ulp, and
    equal to the single rounding of it to bf16 wherever it is not within 2^-40
    of a rounding boundary."""
    rng = np.random.default_rng(12)
    d, k, r, alpha = 48, 64, 16, 32.0
    base = nf4.bf16_rne_bits((rng.standard_normal((d, k)) * 0.02).astype(np.float32))
    a, b = _bf16_vals(rng, (r, k), 1.0 / np.sqrt(r)), _bf16_vals(rng, (d, r), 0.01)
    got = nf4.bf16_bits_to_f32(qlora.merged_weight_bf16(base, a, b, alpha)).astype(np.float64)
    ref = qlora.merged_weight(nf4.bf16_bits_to_f32(base), a, b, alpha)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # distance of ref from the nearest bf16 rounding boundary, relative
    u = np.abs(ref).view(np.uint64)
    frac = (u & np.uint64((1 << 45) - 1)).astype(np.float64) / float(1 << 45)
    far = np.abs(frac - 0.5) > 2.0 ** -30
    direct = nf4.bf16_bits_to_f32(nf4.bf16_nearest_bits_f64(ref)).astype(np.float64)
    assert far.mean() > 0.99 and np.array_equal(got[far], direct[far])


def test_merge_of_a_zero_adapter_and_exact_unmerge():
    rng = np.random.default_rng(13)
    d, k, r = 8, 16, 4
    base = nf4.bf16_rne_bits((rng.standard_normal((d, k)) * 0.02).astype(np.float32))
    a = _bf16_vals(rng, (r, k), 1.0)
    # B = 0: the merge returns the base (signed zeros become +0: -0 + +0 = +0)
    m0 = qlora.merged_weight_bf16(base, a, np.zeros((d, r)), 16.0)
    canon = np.where(base == 0x8000, np.uint16(0), base)
    assert np.array_equal(m0, canon)
    # an adapter whose products and sums are exact in bf16 (powers of two on a
    # coarse grid): merge then unmerge gives the base back bit for bit
    base2 = nf4.bf16_rne_bits(np.round(rng.standard_normal((d, k)) * 8).astype(np.float32) / 8)
    a2 = np.where(rng.random((r, k)) < 0.5, 0.5, -0.25)
    b2 = np.where(rng.random((d, r)) < 0.5, 1.0, 0.0)
    m = qlora.merged_weight_bf16(base2, a2, b2, float(r))  # s = 1
    back = qlora.merged_weight_bf16(m, a2, b2, float(r), sign=-1.0)
    assert np.array_equal(np.where(back == 0x8000, np.uint16(0), back),
                          np.where(base2 == 0x8000, np.uint16(0), base2))


def test_bf16_output_allowance_is_the_references_own_rounding():
    """The GPU tests' per-element allowance for bf16 outputs: the reference
    rounded once to bf16 passes; one bf16 ulp more on one heavy-tailed element
    fails; and without the flag the strict bound applies."""
    import pytest
    from tests.helpers import assert_close, bf16_rounding_error
    rng = np.random.default_rng(40)
    ref = rng.standard_normal(4096)
    ref[7] = 60.0 + 1.0 / 3.0                            # heavy tail: its bf16 rounding exceeds 2e-2 rms
    rounded = nf4.bf16_bits_to_f32(nf4.bf16_nearest_bits_f64(ref)).astype(np.float64)
    assert np.array_equal(bf16_rounding_error(ref), np.abs(rounded - ref))
    assert_close(rounded, ref, "rounded", bf16_output=True)
    with pytest.raises(AssertionError):
        assert_close(rounded, ref, "rounded, strict")     # 60.33 -> 60.25: 0.083 > 2e-2 rms
    bumped = rounded.copy()
    bumped[7] += 0.25 * 2                                 # one bf16 ulp at 60 is 0.25: two ulps off
    with pytest.raises(AssertionError):
        assert_close(bumped, ref, "bumped", bf16_output=True)
