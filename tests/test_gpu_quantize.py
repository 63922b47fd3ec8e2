"""GPU parity: NF4 quantize + double quantization and the standalone
doubleDequant, bit-exact against the CPU oracle (codes, packed bytes, c2, c1,
mean, bf16 weights)."""
import numpy as np
import pytest
import torch

from oracle import nf4
from tests.helpers import bf16_to_host_bits, say, to_dev_f32
from workloads import WORKLOADS, random_weights, workload_layer

pytestmark = pytest.mark.gpu


def gpu_quantize(w0: np.ndarray):
    import bit_nf4_quantized_13_amd as q
    w = q.qlora_nf4_quantize(to_dev_f32(w0))
    what = q.qlora_nf4_dequantize(w)
    torch.cuda.synchronize()
    return {"packed": w.codes.cpu().numpy(), "c2": w.absmax_q.cpu().numpy(),
            "c1": w.absmax_scale.cpu().numpy(), "mean": w.absmax_mean.cpu().numpy()[0],
            "what": bf16_to_host_bits(what)}, w


def assert_bit_exact(w0: np.ndarray, name: str):
    say(f"quantize+dequantize {name} shape={w0.shape}")
    got, _ = gpu_quantize(w0)
    ref = nf4.quantize(w0)
    assert np.array_equal(got["packed"], ref["packed"]), f"{name}: packed codes differ"
    assert np.array_equal(got["c2"], ref["c2"]), f"{name}: c2 differs"
    assert np.array_equal(got["c1"].view(np.uint32), ref["c1"].view(np.uint32)), f"{name}: c1 differs"
    assert np.float32(got["mean"]).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), name
    want = nf4.dequantize(ref, w0.shape)
    assert np.array_equal(got["what"], want), f"{name}: dequantized bf16 differs"


def test_codebook_table_matches_oracle():
    import bit_nf4_quantized_13_amd as q
    assert np.array_equal(np.array(q.qlora_nf4_codebook(), np.float32).view(np.uint32),
                          nf4.nf4_codebook().view(np.uint32))


def test_single_layer_workload():
    assert_bit_exact(workload_layer("single").w0, "single 256x512")


@pytest.mark.parametrize("shape", [(1, 64), (3, 64), (1, 64 * 255), (1, 64 * 257), (37, 64 * 300),
                                   (8, 4096), (64, 1088)])
def test_shapes_and_ragged_groups(shape):
    assert_bit_exact(random_weights(11, shape), f"random {shape}")


def test_layer4096_full():
    assert_bit_exact(workload_layer("layer4096").w0, "layer4096 4096x4096")


@pytest.mark.parametrize("proj", [0, 1])
def test_decode_workload_weights(proj):
    """Both weights of the decode workload (4096x4096 and 14336x4096, seed 2):
    codes, bytes, c2, c1, mean and bf16 weights bit-exact."""
    wl = WORKLOADS["decode"]
    assert_bit_exact(workload_layer("decode", proj).w0, f"decode {wl.projections[proj].name}")


def test_zero_blocks_zero_groups_and_zero_tensor():
    w = random_weights(12, (16, 64 * 64))
    w[0, :64] = 0.0                   # one all-zero block
    w[4:8, :] = 0.0                   # whole DQ group of zero blocks
    w[9, 64:128] = -0.0
    assert_bit_exact(w, "zero blocks")
    assert_bit_exact(np.zeros((8, 512), np.float32), "all-zero tensor")


def test_ties_signed_zeros_and_subnormals():
    c = nf4.nf4_codebook().astype(np.float64)
    mids = ((c[:-1] + c[1:]) / 2).astype(np.float32)
    w = random_weights(13, (4, 64 * 8))
    blk = w.reshape(-1, 64)
    blk[0, :] = 0.0
    blk[0, 0] = 1.0
    blk[0, 1:16] = mids                          # exact (representable) midpoints, scale 1
    blk[0, 16:31] = np.nextafter(mids, np.float32(2))
    blk[0, 31:46] = np.nextafter(mids, np.float32(-2))
    blk[1, :] = 0.0
    blk[1, 0] = 2.0
    blk[1, 1] = 0.32                             # the pages' worked example
    blk[2, :] *= np.float32(1e-38)               # subnormal weights
    blk[3, :] = -0.0
    blk[3, 5] = 3e-45
    blk[4, :] = np.float32(-0.5)                 # constant negative block
    assert_bit_exact(w, "ties / zeros / subnormals")


def test_wide_dynamic_range_of_scales():
    w = random_weights(14, (64, 64 * 64))
    w *= np.logspace(-6, 3, w.shape[0], dtype=np.float32)[:, None]
    assert_bit_exact(w, "scales over 9 decades")


def test_determinism():
    w0 = random_weights(15, (512, 1024))
    a, _ = gpu_quantize(w0)
    b, _ = gpu_quantize(w0)
    for key in a:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key
