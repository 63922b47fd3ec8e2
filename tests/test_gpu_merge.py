"""GPU parity of the adapter merge / unmerge (qlora_adapter_merge,
qlora_adapter_unmerge) against the oracle's merged_weight_bf16: bit for bit,
including ragged tiles (d not a multiple of 64, k not a multiple of 256),
ranks across several 32-rank chunks, and the layer4096 weight."""
import numpy as np
import pytest
import torch

from oracle import nf4, qlora
from tests.helpers import bf16_to_host_bits, say, to_dev_bf16, to_dev_f32
from workloads import bf16_bits_as_f32, make_layer, workload_layer

pytestmark = pytest.mark.gpu


def run_merge(inp, alpha):
    import bit_nf4_quantized_13_amd as q
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    ad, bd = to_dev_bf16(inp.a), to_dev_bf16(inp.b)
    merged = q.qlora_adapter_merge(w, ad, bd, alpha)
    back = q.qlora_adapter_unmerge(merged, ad, bd, alpha)
    inplace = merged.clone()
    q.qlora_adapter_unmerge(inplace, ad, bd, alpha, out=inplace)
    what = q.qlora_nf4_dequantize(w)
    torch.cuda.synchronize()
    return (bf16_to_host_bits(merged), bf16_to_host_bits(back), bf16_to_host_bits(inplace),
            bf16_to_host_bits(what))


def check(inp, alpha, name):
    say(f"merge {name}")
    got_m, got_b, got_i, what = run_merge(inp, alpha)
    ref = nf4.quantize(inp.w0)
    what_ref = nf4.dequantize(ref, inp.w0.shape)
    assert np.array_equal(what, what_ref), "dequantized weight differs"
    a, b = bf16_bits_as_f32(inp.a), bf16_bits_as_f32(inp.b)
    want_m = qlora.merged_weight_bf16(what_ref, a, b, alpha)
    assert np.array_equal(got_m, want_m), f"{name}: merge differs at {np.argwhere(got_m != want_m)[:5]}"
    want_b = qlora.merged_weight_bf16(want_m, a, b, alpha, sign=-1.0)
    assert np.array_equal(got_b, want_b), f"{name}: unmerge differs"
    assert np.array_equal(got_i, want_b), f"{name}: in-place unmerge differs"


@pytest.mark.parametrize("d,k,r,alpha", [(256, 512, 8, 16.0), (200, 1088, 33, 16.0), (64, 64, 1, 1.0),
                                         (520, 320, 128, 32.0), (8, 256, 5, 7.0)])
def test_merge_shapes(d, k, r, alpha):
    check(make_layer(31, r, d, k, 4, r), alpha, f"d={d} k={k} r={r}")


def test_merge_zero_adapter_returns_the_dequantized_weight():
    import bit_nf4_quantized_13_amd as q
    inp = make_layer(32, 0, 128, 256, 4, 8)
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    merged = q.qlora_adapter_merge(w, to_dev_bf16(inp.a), torch.zeros((128, 8), dtype=torch.bfloat16,
                                                                          device="cuda"), 16.0)
    what = q.qlora_nf4_dequantize(w)
    m, wb = bf16_to_host_bits(merged), bf16_to_host_bits(what)
    canon = np.where(wb == 0x8000, np.uint16(0), wb)  # -0 + +0 = +0
    assert np.array_equal(m, canon)


def test_merge_layer4096():
    inp = workload_layer("layer4096")
    check(inp, 16.0, "layer4096 4096x4096 r=8")
