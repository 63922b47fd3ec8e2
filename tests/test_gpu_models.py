"""GPU parity on the two model-layer workloads at their full sizes: every
projection of the 7B-style layer (M = 2048, r = 64) and of the 65B-style layer
(M = 4096, r = 64).

- quantize + doubleDequant of the full weight: bit-exact (codes, c2, c1, mean,
  bf16 weights);
- Y and dX on sampled token rows (both are row-separable; the oracle's fp64
  products over all rows would take minutes), U, dA and dB in full; all within
  relative Frobenius <= 5e-3 and max |diff| <= 2e-2 rms(ref).
"""
import numpy as np
import pytest
import torch

from oracle import nf4, qlora
from tests.helpers import assert_close, bf16_to_host_bits, bf16_to_host_f64, say, to_dev_bf16, to_dev_f32
from workloads import WORKLOADS, bf16_bits_as_f32, workload_layer

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROWS = 96  # sampled token rows for Y and dX


def cases():
    for name in ("llama7b", "llama65b"):
        for i, p in enumerate(WORKLOADS[name].projections):
            yield pytest.param(name, i, id=f"{name}-{p.name}-{p.d}x{p.k}")


@pytest.mark.parametrize("name,proj", list(cases()))
def test_model_projection(name, proj):
    import bit_nf4_quantized_13_amd as q
    wl = WORKLOADS[name]
    p = wl.projections[proj]
    m = wl.m[0]
    say(f"{name} {p.name} {p.d}x{p.k} M={m} r={wl.r}: generating inputs")
    inp = workload_layer(name, proj)
    rows = np.sort(np.random.default_rng(np.random.SeedSequence([wl.seed, proj, 7])).choice(m, ROWS, replace=False))

    say(f"{name} {p.name}: GPU quantize, dequantize, fwd, bwd")
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    what = q.qlora_nf4_dequantize(w)
    xd, ad, bd, dyd = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    y, u = q.qlora_linear_fwd(w, xd, ad, bd, wl.alpha)
    dx, da, db = q.qlora_linear_bwd(w, xd, dyd, ad, bd, wl.alpha, u=u)
    torch.cuda.synchronize()
    rt = torch.from_numpy(rows).cuda()
    got = {"packed": w.codes.cpu().numpy(), "c2": w.absmax_q.cpu().numpy(),
           "c1": w.absmax_scale.cpu().numpy(), "mean": w.absmax_mean.cpu().numpy()[0],
           "what": bf16_to_host_bits(what), "y": bf16_to_host_f64(y[rt]), "dx": bf16_to_host_f64(dx[rt]),
           "u": u.cpu().numpy().astype(np.float64), "da": da.cpu().numpy().astype(np.float64),
           "db": db.cpu().numpy().astype(np.float64)}
    del w, what, xd, ad, bd, dyd, y, u, dx, da, db
    torch.cuda.empty_cache()

    say(f"{name} {p.name}: oracle")
    ref = nf4.quantize(inp.w0)
    assert np.array_equal(got["packed"], ref["packed"]), "packed codes differ"
    assert np.array_equal(got["c2"], ref["c2"]), "c2 differs"
    assert np.array_equal(got["c1"].view(np.uint32), ref["c1"].view(np.uint32)), "c1 differs"
    assert np.float32(got["mean"]).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), "mean differs"
    w_hat_bits = nf4.dequantize(ref, inp.w0.shape)
    assert np.array_equal(got["what"], w_hat_bits), "dequantized bf16 differs"
    w_hat = nf4.bf16_bits_to_f32(w_hat_bits).reshape(p.d, p.k)
    del ref, w_hat_bits

    x = bf16_bits_as_f32(inp.x)
    dy = bf16_bits_as_f32(inp.dy)
    a, b = bf16_bits_as_f32(inp.a), bf16_bits_as_f32(inp.b)
    y_ref, _ = qlora.forward(w_hat, x[rows], a, b, wl.alpha)
    assert_close(got["y"], y_ref, f"{name} {p.name} Y (rows)")
    assert_close(got["u"], qlora.lora_down(x, a), f"{name} {p.name} U")
    dx_ref, _, _ = qlora.backward(w_hat, x[rows], dy[rows], a, b, wl.alpha)
    assert_close(got["dx"], dx_ref, f"{name} {p.name} dX (rows)")
    da_ref, db_ref = qlora.adapter_grads(x, dy, a, b, wl.alpha)
    assert_close(got["da"], da_ref, f"{name} {p.name} dA")
    assert_close(got["db"], db_ref, f"{name} {p.name} dB")
