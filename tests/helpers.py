"""Shared helpers of the GPU parity tests (host-side comparison logic only)."""
from __future__ import annotations

import sys

import numpy as np

from oracle import nf4, qlora
from workloads import bf16_bits_as_f32

REL_FRO_TOL = 5e-3      # relative Frobenius error bound for GEMM outputs and gradients
MAX_ABS_TOL = 2e-2      # max |out - ref| <= MAX_ABS_TOL * rms(ref)


def say(msg: str) -> None:
    """Name the case before a GPU step so a fault is attributable."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_to_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_host_f64(t) -> np.ndarray:
    return bf16_bits_as_f32(bf16_to_host_bits(t)).astype(np.float64)


def bf16_rounding_error(ref: np.ndarray) -> np.ndarray:
    """|bf16(ref) - ref| per element: ref (fp64) rounded once to the nearest
    bf16.  Magnitudes below the bf16 normal range count as 0 (their rounding
    error is under 2^-133)."""
    ref = np.asarray(ref, dtype=np.float64)
    normal = np.abs(ref) >= 2.0 ** -126
    src = np.where(normal, ref, 0.0)
    rounded = nf4.bf16_bits_to_f32(nf4.bf16_nearest_bits_f64(src)).astype(np.float64)
    return np.where(normal, np.abs(rounded - src), 0.0)


def assert_close(out: np.ndarray, ref: np.ndarray, what: str,
                 rel_tol: float = REL_FRO_TOL, abs_tol: float = MAX_ABS_TOL,
                 bf16_output: bool = False) -> dict:
    """Relative Frobenius <= rel_tol and max |out - ref| <= abs_tol * rms(ref).

    bf16_output (only for outputs stored in bf16): the per-element bound
    becomes abs_tol * rms(ref) + |bf16(ref) - ref|, where bf16(ref) is the
    reference itself rounded once to the nearest bf16 -- the part of the error
    that no bf16 output can avoid, element by element.  Elements whose own
    rounding is zero keep the plain bound.
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (what, out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    diff = out - ref
    nref = np.linalg.norm(ref)
    rms = nref / np.sqrt(ref.size) if ref.size else 0.0
    if nref == 0:
        assert np.all(out == 0), f"{what}: reference is exactly zero, output is not"
        return {"rel_fro": 0.0, "max_abs_over_rms": 0.0}
    rel = np.linalg.norm(diff) / nref
    mx = np.abs(diff).max() / rms
    assert rel <= rel_tol, f"{what}: relative Frobenius error {rel:.3e} > {rel_tol}"
    if bf16_output:
        excess = np.abs(diff) - (abs_tol * rms + bf16_rounding_error(ref))
        assert excess.max() <= 0, (f"{what}: max abs error {mx:.3e} x rms(ref) beyond "
                                   f"{abs_tol} x rms(ref) + the reference's own bf16 rounding")
    else:
        assert mx <= abs_tol, f"{what}: max abs error {mx:.3e} x rms(ref) > {abs_tol}"
    return {"rel_fro": float(rel), "max_abs_over_rms": float(mx)}


class OracleLayer:
    """The oracle's view of one layer: its own quantization of W0 and What."""

    def __init__(self, w0: np.ndarray):
        self.d, self.k = w0.shape
        self.q = nf4.quantize(w0)
        self.w_hat_bits = nf4.dequantize(self.q, (self.d, self.k))
        self.w_hat = nf4.bf16_bits_to_f32(self.w_hat_bits).reshape(self.d, self.k)

    def forward(self, x_bits, a_bits, b_bits, alpha):
        return qlora.forward(self.w_hat, bf16_bits_as_f32(x_bits), bf16_bits_as_f32(a_bits),
                             bf16_bits_as_f32(b_bits), alpha)

    def backward(self, x_bits, dy_bits, a_bits, b_bits, alpha):
        return qlora.backward(self.w_hat, bf16_bits_as_f32(x_bits), bf16_bits_as_f32(dy_bits),
                              bf16_bits_as_f32(a_bits), bf16_bits_as_f32(b_bits), alpha)
