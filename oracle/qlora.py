"""The QLoRA linear layer, forward and backward, in float64 -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forward (chkda "How does it work?"; fromzero2ai "Low-Rank Matrix
Factorization"): h = W0 x + (alpha/r) B (A x), with W0 [d x k], A [r x k],
B [d x r] and no bias.  In the batched row-vector form of chkda "Double
quantization and double dequantization" (Y = X doubleDequant(...) + X L1 L2,
with L1 = A^T, L2 = B^T and the scale made explicit) the rows of X [M x k]
are inputs:

    U  = X A^T                     [M x r]
    Y  = X What^T + s U B^T        [M x d],   s = alpha / r

What is the double-dequantized bf16 weight (widened exactly), never the
original W0, so a comparison measures kernel error and not quantization error.

Backward (chkda: gradients flow through the reconstructed base weights into
the adapters only; the 4-bit weights get no update; alpha/r also scales the
adapter gradients, "How does alpha/r control adapter strength?").  With the
upstream gradient dY [M x d] of a loss L(Y):

    G  = dY B                      [M x r]
    dX = dY What + s G A           [M x k]
    dA = s G^T X                   [r x k]
    dB = s dY^T U                  [d x r]

There is no dW.  These are the closed-form derivatives of Y above; the tests
pin them with central finite differences.

Merge (chkda "Merging LoRA weights for inference"): W_merged = W0 + s B A,
in fp64 (merged_weight) and as bf16 under the library's fixed rounding
(merged_weight_bf16, reading R14: the sum over ranks in fp64 in ascending
order, two fp64 roundings, then fp32 and bf16 to nearest even).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def adapter_scale(alpha: float, r: int) -> float:
    """s = alpha / r (chkda "How does alpha/r control adapter strength?")."""
    return float(alpha) / float(r)


def lora_down(x, a) -> np.ndarray:
    """U = X A^T: the adapter's first projection (A acts first)."""
    return _f64(x) @ _f64(a).T


def forward(w_hat, x, a, b, alpha: float) -> tuple[np.ndarray, np.ndarray]:
    """Returns (Y, U) in float64."""
    w_hat, x, a, b = _f64(w_hat), _f64(x), _f64(a), _f64(b)
    s = adapter_scale(alpha, a.shape[0])
    u = x @ a.T
    y = x @ w_hat.T + s * (u @ b.T)
    return y, u


def backward(w_hat, x, dy, a, b, alpha: float) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (dX, dA, dB) in float64; W0 is frozen and gets no gradient."""
    w_hat, x, dy, a, b = _f64(w_hat), _f64(x), _f64(dy), _f64(a), _f64(b)
    s = adapter_scale(alpha, a.shape[0])
    u = x @ a.T
    g = dy @ b
    dx = dy @ w_hat + s * (g @ a)
    da = s * (g.T @ x)
    db = s * (dy.T @ u)
    return dx, da, db


def adapter_grads(x, dy, a, b, alpha: float) -> tuple[np.ndarray, np.ndarray]:
    """(dA, dB) of backward() without its dX product, for shapes whose full dX
    is too large to form on the host: dA = s (dY B)^T X, dB = s dY^T (X A^T)."""
    x, dy, a, b = _f64(x), _f64(dy), _f64(a), _f64(b)
    s = adapter_scale(alpha, a.shape[0])
    return s * ((dy @ b).T @ x), s * (dy.T @ (x @ a.T))


def merged_weight(w_hat, a, b, alpha: float) -> np.ndarray:
    """W_merged = W0 + (alpha/r) B A (chkda "Merging LoRA weights for inference")."""
    a, b = _f64(a), _f64(b)
    return _f64(w_hat) + adapter_scale(alpha, a.shape[0]) * (b @ a)


def merged_weight_bf16(base_bits, a, b, alpha: float, sign: float = 1.0) -> np.ndarray:
    """bf16 bits of base + sign (alpha/r) B A with the merge's fixed rounding
    (chkda "Merging LoRA weights for inference" gives W0 + (alpha/r) B A and
    leaves the arithmetic open; reading R14):

        S = sum over j = 0 .. r-1, ascending, of B[:, j] A[j, :]   (fp64; each
            product of two bf16 values is exact, so each step is one rounding)
        t = s S,  m = base + t                                       (fp64, two roundings)
        out = bf16(fp32(m))                                          (nearest even, twice)

    with s = fp32(alpha / r) as the library computes it.  base_bits: uint16 bf16
    patterns [d x k] -- What for a merge (sign = +1), the merged weight for an
    unmerge (sign = -1)."""
    from .nf4 import bf16_bits_to_f32, bf16_rne_bits
    a, b = _f64(a), _f64(b)
    r = a.shape[0]
    s = np.float64(np.float32(np.float32(alpha) / np.float32(r))) * np.float64(sign)
    acc = np.zeros((b.shape[0], a.shape[1]), dtype=np.float64)
    for j in range(r):
        acc += np.outer(b[:, j], a[j, :])
    m = bf16_bits_to_f32(base_bits).astype(np.float64) + s * acc
    return bf16_rne_bits(m.astype(np.float32))


def trainable_parameters(d: int, k: int, r: int) -> int:
    """(r x k) + (d x r): the adapter's parameter count (fromzero2ai "Why Does
    This Save Memory?")."""
    return r * k + d * r


def forward_flops(m: int, d: int, k: int, r: int) -> int:
    """Algorithmic flops of the forward: base GEMM plus the two adapter GEMMs."""
    return 2 * m * d * k + 2 * m * r * (d + k)


def backward_flops(m: int, d: int, k: int, r: int) -> int:
    """dX base GEMM plus G, s G A, dA and dB (U is saved by the forward)."""
    return 2 * m * d * k + 4 * m * r * (d + k)
