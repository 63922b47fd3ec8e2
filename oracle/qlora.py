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

Adapter dropout (fromzero2ai "Python Implementation: Fine-Tuning with PEFT
and BitsAndBytes" trains with a LoRA dropout rate of 0.05; chkda "Merging LoRA
weights for inference" notes the two-path form equals the merged one only with
dropout disabled).  Reading R17: dropout acts on the adapter's input only,

    Xd = drop(X)                   [M x k]  (bf16: x c kept, +0 dropped)
    U  = Xd A^T,   Y = X What^T + s U B^T
    dA = s G^T Xd, dB = s dY^T U,  dX = dY What + c (M o (s G A))

with c = fl32(1 / fl32(1 - p)) and the keep mask M drawn by Philox4x32-10
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011) from a 64-bit seed: element i = m k + col uses word i mod 4 of the
block for counter (i div 4 as two 32-bit words, 0, 0) and key (seed low, seed
high); it is dropped iff that word < floor(p 2^32).  The pages fix only the
rate p (0.05 in fromzero2ai's configuration); comparing a full 32-bit word
resolves the fp32 value of p to 2^-32, so the realised rate is
floor(p 2^32) / 2^32.

Merge (chkda "Merging LoRA weights for inference"): W_merged = W0 + s B A,
in fp64 (merged_weight) and as bf16 (merged_weight_bf16, reading R14: the
sum computed in fp64, then one rounding to the nearest bf16).
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
    """bf16 bits of base + sign (alpha/r) B A (chkda "Merging LoRA weights for
    inference" gives W0 + (alpha/r) B A and leaves the arithmetic open; reading
    R14): the value computed in fp64, then rounded once to the nearest bf16,

        S = sum over j = 0 .. r-1, ascending, of B[:, j] A[j, :]   (fp64; each
            product of two bf16 values is exact, so each step is one rounding)
        m = base + s S                                               (fp64)
        out = the bf16 nearest m, ties to even                       (one rounding)

    with s the fp32 value of alpha / r, the layer's scale (alpha arrives as
    fp32).  Away from bf16 rounding boundaries this is the exact merge rounded
    once.  base_bits: uint16 bf16 patterns [d x k] -- What for a merge
    (sign = +1), the merged weight for an unmerge (sign = -1)."""
    from .nf4 import bf16_bits_to_f32, bf16_nearest_bits_f64
    a, b = _f64(a), _f64(b)
    r = a.shape[0]
    s = np.float64(np.float32(np.float32(alpha) / np.float32(r))) * np.float64(sign)
    acc = np.zeros((b.shape[0], a.shape[1]), dtype=np.float64)
    for j in range(r):
        acc += np.outer(b[:, j], a[j, :])
    m = bf16_bits_to_f32(base_bits).astype(np.float64) + s * acc
    return bf16_nearest_bits_f64(m)


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


# ----------------------------------------------------------------------------
# adapter dropout (reading R17)
# ----------------------------------------------------------------------------
PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # Philox4x32 round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # Philox4x32 key increments (Weyl sequence)


def philox4x32_10(ctr: np.ndarray, key: tuple[int, int]) -> np.ndarray:
    """Philox4x32 with 10 rounds on an array of counters [n x 4] (uint32).

    A round multiplies counter words 0 and 2 by the two constants (64-bit
    products), and the new counter is (hi(w2 M1) ^ c1 ^ k0, lo(w2 M1),
    hi(w0 M0) ^ c3 ^ k1, lo(w0 M0)); the key gains the Weyl increments
    between rounds.  Returns [n x 4] uint32.
    """
    c = [np.asarray(ctr, dtype=np.uint64)[:, i].copy() for i in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    lo32 = np.uint64(0xFFFFFFFF)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
        p0 = c[0] * np.uint64(PHILOX_M[0])
        p1 = c[2] * np.uint64(PHILOX_M[1])
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & lo32,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & lo32]
    return np.stack(c, axis=1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """floor(p 2^32) for the fp32 value of p in [0, 1) (exact: p 2^32 is a
    power-of-two scaling of an fp32 value)."""
    p = float(np.float32(p))
    assert 0.0 <= p < 1.0
    return int(np.floor(p * 2.0 ** 32))


def dropout_scale(p: float) -> np.float32:
    """c = fl32(1 / fl32(1 - p)), the inverse keep probability."""
    return np.float32(np.float32(1.0) / np.float32(np.float32(1.0) - np.float32(p)))


def dropout_keep_mask(m: int, k: int, p: float, seed: int) -> np.ndarray:
    """Keep mask [m x k] (bool) of reading R17."""
    n = m * k
    blocks = np.arange((n + 3) // 4, dtype=np.uint64)
    ctr = np.zeros((blocks.size, 4), dtype=np.uint64)
    ctr[:, 0] = blocks & np.uint64(0xFFFFFFFF)
    ctr[:, 1] = blocks >> np.uint64(32)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(-1)[:n]
    return (words.astype(np.int64) >= dropout_threshold(p)).reshape(m, k)


def lora_dropout_bits(x_bits: np.ndarray, p: float, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Xd as bf16 bits: bf16(fl32(x c)) where kept, +0 where dropped; and the mask."""
    from .nf4 import bf16_bits_to_f32, bf16_rne_bits
    m, k = x_bits.shape
    keep = dropout_keep_mask(m, k, p, seed)
    xs = (bf16_bits_to_f32(x_bits) * dropout_scale(p)).astype(np.float32)   # one fp32 rounding
    out = bf16_rne_bits(xs)
    out[~keep] = 0
    return out, keep


def forward_dropout(w_hat, x, xd, a, b, alpha: float) -> tuple[np.ndarray, np.ndarray]:
    """(Y, U) with dropout on the adapter input: U = Xd A^T, Y = X What^T + s U B^T."""
    w_hat, x, xd, a, b = _f64(w_hat), _f64(x), _f64(xd), _f64(a), _f64(b)
    s = adapter_scale(alpha, a.shape[0])
    u = xd @ a.T
    return x @ w_hat.T + s * (u @ b.T), u


def backward_dropout(w_hat, xd, keep, dy, a, b, alpha: float, p: float):
    """(dX, dA, dB) of forward_dropout (keep: the mask, c = dropout_scale(p))."""
    w_hat, xd, dy, a, b = _f64(w_hat), _f64(xd), _f64(dy), _f64(a), _f64(b)
    s = adapter_scale(alpha, a.shape[0])
    c = float(dropout_scale(p))
    u = xd @ a.T
    g = dy @ b
    dx = dy @ w_hat + c * np.where(keep, s * (g @ a), 0.0)
    return dx, s * (g.T @ xd), s * (dy.T @ u)
