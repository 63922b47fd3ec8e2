"""Python binding of libqlora_nf4.so -- the MI355X QLoRA NF4 linear layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory (outputs and workspaces are allocated
as torch tensors) and the current HIP stream.  There is no fallback: if the
library is not built, importing the binding raises.

Functions carry the C ABI's names (include/qlora_nf4.h):

    qlora_nf4_quantize(W0)                    -> NF4Weight
    qlora_nf4_dequantize(w)                   -> bf16 [d, k]
    qlora_linear_fwd(w, x, A, B, alpha)       -> (Y, U)
    qlora_linear_bwd(w, x, dY, A, B, alpha, U=None, need_dx=True) -> (dX, dA, dB)
    qlora_nf4_codebook(), qlora_nf4_thresholds()   (host only, no GPU needed)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

QLORA_OK, QLORA_EINVAL, QLORA_ENOTSUP, QLORA_EALIGN, QLORA_EWORKSPACE, QLORA_EHIP, QLORA_ESCRATCH = range(7)
BLOCK = 64
DQ_BLOCK = 256
NO_DQ = 0  # dq_block of the format without double quantization (fp32 absmax per block)
C2_INT8, C2_FP8_E4M3 = 0, 1  # c2_format: how the c2 bytes of a double-quantized weight encode values

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python bit_nf4_quantized_13_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)


class _CWeight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("absmax_mean", ctypes.c_void_p),
                ("d", ctypes.c_int64), ("k", ctypes.c_int64),
                ("block", ctypes.c_int32), ("dq_block", ctypes.c_int32),
                ("c2_format", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_WP = ctypes.POINTER(_CWeight)

_SIGS = {
    "qlora_abi_version": (ctypes.c_int, []),
    "qlora_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_nf4_thresholds": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_nf4_quantize_workspace": (_SZ, [_I64, _I64, _I32, _I32]),
    "qlora_nf4_quantize": (ctypes.c_int, [_P, _WP, _P, _SZ, _P]),
    "qlora_nf4_dequantize": (ctypes.c_int, [_WP, _P, _P]),
    "qlora_linear_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_fwd": (ctypes.c_int, [_WP, _P, _I64, _P, _P, _I32, ctypes.c_float, _P, _P, _P,
                                        _SZ, _P]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_WP, _P, _I64, _P, _P, _I32, ctypes.c_float, _P, _P, _P]),
    "qlora_linear_bwd": (ctypes.c_int, [_WP, _P, _P, _P, _P, _P, _I64, _I32, ctypes.c_float, _P,
                                        _P, _P, _P, _SZ, _P]),
    "qlora_linear_gemm_only": (ctypes.c_int, [_WP, _I32, _I32, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "qlora_time_next_kernel": (ctypes.c_int, [_I32, _P]),
    "qlora_wall_clock_khz": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32)]),
    "qlora_adapter_merge": (ctypes.c_int, [_WP, _P, _P, _I32, ctypes.c_float, _P, _P]),
    "qlora_adapter_unmerge": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, ctypes.c_float, _P, _P]),
    "qlora_lora_dropout": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_float, ctypes.c_uint64, _P, _P]),
    "qlora_linear_dropout_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "qlora_linear_fwd_dropout": (ctypes.c_int, [_WP, _P, _I64, _P, _P, _I32, ctypes.c_float, ctypes.c_float,
                                                ctypes.c_uint64, _P, _P, _P, _SZ, _P]),
    "qlora_linear_bwd_dropout": (ctypes.c_int, [_WP, _P, _P, _P, _P, _P, _I64, _I32, ctypes.c_float,
                                                ctypes.c_float, ctypes.c_uint64, _P, _P, _P, _P, _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    if not hasattr(_lib, _name):
        raise ImportError(f"{LIB_PATH} lacks {_name}: it predates its sources; rebuild it with "
                          "`python bit_nf4_quantized_13_amd/build.py`")
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class QloraError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {status_str(status)}")
        self.status = status


def status_str(status: int) -> str:
    return _lib.qlora_status_str(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != QLORA_OK:
        raise QloraError(status, call)


def library() -> ctypes.CDLL:
    """The loaded ctypes handle (for tests that call the C ABI directly)."""
    return _lib


def abi_version() -> int:
    return int(_lib.qlora_abi_version())


def qlora_nf4_codebook() -> list[float]:
    out = (ctypes.c_float * 16)()
    _check(_lib.qlora_nf4_codebook(out), "qlora_nf4_codebook")
    return list(out)


def qlora_nf4_thresholds() -> list[float]:
    out = (ctypes.c_float * 15)()
    _check(_lib.qlora_nf4_thresholds(out), "qlora_nf4_thresholds")
    return list(out)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev_tensor(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class NF4Weight:
    """Device buffers of one quantized W0 [d x k] (see qlora_nf4_weight).

    Double-quantized (dq_block == DQ_BLOCK): absmax_q holds c2, absmax_scale
    c1 per group of 256 blocks and absmax_mean the mean; c2_format says
    whether the c2 bytes are int8 values or OCP FP8 e4m3 bit patterns
    (absmax_q is then uint8; `.view(torch.float8_e4m3fn)` reads them).
    Without double quantization (dq_block == NO_DQ): absmax_scale holds the
    fp32 absmax of every block and absmax_q / absmax_mean are None.
    """
    codes: torch.Tensor                  # uint8 [d*k/2]
    absmax_q: torch.Tensor | None        # int8 or uint8 (e4m3 bits) [nb] (double-quantized only)
    absmax_scale: torch.Tensor           # float32 [G] (double-quantized) or [nb]
    absmax_mean: torch.Tensor | None     # float32 [1] (double-quantized only)
    d: int
    k: int
    block: int = BLOCK
    dq_block: int = DQ_BLOCK
    c2_format: int = C2_INT8

    @staticmethod
    def empty(d: int, k: int, device="cuda", double_quant: bool = True,
              c2_fp8: bool = False, block: int = BLOCK) -> "NF4Weight":
        """Uninitialised buffers for W0 [d, k] in blocks of `block` (64, 128 or 256) weights."""
        nb = (d * k) // block
        codes = torch.empty(d * k // 2, dtype=torch.uint8, device=device)
        if not double_quant:
            return NF4Weight(codes, None, torch.empty(nb, dtype=torch.float32, device=device), None,
                             d, k, block=block, dq_block=NO_DQ)
        g = -(-nb // DQ_BLOCK)
        return NF4Weight(codes, torch.empty(nb, dtype=torch.uint8 if c2_fp8 else torch.int8, device=device),
                         torch.empty(g, dtype=torch.float32, device=device),
                         torch.empty(1, dtype=torch.float32, device=device), d, k, block=block,
                         c2_format=C2_FP8_E4M3 if c2_fp8 else C2_INT8)

    @property
    def double_quant(self) -> bool:
        return self.dq_block != NO_DQ

    def c_struct(self) -> _CWeight:
        return _CWeight(self.codes.data_ptr(), _ptr(self.absmax_q),
                        self.absmax_scale.data_ptr(), _ptr(self.absmax_mean),
                        self.d, self.k, self.block, self.dq_block, self.c2_format)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.codes, self.absmax_q, self.absmax_scale, self.absmax_mean)
                   if t is not None)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def quantize_workspace_bytes(d: int, k: int, dq_block: int = DQ_BLOCK, block: int = BLOCK) -> int:
    return int(_lib.qlora_nf4_quantize_workspace(d, k, block, dq_block))


def linear_workspace_bytes(m: int, d: int, k: int, r: int, dropout: bool = False) -> int:
    if dropout:
        return int(_lib.qlora_linear_dropout_workspace(m, d, k, r))
    return int(_lib.qlora_linear_workspace(m, d, k, r))


def qlora_lora_dropout(x: torch.Tensor, p: float, seed: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Xd = dropout of bf16 x [M, k] on the adapter input (Philox keep mask of
    (p, seed); kept values x / (1 - p) rounded to bf16, dropped +0)."""
    _dev_tensor(x, torch.bfloat16, "x")
    m, k = x.shape
    xd = out if out is not None else torch.empty_like(x)
    _check(_lib.qlora_lora_dropout(x.data_ptr(), m, k, float(p), int(seed) & (2**64 - 1), xd.data_ptr(),
                                   _stream()), "qlora_lora_dropout")
    return xd


def qlora_nf4_quantize(w0: torch.Tensor, out: NF4Weight | None = None,
                       workspace: torch.Tensor | None = None,
                       double_quant: bool = True, c2_fp8: bool = False, block: int = BLOCK) -> NF4Weight:
    """NF4 in blocks of `block` weights (64, 128 or 256) (+ double quantization
    of the block absmax, c2 in int8 or, with c2_fp8, OCP FP8 e4m3) of fp32 W0
    [d, k] on the current stream.  With `out` given, its block, dq_block and
    c2_format decide the format."""
    _dev_tensor(w0, torch.float32, "W0")
    d, k = w0.shape
    w = out if out is not None else NF4Weight.empty(d, k, w0.device, double_quant, c2_fp8, block)
    ws_bytes = quantize_workspace_bytes(d, k, w.dq_block, w.block)
    ws = workspace if workspace is not None else _workspace(ws_bytes, w0.device)
    cw = w.c_struct()
    _check(_lib.qlora_nf4_quantize(w0.data_ptr(), ctypes.byref(cw), ws.data_ptr(),
                                   ws.numel(), _stream()), "qlora_nf4_quantize")
    return w


def qlora_nf4_dequantize(w: NF4Weight, out: torch.Tensor | None = None) -> torch.Tensor:
    """doubleDequant of W0 into bf16 [d, k]."""
    y = out if out is not None else torch.empty((w.d, w.k), dtype=torch.bfloat16,
                                                device=w.codes.device)
    cw = w.c_struct()
    _check(_lib.qlora_nf4_dequantize(ctypes.byref(cw), y.data_ptr(), _stream()),
           "qlora_nf4_dequantize")
    return y


def qlora_linear_fwd(w: NF4Weight, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                     alpha: float, save_u: bool = True, out: torch.Tensor | None = None,
                     u_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     dropout: float = 0.0, seed: int = 0):
    """Y = x What^T + (alpha/r) (x A^T) B^T.  Returns (Y bf16 [M, d], U fp32 [M, r] or None).

    dropout > 0: the adapter's input is Xd = drop(x) (qlora_lora_dropout with
    this seed), U = Xd A^T; the backward takes the same dropout and seed."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(a, torch.bfloat16, "A")
    _dev_tensor(b, torch.bfloat16, "B")
    m, r = x.shape[0], a.shape[0]
    y = out if out is not None else torch.empty((m, w.d), dtype=torch.bfloat16, device=x.device)
    if u_out is not None:
        u = _dev_tensor(u_out, torch.float32, "U")
    else:
        u = torch.empty((m, r), dtype=torch.float32, device=x.device) if save_u else None
    ws = workspace if workspace is not None else _workspace(
        linear_workspace_bytes(m, w.d, w.k, r, dropout > 0), x.device)
    cw = w.c_struct()
    if dropout > 0:
        _check(_lib.qlora_linear_fwd_dropout(ctypes.byref(cw), x.data_ptr(), m, a.data_ptr(), b.data_ptr(), r,
                                             float(alpha), float(dropout), int(seed) & (2**64 - 1), y.data_ptr(),
                                             _ptr(u), ws.data_ptr(), ws.numel(), _stream()),
               "qlora_linear_fwd_dropout")
        return y, u
    _check(_lib.qlora_linear_fwd(ctypes.byref(cw), x.data_ptr(), m, a.data_ptr(), b.data_ptr(), r,
                                 float(alpha), y.data_ptr(), _ptr(u), ws.data_ptr(), ws.numel(),
                                 _stream()), "qlora_linear_fwd")
    return y, u


def qlora_linear_fwd_noalloc(w: NF4Weight, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                             alpha: float, out: torch.Tensor, u_out: torch.Tensor | None = None):
    """The decode-shaped forward (M <= 16) through qlora_linear_fwd_noalloc: no
    workspace and no allocation in the call (the caller passes Y, and U if
    wanted).  Returns (Y, U or None)."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(a, torch.bfloat16, "A")
    _dev_tensor(b, torch.bfloat16, "B")
    _dev_tensor(out, torch.bfloat16, "Y")
    if u_out is not None:
        _dev_tensor(u_out, torch.float32, "U")
    cw = w.c_struct()
    _check(_lib.qlora_linear_fwd_noalloc(ctypes.byref(cw), x.data_ptr(), x.shape[0], a.data_ptr(), b.data_ptr(),
                                         a.shape[0], float(alpha), out.data_ptr(), _ptr(u_out), _stream()),
           "qlora_linear_fwd_noalloc")
    return out, u_out


def qlora_linear_bwd(w: NF4Weight, x: torch.Tensor, dy: torch.Tensor, a: torch.Tensor,
                     b: torch.Tensor, alpha: float, u: torch.Tensor | None = None,
                     need_dx: bool = True, workspace: torch.Tensor | None = None,
                     outs: tuple | None = None, dropout: float = 0.0, seed: int = 0):
    """Returns (dX bf16 [M, k] or None, dA fp32 [r, k], dB fp32 [d, r]).  dropout and
    seed: those of the forward."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(dy, torch.bfloat16, "dY")
    _dev_tensor(a, torch.bfloat16, "A")
    _dev_tensor(b, torch.bfloat16, "B")
    if u is not None:
        _dev_tensor(u, torch.float32, "U")
    m, r = x.shape[0], a.shape[0]
    if outs is not None:
        dx, da, db = outs
    else:
        dx = torch.empty((m, w.k), dtype=torch.bfloat16, device=x.device) if need_dx else None
        da = torch.empty((r, w.k), dtype=torch.float32, device=x.device)
        db = torch.empty((w.d, r), dtype=torch.float32, device=x.device)
    ws = workspace if workspace is not None else _workspace(
        linear_workspace_bytes(m, w.d, w.k, r, dropout > 0), x.device)
    cw = w.c_struct()
    if dropout > 0:
        _check(_lib.qlora_linear_bwd_dropout(ctypes.byref(cw), x.data_ptr(), dy.data_ptr(), a.data_ptr(),
                                             b.data_ptr(), _ptr(u), m, r, float(alpha), float(dropout),
                                             int(seed) & (2**64 - 1), _ptr(dx), da.data_ptr(), db.data_ptr(),
                                             ws.data_ptr(), ws.numel(), _stream()), "qlora_linear_bwd_dropout")
        return dx, da, db
    _check(_lib.qlora_linear_bwd(ctypes.byref(cw), x.data_ptr(), dy.data_ptr(), a.data_ptr(),
                                 b.data_ptr(), _ptr(u), m, r, float(alpha), _ptr(dx), da.data_ptr(),
                                 db.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "qlora_linear_bwd")
    return dx, da, db


def qlora_linear_gemm_only(w: NF4Weight, backward: bool, a: torch.Tensor, r: int,
                           out: torch.Tensor, workspace: torch.Tensor, expand: bool = False) -> torch.Tensor:
    """Measurement only: re-run the dequant-GEMM kernel of the preceding
    qlora_linear_fwd (a = x, out = Y) or qlora_linear_bwd (a = dY, out = dX) call
    alone, on the workspace that call prepared; expand=True runs the kernel that
    expands the NF4 codes tile by tile instead (with its block scales)."""
    _dev_tensor(a, torch.bfloat16, "a")
    _dev_tensor(out, torch.bfloat16, "out")
    cw = w.c_struct()
    _check(_lib.qlora_linear_gemm_only(ctypes.byref(cw), 1 if backward else 0, 1 if expand else 0, a.data_ptr(),
                                       a.shape[0], r, out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                       _stream()), "qlora_linear_gemm_only")
    return out


TIMED_KERNELS = {"fwd_gemm": 0, "dx_gemm": 1, "decode": 2}


def qlora_time_next_kernel(kernel: str, span: torch.Tensor | None) -> None:
    """Measurement only: the next launch of `kernel` ("fwd_gemm", "dx_gemm",
    "decode") records its start and end clock readings into `span` (a device
    int64 tensor of 2 elements filled with [-1, 0] beforehand: all bits set
    reads as UINT64_MAX); span_duration_us turns it into microseconds."""
    if span is not None:
        _dev_tensor(span, torch.int64, "span")
    _check(_lib.qlora_time_next_kernel(TIMED_KERNELS[kernel], _ptr(span)), "qlora_time_next_kernel")


def wall_clock_khz() -> int:
    v = ctypes.c_int32(0)
    _check(_lib.qlora_wall_clock_khz(ctypes.byref(v)), "qlora_wall_clock_khz")
    return int(v.value)


def span_duration_us(spans: torch.Tensor, khz: int):
    """Durations in microseconds of [n, 2] spans (read back to the host)."""
    s = spans.detach().cpu().view(-1, 2)
    return ((s[:, 1] - s[:, 0]).double() * 1e3 / khz).tolist()


def qlora_adapter_merge(w: NF4Weight, a: torch.Tensor, b: torch.Tensor, alpha: float,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [d, k] = What + (alpha/r) B A (qlora_adapter_merge's fixed rounding)."""
    _dev_tensor(a, torch.bfloat16, "A")
    _dev_tensor(b, torch.bfloat16, "B")
    y = out if out is not None else torch.empty((w.d, w.k), dtype=torch.bfloat16, device=a.device)
    _dev_tensor(y, torch.bfloat16, "out")
    cw = w.c_struct()
    _check(_lib.qlora_adapter_merge(ctypes.byref(cw), a.data_ptr(), b.data_ptr(), a.shape[0], float(alpha),
                                    y.data_ptr(), _stream()), "qlora_adapter_merge")
    return y


def qlora_adapter_unmerge(w_in: torch.Tensor, a: torch.Tensor, b: torch.Tensor, alpha: float,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [d, k] = W_in - (alpha/r) B A; out may be w_in (in place)."""
    _dev_tensor(w_in, torch.bfloat16, "W_in")
    _dev_tensor(a, torch.bfloat16, "A")
    _dev_tensor(b, torch.bfloat16, "B")
    d, k = w_in.shape
    y = out if out is not None else torch.empty_like(w_in)
    _dev_tensor(y, torch.bfloat16, "out")
    _check(_lib.qlora_adapter_unmerge(w_in.data_ptr(), d, k, a.data_ptr(), b.data_ptr(), a.shape[0],
                                      float(alpha), y.data_ptr(), _stream()), "qlora_adapter_unmerge")
    return y


__all__ = [
    "NF4Weight", "QloraError", "qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd",
    "qlora_linear_fwd_noalloc",
    "qlora_linear_bwd", "qlora_linear_gemm_only", "qlora_time_next_kernel", "wall_clock_khz",
    "span_duration_us", "qlora_adapter_merge", "qlora_adapter_unmerge",
    "qlora_lora_dropout",
    "qlora_nf4_codebook", "qlora_nf4_thresholds", "status_str", "library",
    "abi_version", "quantize_workspace_bytes", "linear_workspace_bytes",
    "BLOCK", "DQ_BLOCK", "NO_DQ", "C2_INT8", "C2_FP8_E4M3",
]
