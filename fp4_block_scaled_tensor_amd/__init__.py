"""Block-scaled FP4 quantization and FP4 GEMMs for MI355X (gfx950).

Python binding of libfp4bs.so (include/fp4bs.h). PyTorch provides device memory and the
current HIP stream; every step of the path runs in the library's HIP kernels. There is no
CPU or PyTorch fallback: importing works without the library, the first call raises if it
is missing.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (FP4_UE5M3, FP4_E4M3, FP4_E8M0, FP4_VIEW_ROW, FP4_VIEW_COL, FP4_VIEW_TILE2D,
                   FP4_SCALES_1D, FP4_SCALES_2D, FP4_SCALES_2D_T, FP4Error)

UE5M3, E4M3, E8M0 = FP4_UE5M3, FP4_E4M3, FP4_E8M0
ROW, COL, TILE2D = FP4_VIEW_ROW, FP4_VIEW_COL, FP4_VIEW_TILE2D

__all__ = ["UE5M3", "E4M3", "E8M0", "ROW", "COL", "TILE2D", "QTensor", "AmaxCache", "quantize", "quantize_rowcol",
           "fake_quant", "dequantize", "FakeQuantPolicy", "mxfp4_to_fp8", "quantize_local",
           "tensor_amax",
           "gemm_fprop", "gemm_dgrad", "gemm_wgrad", "gemm_fprop_q", "gemm_dgrad_q", "decode_f16", "gemm_f16", "scale_range", "check_range", "new_stats", "debug_encode",
           "FP4Error", "library"]


def library() -> ctypes.CDLL:
    return _lib.load()


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_check(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("FP4 kernels take device tensors (the path has no CPU implementation)")


@dataclass
class QTensor:
    """A quantized GEMM operand [rows x k]: packed E2M1 payload, scale codes, decode scale g."""
    q: torch.Tensor          # uint8 [rows, k // 2]
    s: torch.Tensor          # uint8 scale codes
    g: torch.Tensor          # float32 [1]
    fmt: int
    block: int
    layout: int              # FP4_SCALES_*
    rows: int
    k: int
    g_stripe: int = 0        # 0: g holds one float; else one float per stripe of g_stripe rows

    def operand(self) -> _lib.Operand:
        return _lib.Operand(self.q.data_ptr(), self.s.data_ptr(), self.g.data_ptr(), self.fmt, self.block,
                            self.layout, self.g_stripe, self.rows, self.k)


def _cfg(fmt, block, view, stochastic, hadamard_n, T, seed, offset) -> _lib.QuantCfg:
    return _lib.QuantCfg(int(fmt), int(block), int(view), int(bool(stochastic)), int(hadamard_n), float(T),
                         int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1))


def quantize(x: torch.Tensor, fmt: int = UE5M3, block: int = 16, view: int = ROW, amax: torch.Tensor | None = None,
             T: float = 448.0, stochastic: bool = False, seed: int = 0, offset: int = 0, hadamard_n: int = 0,
             amax_obs: torch.Tensor | None = None, stats: torch.Tensor | None = None):
    """fp4_quantize. x: bf16 or fp32 [rows, cols] on the GPU (row stride x.stride(0)).
    stats: optional int32 device tensor of 3 receiving the call's health counts (saturated,
    zero-scale, non-finite blocks).

    Returns a QTensor; for TILE2D a pair (forward operand [rows x cols], dgrad operand
    [cols x rows]) sharing the 2D scale grid and g."""
    lib = _lib.load()
    _dev_check(x, amax, amax_obs, stats)
    _stats_check(stats)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype == torch.bfloat16:
        dt = _lib.FP4_IN_BF16
    elif x.dtype == torch.float32:
        dt = _lib.FP4_IN_FP32
    else:
        raise ValueError("x must be bfloat16 or float32")
    rows, cols = x.shape
    cfg = _cfg(fmt, block, view, stochastic, hadamard_n, T, seed, offset)
    qb, sb, qtb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.fp4_quantize_sizes(rows, cols, ctypes.byref(cfg), ctypes.byref(qb), ctypes.byref(sb),
                                      ctypes.byref(qtb)))
    dev = x.device
    if view == COL:
        q = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((cols, rows // block), dtype=torch.uint8, device=dev)
    elif view == TILE2D:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows // 16, cols // 16), dtype=torch.uint8, device=dev)
    else:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // block), dtype=torch.uint8, device=dev)
    qt = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev) if view == TILE2D else None
    g = torch.empty(1, dtype=torch.float32, device=dev)
    _lib.check(lib.fp4_quantize(_ptr(x), dt, rows, cols, x.stride(0), ctypes.byref(cfg), _ptr(amax), _ptr(q), _ptr(s),
                                _ptr(qt), _ptr(g), _ptr(amax_obs), _ptr(stats), _stream()))
    if view == ROW:
        return QTensor(q, s, g, fmt, block, FP4_SCALES_1D, rows, cols)
    if view == COL:
        return QTensor(q, s, g, fmt, block, FP4_SCALES_1D, cols, rows)
    return (QTensor(q, s, g, fmt, 16, FP4_SCALES_2D, rows, cols),
            QTensor(qt, s, g, fmt, 16, FP4_SCALES_2D_T, cols, rows))


def _stats_check(stats):
    if stats is not None and (stats.dtype != torch.int32 or stats.numel() < 3 or not stats.is_contiguous()):
        raise ValueError("stats must be a contiguous int32 device tensor of at least 3 elements")


def new_stats(device="cuda") -> torch.Tensor:
    """A device buffer for the health counts of one quantize call (int32 x 3: saturated,
    zero-scale and non-finite blocks)."""
    return torch.zeros(3, dtype=torch.int32, device=device)


def _in_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return _lib.FP4_IN_BF16
    if x.dtype == torch.float32:
        return _lib.FP4_IN_FP32
    raise ValueError("x must be bfloat16 or float32")


def quantize_rowcol(x: torch.Tensor, fmt: int = UE5M3, block: int = 16, amax_row: torch.Tensor | None = None,
                    amax_col: torch.Tensor | None = None, T_row: float = 448.0, T_col: float = 448.0,
                    stochastic_row: bool = False, stochastic_col: bool = False, seed_row: int = 0,
                    offset_row: int = 0, seed_col: int = 0, offset_col: int = 0, hadamard_n: int = 0,
                    amax_obs_row: torch.Tensor | None = None, amax_obs_col: torch.Tensor | None = None,
                    stats_row: torch.Tensor | None = None, stats_col: torch.Tensor | None = None):
    """fp4_quantize_rowcol: (ROW operand [rows x cols], COL operand x^T [cols x rows]) from one pass
    over x; each equals the matching fp4_quantize call. hadamard_n rotates the COL view only;
    stats_row / stats_col receive each view's health counts as in quantize()."""
    lib = _lib.load()
    _dev_check(x, amax_row, amax_col, amax_obs_row, amax_obs_col, stats_row, stats_col)
    _stats_check(stats_row)
    _stats_check(stats_col)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _in_dtype(x)
    rows, cols = x.shape
    cr = _cfg(fmt, block, ROW, stochastic_row, 0, T_row, seed_row, offset_row)
    cc = _cfg(fmt, block, COL, stochastic_col, hadamard_n, T_col, seed_col, offset_col)
    for cfg in (cr, cc):
        qb, sb, qtb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _lib.check(lib.fp4_quantize_sizes(rows, cols, ctypes.byref(cfg), ctypes.byref(qb), ctypes.byref(sb),
                                          ctypes.byref(qtb)))
    dev = x.device
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, cols // block), dtype=torch.uint8, device=dev)
    qt = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
    st = torch.empty((cols, rows // block), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    gt = torch.empty(1, dtype=torch.float32, device=dev)
    _lib.check(lib.fp4_quantize_rowcol(_ptr(x), dt, rows, cols, x.stride(0), ctypes.byref(cr), ctypes.byref(cc),
                                       _ptr(amax_row), _ptr(amax_col), _ptr(q), _ptr(s), _ptr(g), _ptr(amax_obs_row),
                                       _ptr(qt), _ptr(st), _ptr(gt), _ptr(amax_obs_col), _ptr(stats_row),
                                       _ptr(stats_col), _stream()))
    return (QTensor(q, s, g, fmt, block, FP4_SCALES_1D, rows, cols),
            QTensor(qt, st, gt, fmt, block, FP4_SCALES_1D, cols, rows))


def _out_dtype(dtype) -> int:
    if dtype == torch.bfloat16:
        return _lib.FP4_IN_BF16
    if dtype == torch.float32:
        return _lib.FP4_IN_FP32
    raise ValueError("output dtype must be bfloat16 or float32")


def fake_quant(x: torch.Tensor, fmt: int = UE5M3, block: int = 16, amax: torch.Tensor | None = None,
               T: float = 448.0, out_dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_fake_quant: the decoded value of x's ROW-view FP4 quantization, [rows, cols]."""
    lib = _lib.load()
    _dev_check(x, amax, out)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=x.device)
    if out.dim() != 2 or out.shape != x.shape or out.stride(1) != 1:
        raise ValueError("out must be [rows, cols] with unit column stride")
    cfg = _cfg(fmt, block, ROW, False, 0, T, 0, 0)
    _lib.check(lib.fp4_fake_quant(_ptr(x), _in_dtype(x), rows, cols, x.stride(0), ctypes.byref(cfg), _ptr(amax),
                                  _ptr(out), _out_dtype(out.dtype), out.stride(0), _stream()))
    return out


def dequantize(a: QTensor, out_dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_dequantize: the decoded values [rows, k] of a quantized operand."""
    lib = _lib.load()
    if out is None:
        out = torch.empty((a.rows, a.k), dtype=out_dtype, device=a.q.device)
    _dev_check(out)
    if out.dim() != 2 or tuple(out.shape) != (a.rows, a.k) or out.stride(1) != 1:
        raise ValueError("out must be [rows, k] with unit column stride")
    op = a.operand()
    _lib.check(lib.fp4_dequantize(ctypes.byref(op), _ptr(out), _out_dtype(out.dtype), out.stride(0), _stream()))
    return out


def quantize_local(x: torch.Tensor, fmt: int = E4M3, block: int = 16, stripe: int = 16, T: float = 448.0,
                   stochastic: bool = False, seed: int = 0, offset: int = 0,
                   amax_obs: torch.Tensor | None = None) -> QTensor:
    """fp4_quantize_local: ROW-view operand with one tensor scale per stripe of `stripe` rows
    (its g holds ceil(rows / stripe) floats)."""
    lib = _lib.load()
    _dev_check(x, amax_obs)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    dev = x.device
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((rows, cols // block), dtype=torch.uint8, device=dev)
    g = torch.empty(max(1, -(-rows // stripe)), dtype=torch.float32, device=dev)
    cfg = _cfg(fmt, block, ROW, stochastic, 0, T, seed, offset)
    _lib.check(lib.fp4_quantize_local(_ptr(x), _in_dtype(x), rows, cols, x.stride(0), ctypes.byref(cfg), int(stripe),
                                      _ptr(q), _ptr(s), _ptr(g), _ptr(amax_obs), _stream()))
    return QTensor(q, s, g, fmt, block, FP4_SCALES_1D, rows, cols, g_stripe=int(stripe))


def mxfp4_to_fp8(a: QTensor, transpose: bool = False):
    """fp4_mxfp4_to_fp8: (E4M3 bytes [rows, k] or [k, rows] as uint8, chunk scale codes
    [rows, k/128] as uint8) of an MXFP4 operand."""
    lib = _lib.load()
    dev = a.q.device
    y = torch.empty((a.k, a.rows) if transpose else (a.rows, a.k), dtype=torch.uint8, device=dev)
    s8 = torch.empty((a.rows, a.k // 128), dtype=torch.uint8, device=dev)
    op = a.operand()
    _lib.check(lib.fp4_mxfp4_to_fp8(ctypes.byref(op), int(bool(transpose)), _ptr(y), _ptr(s8), _stream()))
    return y, s8


class FakeQuantPolicy:
    """Activation-scale policy of fake-quantized inference requests, taken in order: 'delayed'
    (sample-and-hold cache, period D, 50 by default), 'current' (D = 1) or 'frozen' (a fixed
    calibration amax). The sampling decision and the amax stay on the device."""

    def __init__(self, kind: str, fmt: int = UE5M3, block: int = 16, T: float = 448.0, D: int | None = None,
                 amax: float | None = None, device="cuda"):
        if kind not in ("delayed", "current", "frozen"):
            raise ValueError(kind)
        self.kind, self.fmt, self.block, self.T = kind, fmt, block, T
        if kind == "frozen":
            if amax is None:
                raise ValueError("a frozen policy needs its calibration amax")
            self.cache = None
            self.amax = torch.full((1,), float(amax), dtype=torch.float32, device=device)
        else:
            self.cache = AmaxCache(1 if kind == "current" else (50 if D is None else D), device=device)
            self.amax = self.cache.amax
            self._obs = torch.empty(1, dtype=torch.float32, device=device)

    def __call__(self, request: int, x: torch.Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None):
        if self.cache is not None and self.fmt != E8M0 and self.cache.needs_sample(request):
            tensor_amax(x, out=self._obs)
            self.cache.update(request, self._obs)
        return fake_quant(x, self.fmt, self.block, amax=None if self.fmt == E8M0 else self.amax, T=self.T,
                          out_dtype=out_dtype, out=out)


def tensor_amax(x: torch.Tensor, hadamard_n: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_tensor_amax: max|x| (after the blockwise FWHT along rows if hadamard_n) into a [1] float32 tensor."""
    lib = _lib.load()
    _dev_check(x)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    dt = _lib.FP4_IN_FP32 if x.dtype == torch.float32 else _lib.FP4_IN_BF16
    if x.dtype not in (torch.float32, torch.bfloat16) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16/fp32 tensor with unit column stride")
    _lib.check(lib.fp4_tensor_amax(_ptr(x), dt, x.shape[0], x.shape[1], x.stride(0), int(hadamard_n), _ptr(out),
                                   _stream()))
    return out


class AmaxCache:
    """Device-resident sample-and-hold amax cache (amax_cache_update / amax_cache_reset)."""

    def __init__(self, D: int = 50, device: str | torch.device = "cuda"):
        self.D = int(D)
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        self.valid = torch.zeros(1, dtype=torch.int32, device=device)
        self._host_valid = False   # mirror of the device flag, kept by this object

    def _c(self) -> _lib.AmaxCacheC:
        return _lib.AmaxCacheC(self.amax.data_ptr(), self.valid.data_ptr(), self.D)

    def needs_sample(self, step: int) -> bool:
        return (not self._host_valid) or step % self.D == 0

    def update(self, step: int, amax_obs: torch.Tensor) -> None:
        lib = _lib.load()
        c = self._c()
        _lib.check(lib.amax_cache_update(ctypes.byref(c), int(step), _ptr(amax_obs), _stream()))
        self._host_valid = True

    def reset(self) -> None:
        lib = _lib.load()
        c = self._c()
        _lib.check(lib.amax_cache_reset(ctypes.byref(c), _stream()))
        self._host_valid = False


def _gemm(name: str, a: QTensor, b: QTensor, canon: bool, hadamard_n: int | None, out: torch.Tensor | None):
    lib = _lib.load()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.q.device)
    if out.shape != (a.rows, b.rows) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, N] tensor")
    oa, ob = a.operand(), b.operand()
    fn = getattr(lib, name)
    if hadamard_n is None:
        st = fn(ctypes.byref(oa), ctypes.byref(ob), _ptr(out), int(bool(canon)), _stream())
    else:
        st = fn(ctypes.byref(oa), ctypes.byref(ob), _ptr(out), int(hadamard_n), int(bool(canon)), _stream())
    _lib.check(st)
    return out


def _gemm_q(name: str, a: QTensor, b: QTensor, fmt: int, block: int, amax: torch.Tensor | None, T: float,
            stochastic: bool, seed: int, offset: int, canon: bool, want_f32: bool, amax_obs, stats):
    lib = _lib.load()
    _dev_check(amax, amax_obs, stats)
    _stats_check(stats)
    M, N = a.rows, b.rows
    dev = a.q.device
    y = torch.empty((M, N), dtype=torch.float32, device=dev) if want_f32 else None
    q = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M, N // block), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    cfg = _cfg(fmt, block, ROW, stochastic, 0, T, seed, offset)
    oa, ob = a.operand(), b.operand()
    _lib.check(getattr(lib, name)(ctypes.byref(oa), ctypes.byref(ob), _ptr(y), int(bool(canon)), ctypes.byref(cfg),
                                  _ptr(amax), _ptr(q), _ptr(s), _ptr(g), _ptr(amax_obs), _ptr(stats), _stream()))
    return QTensor(q, s, g, fmt, block, FP4_SCALES_1D, M, N), y


def gemm_fprop_q(x: QTensor, w: QTensor, fmt: int = UE5M3, block: int = 16, amax: torch.Tensor | None = None,
                 T: float = 448.0, stochastic: bool = False, seed: int = 0, offset: int = 0, canon: bool = False,
                 want_f32: bool = False, amax_obs: torch.Tensor | None = None, stats: torch.Tensor | None = None):
    """fp4_gemm_fprop_q: (Y quantized as the next fprop's ROW-view operand, float32 Y or None)."""
    return _gemm_q("fp4_gemm_fprop_q", x, w, fmt, block, amax, T, stochastic, seed, offset, canon, want_f32,
                   amax_obs, stats)


def gemm_dgrad_q(dy: QTensor, wt: QTensor, fmt: int = UE5M3, block: int = 16, amax: torch.Tensor | None = None,
                 T: float = 448.0, stochastic: bool = True, seed: int = 0, offset: int = 0, canon: bool = False,
                 want_f32: bool = False, amax_obs: torch.Tensor | None = None, stats: torch.Tensor | None = None):
    """fp4_gemm_dgrad_q: (dX quantized as the previous dgrad's ROW-view dY operand, float32 dX or None)."""
    return _gemm_q("fp4_gemm_dgrad_q", dy, wt, fmt, block, amax, T, stochastic, seed, offset, canon, want_f32,
                   amax_obs, stats)


def decode_f16(a: QTensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_decode_f16: the UE5M3/E4M3 operand decoded to float16 [rows, K] (E2M1 x block scale
    x 2^-3, exact; no tensor scale)."""
    lib = _lib.load()
    if out is None:
        out = torch.empty((a.rows, a.k), dtype=torch.float16, device=a.q.device)
    if out.shape != (a.rows, a.k) or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float16 [rows, K] tensor")
    op = a.operand()
    _lib.check(lib.fp4_decode_f16(ctypes.byref(op), _ptr(out), _stream()))
    return out


def gemm_f16(a: QTensor, b: QTensor, a16: torch.Tensor | None = None, b16: torch.Tensor | None = None,
             hadamard_n: int = 0, canon: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_gemm_f16: C = A . B^T from the operands' fp16 decodes (decoded here when not given),
    bit-identical to gemm_fprop / gemm_dgrad / gemm_wgrad on the same operands."""
    lib = _lib.load()
    a16 = decode_f16(a) if a16 is None else a16
    b16 = decode_f16(b) if b16 is None else b16
    _dev_check(a16, b16)
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.q.device)
    if out.shape != (a.rows, b.rows) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [M, N] tensor")
    oa, ob = a.operand(), b.operand()
    _lib.check(lib.fp4_gemm_f16(ctypes.byref(oa), _ptr(a16), ctypes.byref(ob), _ptr(b16), _ptr(out), int(hadamard_n),
                                int(bool(canon)), _stream()))
    return out


def scale_range(a: QTensor) -> torch.Tensor:
    """fp4_scale_range: int32 device tensor [min code, max code] of the operand's scale codes."""
    lib = _lib.load()
    out = torch.empty(2, dtype=torch.int32, device=a.q.device)
    op = a.operand()
    _lib.check(lib.fp4_scale_range(ctypes.byref(op), _ptr(out), _stream()))
    return out


def check_range(a: QTensor, b: QTensor) -> None:
    """Checked mode of a GEMM: raises FP4Error (FP4_ERANGE) when the two operands' scale codes
    could take a block partial outside the GEMM's exact range. Synchronises (the ranges are
    read back to the host)."""
    lib = _lib.load()
    ra, rb = scale_range(a).cpu().numpy(), scale_range(b).cpu().numpy()
    A = (ctypes.c_int32 * 2)(int(ra[0]), int(ra[1]))
    B = (ctypes.c_int32 * 2)(int(rb[0]), int(rb[1]))
    _lib.check(lib.fp4_gemm_check_range(int(a.fmt), A, B))


def gemm_fprop(x: QTensor, w: QTensor, canon: bool = False, out: torch.Tensor | None = None,
               checked: bool = False) -> torch.Tensor:
    """Y = X . W^T (fp4_gemm_fprop). checked: verify the exact range first (check_range)."""
    if checked:
        check_range(x, w)
    return _gemm("fp4_gemm_fprop", x, w, canon, None, out)


def gemm_dgrad(dy: QTensor, wt: QTensor, canon: bool = False, out: torch.Tensor | None = None,
               checked: bool = False) -> torch.Tensor:
    """dX = dY . W (fp4_gemm_dgrad); wt is the weight's transposed operand."""
    if checked:
        check_range(dy, wt)
    return _gemm("fp4_gemm_dgrad", dy, wt, canon, None, out)


def gemm_wgrad(dyt: QTensor, xt: QTensor, hadamard_n: int = 0, canon: bool = False,
               out: torch.Tensor | None = None, checked: bool = False) -> torch.Tensor:
    """dW = dY^T . X (fp4_gemm_wgrad) from the two COL-view operands."""
    if checked:
        check_range(dyt, xt)
    return _gemm("fp4_gemm_wgrad", dyt, xt, canon, hadamard_n, out)


def debug_encode(x: torch.Tensor, which: int, u16: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_debug_encode: device encoder codes for float32 inputs (parity tests)."""
    lib = _lib.load()
    _dev_check(x, u16)
    x = x.contiguous()
    out = torch.empty(x.numel(), dtype=torch.uint8, device=x.device)
    _lib.check(lib.fp4_debug_encode(_ptr(x), _ptr(u16), x.numel(), int(which), _ptr(out), _stream()))
    return out
