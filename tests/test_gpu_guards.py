"""Guard bands around every output buffer: each entry point of the C ABI writes exactly its
outputs and nothing around them.

Every output (payload, scales, g, observed amax, health counts, GEMM outputs, decodes, FP8
bytes, row-strided fake-quant and decode outputs with their inter-row gaps) is placed inside a
larger device allocation whose surrounding bytes hold a fill pattern; after the call the
pattern must be intact. Shapes are ragged (partial tiles in both dimensions) so that the edge
paths of the kernels run. The values themselves are checked elsewhere against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as OF
from tests._helpers import dev_scalar, qtensor_from_oracle, random_operand

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")
from fp4_block_scaled_tensor_amd import _lib  # noqa: E402

G = 4096          # guard bytes on each side
PAT = 0xA5


class Guarded:
    """nbytes of device memory at a 256-byte aligned address, surrounded by guard bytes."""

    def __init__(self, nbytes: int):
        self.n = int(nbytes)
        self.buf = torch.full((G + ((self.n + 255) // 256) * 256 + G,), PAT, dtype=torch.uint8, device="cuda")
        self.ptr = ctypes.c_void_p(self.buf.data_ptr() + G)

    def check(self, what: str):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        head, tail = b[:G], b[G + self.n:]
        assert np.all(head == PAT), f"{what}: {int(np.sum(head != PAT))} bytes written before the buffer"
        assert np.all(tail == PAT), f"{what}: {int(np.sum(tail != PAT))} bytes written after the buffer"


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _x(rows, cols, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn((rows, cols), generator=g) * 3).to(dtype).cuda()


@pytest.mark.parametrize("view,rows,cols,fmt,block,sr,hn", [
    (0, 130, 160, OF.UE5M3, 16, False, 0),
    (0, 72, 352, OF.E8M0, 32, True, 0),
    (1, 96, 136, OF.UE5M3, 16, True, 16),
    (1, 64, 200, OF.E8M0, 32, False, 32),
    (2, 144, 160, OF.E4M3, 16, False, 0),
])
def test_quantize_writes_only_its_outputs(view, rows, cols, fmt, block, sr, hn):
    lib = _lib.load()
    x = _x(rows, cols, rows + cols)
    cfg = fp4._cfg(fmt, block, view, sr, hn, 448.0, 3, 5)
    qb, sb, qtb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(lib.fp4_quantize_sizes(rows, cols, ctypes.byref(cfg), ctypes.byref(qb), ctypes.byref(sb),
                                      ctypes.byref(qtb)))
    q, s, g, obs, st = Guarded(qb.value), Guarded(sb.value), Guarded(4), Guarded(4), Guarded(12)
    qt = Guarded(qtb.value) if qtb.value else None
    amax = None if fmt == OF.E8M0 else dev_scalar(float(x.float().abs().max()))
    _lib.check(lib.fp4_quantize(ctypes.c_void_p(x.data_ptr()), _lib.FP4_IN_BF16, rows, cols, x.stride(0),
                                ctypes.byref(cfg), fp4._ptr(amax), q.ptr, s.ptr, qt.ptr if qt else None, g.ptr,
                                obs.ptr, st.ptr, _stream()))
    for name, b in (("q", q), ("s", s), ("g", g), ("amax_obs", obs), ("stats", st)) + ((("q_t", qt),) if qt else ()):
        b.check(f"view {view} {name}")


def test_quantize_rowcol_writes_only_its_outputs():
    lib = _lib.load()
    rows, cols = 96, 208          # both views ragged against their tiles
    x = _x(rows, cols, 7)
    cr = fp4._cfg(OF.UE5M3, 16, fp4.ROW, False, 0, 448.0, 0, 0)
    cc = fp4._cfg(OF.UE5M3, 16, fp4.COL, True, 16, 2048.0, 42, 1)
    a = dev_scalar(float(x.float().abs().max()) * 2)
    bufs = dict(q=Guarded(rows * cols // 2), s=Guarded(rows * cols // 16), g=Guarded(4), obs=Guarded(4),
                qt=Guarded(rows * cols // 2), st=Guarded(rows * cols // 16), gt=Guarded(4), obst=Guarded(4),
                sr=Guarded(12), sc=Guarded(12))
    _lib.check(lib.fp4_quantize_rowcol(ctypes.c_void_p(x.data_ptr()), _lib.FP4_IN_BF16, rows, cols, x.stride(0),
                                       ctypes.byref(cr), ctypes.byref(cc), fp4._ptr(a), fp4._ptr(a), bufs["q"].ptr,
                                       bufs["s"].ptr, bufs["g"].ptr, bufs["obs"].ptr, bufs["qt"].ptr, bufs["st"].ptr,
                                       bufs["gt"].ptr, bufs["obst"].ptr, bufs["sr"].ptr, bufs["sc"].ptr, _stream()))
    for k, b in bufs.items():
        b.check(f"rowcol {k}")


@pytest.mark.parametrize("fmt,block", [(OF.UE5M3, 16), (OF.E8M0, 32), (OF.E4M3, 16)])
def test_gemms_write_only_their_outputs(fmt, block):
    lib = _lib.load()
    M, N, K = 200, 144, 320          # N: a multiple of the output block, not of any tile
    rng = np.random.default_rng(M + N + K + fmt)
    qa = qtensor_from_oracle(random_operand(rng, M, K, fmt, block, 3))
    qb = qtensor_from_oracle(random_operand(rng, N, K, fmt, block, 3))
    oa, ob = qa.operand(), qb.operand()
    for name in ("fp4_gemm_fprop", "fp4_gemm_dgrad"):
        c = Guarded(M * N * 4)
        _lib.check(getattr(lib, name)(ctypes.byref(oa), ctypes.byref(ob), c.ptr, 0, _stream()))
        c.check(name)
    c = Guarded(M * N * 4)
    _lib.check(lib.fp4_gemm_wgrad(ctypes.byref(oa), ctypes.byref(ob), c.ptr, 16, 1, _stream()))
    c.check("fp4_gemm_wgrad")
    # epilogue-quantized output (UE5M3 block 16 ROW view of C), with and without float32 C
    cfg = fp4._cfg(OF.UE5M3, 16, fp4.ROW, True, 0, 448.0, 9, 2)
    amax = dev_scalar(50.0)
    for name, with_c in (("fp4_gemm_fprop_q", True), ("fp4_gemm_fprop_q", False), ("fp4_gemm_dgrad_q", True)):
        c = Guarded(M * N * 4) if with_c else None
        q, s, g, obs, st = Guarded(M * N // 2), Guarded(M * N // 16), Guarded(4), Guarded(4), Guarded(12)
        _lib.check(getattr(lib, name)(ctypes.byref(oa), ctypes.byref(ob), c.ptr if c else None, 0, ctypes.byref(cfg),
                                      fp4._ptr(amax), q.ptr, s.ptr, g.ptr, obs.ptr, st.ptr, _stream()))
        for nm, b in (("q", q), ("s", s), ("g", g), ("obs", obs), ("stats", st)) + ((("c", c),) if c else ()):
            b.check(f"{name} {nm}")
    if fmt != OF.E8M0:
        a16, b16 = Guarded(M * K * 2), Guarded(N * K * 2)
        _lib.check(lib.fp4_decode_f16(ctypes.byref(oa), a16.ptr, _stream()))
        _lib.check(lib.fp4_decode_f16(ctypes.byref(ob), b16.ptr, _stream()))
        a16.check("decode_f16 A")
        b16.check("decode_f16 B")
        c = Guarded(M * N * 4)
        _lib.check(lib.fp4_gemm_f16(ctypes.byref(oa), a16.ptr, ctypes.byref(ob), b16.ptr, c.ptr, 0, 0, _stream()))
        c.check("gemm_f16")
    r = Guarded(8)
    _lib.check(lib.fp4_scale_range(ctypes.byref(oa), r.ptr, _stream()))
    r.check("scale_range")


def test_row_strided_outputs_leave_the_gaps_between_rows():
    """fake_quant and dequantize with a row stride above the row length: the bytes between
    rows (and around the whole output) stay untouched."""
    rows, cols, ld = 70, 192, 232      # operands need K % 64 == 0
    x = _x(rows, cols, 11)
    for dtype, esz in ((torch.bfloat16, 2), (torch.float32, 4)):
        gbuf = Guarded(rows * ld * esz)
        view = gbuf.buf[G:G + rows * ld * esz].view(dtype).view(rows, ld)
        out = view[:, :cols]
        fp4.fake_quant(x, OF.UE5M3, 16, amax=dev_scalar(float(x.float().abs().max())), T=448.0, out=out)
        torch.cuda.synchronize()
        raw = view.view(torch.uint8).reshape(rows, ld * esz).cpu().numpy()
        assert np.all(raw[:, cols * esz:] == PAT), f"fake_quant {dtype}: inter-row gap written"
        gbuf.check(f"fake_quant {dtype}")
    q = fp4.quantize(x, OF.E8M0, 32, fp4.ROW)
    gbuf = Guarded(rows * ld * 2)
    view = gbuf.buf[G:G + rows * ld * 2].view(torch.bfloat16).view(rows, ld)
    fp4.dequantize(q, out=view[:, :cols])
    torch.cuda.synchronize()
    raw = view.view(torch.uint8).reshape(rows, ld * 2).cpu().numpy()
    assert np.all(raw[:, cols * 2:] == PAT), "dequantize: inter-row gap written"
    gbuf.check("dequantize")


@pytest.mark.parametrize("transpose", [0, 1])
def test_mxfp4_to_fp8_and_local_and_amax_write_only_their_outputs(transpose):
    lib = _lib.load()
    rows, K = 80, 384
    x = _x(rows, K, 13)
    q = fp4.quantize(x, OF.E8M0, 32, fp4.ROW)
    op = q.operand()
    y, s8 = Guarded(rows * K), Guarded(rows * (K // 128))
    _lib.check(lib.fp4_mxfp4_to_fp8(ctypes.byref(op), transpose, y.ptr, s8.ptr, _stream()))
    y.check("mxfp4_to_fp8 y")
    s8.check("mxfp4_to_fp8 s8")
    cfg = fp4._cfg(OF.E4M3, 16, fp4.ROW, False, 0, 448.0, 0, 0)
    ql, sl, gl, ol = Guarded(rows * K // 2), Guarded(rows * K // 16), Guarded(4 * ((rows + 15) // 16)), \
        Guarded(4 * ((rows + 15) // 16))      # g and amax_obs: one float per stripe
    _lib.check(lib.fp4_quantize_local(ctypes.c_void_p(x.data_ptr()), _lib.FP4_IN_BF16, rows, K, x.stride(0),
                                      ctypes.byref(cfg), 16, ql.ptr, sl.ptr, gl.ptr, ol.ptr, _stream()))
    for nm, b in (("q", ql), ("s", sl), ("g", gl), ("obs", ol)):
        b.check(f"quantize_local {nm}")
    out = Guarded(4)
    _lib.check(lib.fp4_tensor_amax(ctypes.c_void_p(x.data_ptr()), _lib.FP4_IN_BF16, rows, K, x.stride(0),
                                   16 if transpose else 0, out.ptr, _stream()))
    out.check("tensor_amax")


@pytest.mark.parametrize("bad", [0.0, float("inf"), float("nan")])
def test_degenerate_amax_through_the_cache(bad):
    """A zero, infinite or NaN observed amax fed to the D = 50 cache at step 0 is held through
    step 22; a reset before step 23 (a resumed run) samples again there. The cache holds what
    the oracle's does at every step, and a quantization with the degenerate cached amax falls
    back to unit tensor scales as in the oracle."""
    cache, ref = fp4.AmaxCache(D=50), oracle.AmaxCache(50)
    for step in range(30):
        v = bad if step == 0 else 3.0 + step
        if step == 23:
            cache.reset()
            ref.reset()
        cache.update(step, dev_scalar(v))
        ref.update(step, np.float32(v))
        if step == 0:
            x = _x(32, 64, 17, torch.float32)
            got = fp4.quantize(x, OF.UE5M3, 16, fp4.ROW, amax=cache.amax, T=448.0)
            want = oracle.quantize_1d(x.cpu().numpy(), OF.UE5M3, 16, amax=np.float32(bad), T=448.0)
            torch.cuda.synchronize()
            assert np.array_equal(got.q.cpu().numpy(), want.packed) and np.array_equal(got.s.cpu().numpy(),
                                                                                       want.scales)
            assert got.g.item() == np.float32(want.g) == np.float32(1.0)
        torch.cuda.synchronize()
        c, r = cache.amax.item(), float(ref.amax)
        assert (np.isnan(c) and np.isnan(r)) or c == r, f"step {step}: cache {c} vs oracle {r}"
    assert cache.amax.item() == np.float32(3.0 + 23)     # sampled again at the step after the reset
