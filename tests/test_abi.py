"""The C ABI on the host: the library loads, exports every function include/fp4bs.h declares,
and rejects invalid arguments before enqueuing anything (no GPU needed for these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

from fp4_block_scaled_tensor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4bs.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfp4bs.so is not built; run `python -m fp4_block_scaled_tensor_amd.build`")
    return _lib.load()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:fp4_status|const char\*|int32_t)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTED), decl
    assert len(decl) == 22


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_abi_version(lib):
    assert lib.fp4_abi_version() == _lib.ABI_VERSION


def cfg(fmt=0, block=16, view=0, sr=0, hn=0, T=448.0):
    return _lib.QuantCfg(fmt, block, view, sr, hn, T, 0, 0)


def test_quantize_sizes(lib):
    q, s, qt = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    c = cfg()
    assert lib.fp4_quantize_sizes(8192, 4096, ctypes.byref(c), ctypes.byref(q), ctypes.byref(s), ctypes.byref(qt)) == 0
    assert (q.value, s.value, qt.value) == (8192 * 2048, 8192 * 256, 0)
    c = cfg(view=2)
    assert lib.fp4_quantize_sizes(14336, 4096, ctypes.byref(c), ctypes.byref(q), ctypes.byref(s), ctypes.byref(qt)) == 0
    assert (q.value, s.value, qt.value) == (14336 * 2048, 896 * 256, 14336 * 2048)
    c = cfg(fmt=2, block=32, view=1)
    assert lib.fp4_quantize_sizes(8192, 4096, ctypes.byref(c), ctypes.byref(q), ctypes.byref(s), ctypes.byref(qt)) == 0
    assert (q.value, s.value) == (4096 * 4096, 4096 * 256)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=2, block=16), _lib.FP4_EUNSUPPORTED),      # E8M0 needs block 32
    (dict(block=8), _lib.FP4_EUNSUPPORTED),
    (dict(fmt=7), _lib.FP4_EINVAL),
    (dict(view=2, block=32), _lib.FP4_EUNSUPPORTED),     # 2D tiles are 16x16
    (dict(view=2, sr=1), _lib.FP4_EUNSUPPORTED),         # weights: nearest-even only
    (dict(hn=16), _lib.FP4_EUNSUPPORTED),                # Hadamard only on the COL view
    (dict(view=1, hn=8), _lib.FP4_EINVAL),
    (dict(T=-1.0), _lib.FP4_EINVAL),
])
def test_quantize_rejects_bad_config(lib, kw, status):
    c = cfg(**kw)
    st = lib.fp4_quantize(ctypes.c_void_p(16), 0, 64, 64, 64, ctypes.byref(c), ctypes.c_void_p(16),
                          ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, None, None, None)
    assert st == status
    assert lib.fp4_last_error().decode()


def test_quantize_rejects_bad_shapes_and_pointers(lib):
    c = cfg()
    P = ctypes.c_void_p(4096)
    assert lib.fp4_quantize(P, 0, 64, 40, 40, ctypes.byref(c), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    assert lib.fp4_quantize(P, 0, 64, 64, 32, ctypes.byref(c), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    assert lib.fp4_quantize(None, 0, 64, 64, 64, ctypes.byref(c), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    assert lib.fp4_quantize(ctypes.c_void_p(4098), 0, 64, 64, 64, ctypes.byref(c), P, P, P, None, None, None,
                            None, None) == _lib.FP4_EALIGN
    assert lib.fp4_quantize(P, 0, 64, 64, 68, ctypes.byref(c), P, P, P, None, None, None, None, None) == _lib.FP4_EALIGN
    assert lib.fp4_quantize(P, 0, 64, 64, 64, ctypes.byref(c), None, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    assert lib.fp4_quantize(P, 3, 64, 64, 64, ctypes.byref(c), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    c2 = cfg(view=1)
    assert lib.fp4_quantize(P, 0, 40, 64, 64, ctypes.byref(c2), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    c3 = cfg(view=2)
    assert lib.fp4_quantize(P, 0, 64, 64, 64, ctypes.byref(c3), P, P, P, None, None, None, None, None) == _lib.FP4_EINVAL
    assert "q_t" in lib.fp4_last_error().decode()
    # the health-count output is 4-byte aligned
    assert lib.fp4_quantize(P, 0, 64, 64, 64, ctypes.byref(c), P, P, P, None, None, None, ctypes.c_void_p(4098),
                            None) == _lib.FP4_EALIGN
    assert "stats" in lib.fp4_last_error().decode()


def op(rows=64, k=128, fmt=0, block=16, layout=0, q=4096, s=4096):
    return _lib.Operand(q, s, None, fmt, block, layout, 0, rows, k)


def test_gemm_rejects_bad_operands(lib):
    y = ctypes.c_void_p(4096)
    a, b = op(), op(k=192)
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(b), y, 0, None) == _lib.FP4_EINVAL      # K mismatch
    a, b = op(k=96), op(k=96)
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(b), y, 0, None) == _lib.FP4_EINVAL      # K % 64
    a, b = op(), op(fmt=1)
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(b), y, 0, None) == _lib.FP4_EUNSUPPORTED
    a, b = op(), op(layout=2)
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(b), y, 0, None) == _lib.FP4_EUNSUPPORTED
    assert lib.fp4_gemm_dgrad(ctypes.byref(op()), ctypes.byref(op(layout=1)), y, 0, None) == _lib.FP4_EUNSUPPORTED
    assert lib.fp4_gemm_wgrad(ctypes.byref(op()), ctypes.byref(op()), y, 8, 0, None) == _lib.FP4_EINVAL
    assert lib.fp4_gemm_fprop(ctypes.byref(op(q=4097)), ctypes.byref(op()), y, 0, None) == _lib.FP4_EALIGN
    assert lib.fp4_gemm_fprop(ctypes.byref(op()), ctypes.byref(op()), None, 0, None) == _lib.FP4_EINVAL
    assert lib.fp4_gemm_fprop(ctypes.byref(op(fmt=2, block=32, layout=1, rows=64)), ctypes.byref(op(fmt=2, block=32)),
                              y, 0, None) == _lib.FP4_EUNSUPPORTED
    assert lib.fp4_gemm_fprop(None, ctypes.byref(op()), y, 0, None) == _lib.FP4_EINVAL


def test_gemm_empty_is_noop(lib):
    assert lib.fp4_gemm_fprop(ctypes.byref(op(rows=0)), ctypes.byref(op()), None, 0, None) == _lib.FP4_OK


def test_cache_and_debug_validation(lib):
    c = _lib.AmaxCacheC(None, None, 50)
    assert lib.amax_cache_update(ctypes.byref(c), 0, ctypes.c_void_p(16), None) == _lib.FP4_EINVAL
    c = _lib.AmaxCacheC(16, 16, 0)
    assert lib.amax_cache_update(ctypes.byref(c), 0, ctypes.c_void_p(16), None) == _lib.FP4_EINVAL
    assert lib.fp4_debug_encode(None, None, 10, 0, None, None) == _lib.FP4_EINVAL
    assert lib.fp4_tensor_amax(ctypes.c_void_p(16), 0, 64, 64, 64, 8, ctypes.c_void_p(16), None) == _lib.FP4_EINVAL


def test_binding_fails_loudly_without_gpu_tensors():
    import numpy as np
    import torch
    import fp4_block_scaled_tensor_amd as fp4
    with pytest.raises(ValueError, match="device tensors"):
        fp4.quantize(torch.zeros((16, 64), dtype=torch.bfloat16), fp4.UE5M3, 16, fp4.ROW,
                     amax=torch.ones(1))


def rowcol(lib, cr, cc, rows=64, cols=64, ld=64, x=4096, q=4096, qt=4096, a_r=16, a_c=16, st_r=None, st_c=None):
    P = ctypes.c_void_p(4096)
    return lib.fp4_quantize_rowcol(ctypes.c_void_p(x), 0, rows, cols, ld, ctypes.byref(cr), ctypes.byref(cc),
                                   ctypes.c_void_p(a_r), ctypes.c_void_p(a_c), ctypes.c_void_p(q), P, None, None,
                                   ctypes.c_void_p(qt), P, None, None, st_r, st_c, None)


def test_rowcol_rejects_bad_arguments(lib):
    r, c = cfg(view=0), cfg(view=1, hn=16)
    assert rowcol(lib, c, c) == _lib.FP4_EINVAL                       # first cfg must be ROW
    assert rowcol(lib, r, r) == _lib.FP4_EINVAL                       # second cfg must be COL
    assert rowcol(lib, r, cfg(view=1, block=32)) == _lib.FP4_EUNSUPPORTED   # same block
    assert rowcol(lib, r, cfg(view=1, fmt=1)) == _lib.FP4_EUNSUPPORTED      # same format
    assert rowcol(lib, cfg(view=0, hn=16), c) == _lib.FP4_EUNSUPPORTED      # Hadamard is COL-only
    assert rowcol(lib, r, c, rows=40) == _lib.FP4_EINVAL                    # rows % B (COL)
    assert rowcol(lib, r, c, cols=40, ld=40) == _lib.FP4_EINVAL             # cols % B (ROW)
    assert rowcol(lib, r, cfg(view=1, hn=32), rows=48) == _lib.FP4_EINVAL   # rows % hadamard_n
    assert rowcol(lib, r, c, qt=0) == _lib.FP4_EINVAL                       # q_t required
    assert rowcol(lib, r, c, q=4100) == _lib.FP4_EALIGN
    assert rowcol(lib, r, c, ld=68) == _lib.FP4_EALIGN
    assert rowcol(lib, r, c, a_c=0) == _lib.FP4_EINVAL                      # UE5M3 needs both amax values
    assert rowcol(lib, r, c, rows=(1 << 24) + 32) == _lib.FP4_EUNSUPPORTED  # 32-bit in-tile offsets
    mr, mc = cfg(fmt=2, block=32, view=0, T=0.0), cfg(fmt=2, block=32, view=1, T=0.0)
    assert rowcol(lib, mr, mc, rows=48) == _lib.FP4_EINVAL                  # 48 % 32
    assert rowcol(lib, r, c, st_c=ctypes.c_void_p(4098)) == _lib.FP4_EALIGN  # health counts are words
    assert lib.fp4_last_error().decode()


def test_fake_quant_and_dequantize_reject_bad_arguments(lib):
    P = ctypes.c_void_p(4096)
    fq = lambda c, rows=64, cols=64, ld=64, ydt=0, ldy=64, y=P, amax=P: lib.fp4_fake_quant(
        P, 0, rows, cols, ld, ctypes.byref(c), amax, y, ydt, ldy, None)
    assert fq(cfg(view=1)) == _lib.FP4_EUNSUPPORTED                 # ROW view only
    assert fq(cfg(sr=1)) == _lib.FP4_EUNSUPPORTED                   # nearest-even only
    assert fq(cfg(), cols=40, ld=40, ldy=40) == _lib.FP4_EINVAL    # cols % B
    assert fq(cfg(), ydt=5) == _lib.FP4_EINVAL
    assert fq(cfg(), ldy=32) == _lib.FP4_EINVAL                    # ldy < cols
    assert fq(cfg(), y=ctypes.c_void_p(4100)) == _lib.FP4_EALIGN
    assert fq(cfg(), ldy=68) == _lib.FP4_EALIGN                    # 68 * 2 bytes
    assert fq(cfg(), amax=None) == _lib.FP4_EINVAL                 # UE5M3 needs the cached amax
    y = ctypes.c_void_p(4096)
    assert lib.fp4_dequantize(ctypes.byref(op(k=96)), y, 0, 96, None) == _lib.FP4_EINVAL          # K % 64
    assert lib.fp4_dequantize(ctypes.byref(op()), y, 7, 128, None) == _lib.FP4_EINVAL
    assert lib.fp4_dequantize(ctypes.byref(op()), y, 0, 64, None) == _lib.FP4_EINVAL             # ldy < k
    assert lib.fp4_dequantize(ctypes.byref(op()), None, 0, 128, None) == _lib.FP4_EINVAL
    assert lib.fp4_dequantize(ctypes.byref(op(fmt=2, block=32, layout=1)), y, 0, 128, None) == _lib.FP4_EUNSUPPORTED
    assert lib.fp4_last_error().decode()


def test_mxfp4_to_fp8_rejects_bad_arguments(lib):
    P = ctypes.c_void_p(4096)
    mx = lambda **kw: op(fmt=2, block=32, **kw)
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(op()), 0, P, P, None) == _lib.FP4_EUNSUPPORTED       # not MXFP4
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(mx(k=192)), 0, P, P, None) == _lib.FP4_EINVAL        # k % 128
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(mx(rows=40)), 1, P, P, None) == _lib.FP4_EINVAL      # rows % 16
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(mx()), 2, P, P, None) == _lib.FP4_EINVAL
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(mx()), 0, None, P, None) == _lib.FP4_EINVAL
    assert lib.fp4_mxfp4_to_fp8(ctypes.byref(mx()), 0, ctypes.c_void_p(4104), P, None) == _lib.FP4_EALIGN
    assert lib.fp4_last_error().decode()


def test_quantize_local_and_stripe_operands_reject_bad_arguments(lib):
    P = ctypes.c_void_p(4096)
    ql = lambda c, stripe=16, rows=64, cols=64: lib.fp4_quantize_local(P, 0, rows, cols, cols, ctypes.byref(c), stripe,
                                                                        P, P, P, None, None)
    assert ql(cfg(fmt=1), stripe=8) == _lib.FP4_EINVAL
    assert ql(cfg(fmt=2, block=32)) == _lib.FP4_EUNSUPPORTED        # E8M0 has no tensor scale
    assert ql(cfg(fmt=1, view=1)) == _lib.FP4_EUNSUPPORTED          # ROW view only
    assert ql(cfg(fmt=1), cols=40) == _lib.FP4_EINVAL               # cols % B
    y = ctypes.c_void_p(4096)
    a = _lib.Operand(4096, 4096, 4096, 1, 16, 0, 24, 64, 128)       # g_stripe 24
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(op(fmt=1)), y, 0, None) == _lib.FP4_EINVAL
    a = _lib.Operand(4096, 4096, 4096, 2, 32, 0, 16, 64, 128)       # MXFP4 with a stripe g
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(op(fmt=2, block=32)), y, 0, None) == _lib.FP4_EUNSUPPORTED
    a = _lib.Operand(4096, 4096, None, 1, 16, 0, 32, 64, 128)       # stripe g without the array
    assert lib.fp4_gemm_fprop(ctypes.byref(a), ctypes.byref(op(fmt=1)), y, 0, None) == _lib.FP4_EINVAL


def test_gemm_check_range_bounds(lib):
    """Host-only range check of the MXFP4 GEMM (no launch): combined exponents Ea + Eb in
    [-124, 116] pass, one step outside either edge is FP4_ERANGE; UE5M3/E4M3 always pass."""
    R = lambda lo, hi: (ctypes.c_int32 * 2)(lo, hi)
    E8, UE = _lib.FP4_E8M0, _lib.FP4_UE5M3
    assert lib.fp4_gemm_check_range(E8, R(120, 140), R(110, 130)) == _lib.FP4_OK
    assert lib.fp4_gemm_check_range(E8, R(65, 185), R(65, 185)) == _lib.FP4_OK        # -124 .. +116 exactly
    assert lib.fp4_gemm_check_range(E8, R(64, 185), R(65, 185)) == _lib.FP4_ERANGE    # -125
    assert "-125" in lib.fp4_last_error().decode()
    assert lib.fp4_gemm_check_range(E8, R(65, 186), R(65, 185)) == _lib.FP4_ERANGE    # +117
    assert lib.fp4_gemm_check_range(E8, R(0, 254), R(127, 127)) == _lib.FP4_ERANGE
    assert lib.fp4_gemm_check_range(E8, R(255, 0), R(0, 254)) == _lib.FP4_OK          # an empty operand
    assert lib.fp4_gemm_check_range(UE, R(0, 247), R(0, 247)) == _lib.FP4_OK
    assert lib.fp4_gemm_check_range(E8, R(10, 5), R(0, 1)) == _lib.FP4_EINVAL
    assert lib.fp4_gemm_check_range(E8, None, R(0, 1)) == _lib.FP4_EINVAL
    assert lib.fp4_scale_range(None, ctypes.c_void_p(16), None) == _lib.FP4_EINVAL


def test_exact_range_edges_match_the_oracle_contract():
    """The check's edges against the oracle model: at combined exponents -124 and +116 the
    smallest and largest block partials and group sums are normal float32 numbers and the
    oracle's result for worst-case operands is finite and exact; at +117 the largest group sum
    (two block partials of 1152 * 2^117) overflows float32; at -125 the smallest partial is
    subnormal."""
    import numpy as np
    import oracle
    q6 = np.full((1, 64), 6.0)
    qh = np.full((1, 64), 0.5)
    for e, ok in ((116, True), (117, False)):
        sa = np.full((1, 2), 2.0 ** (e // 2))
        sb = np.full((1, 2), 2.0 ** (e - e // 2))
        if ok:
            y = oracle.gemm_model(q6, sa, q6, sb, 32)
            assert np.isfinite(y).all() and y[0, 0] == np.float32(2304 * 2.0 ** e)
        else:
            with np.errstate(over="ignore"):
                assert not np.isfinite(oracle.gemm_model(q6, sa, q6, sb, 32)).any()
    tiny = lambda e: 0.25 * 2.0 ** e
    assert tiny(-124) == 2.0 ** -126 and tiny(-125) < 2.0 ** -126


def test_quantized_output_gemms_reject_bad_arguments(lib):
    """fp4_gemm_fprop_q / fp4_gemm_dgrad_q: every argument error returns its status before
    anything is launched (no GPU here)."""
    P = ctypes.c_void_p
    y, q, s, g, amax = P(4096), P(8192), P(12288), P(16384), P(20480)

    def cfg(fmt=0, block=16, view=0, sr=0, hn=0, T=448.0):
        return _lib.QuantCfg(fmt, block, view, sr, hn, T, 0, 0)

    def call(name, a, b, c, amx=amax, qq=q, ss=s, yy=y):
        return getattr(lib, name)(ctypes.byref(a), ctypes.byref(b), yy, 0, ctypes.byref(c), amx, qq, ss, g, None,
                                  None, None)
    a, b = op(), op()
    for name in ("fp4_gemm_fprop_q", "fp4_gemm_dgrad_q"):
        assert call(name, a, b, cfg(view=1)) == _lib.FP4_EUNSUPPORTED                  # COL view of C
        assert call(name, a, b, cfg(hn=16)) == _lib.FP4_EUNSUPPORTED                  # rotation
        assert call(name, a, b, cfg(block=8)) != _lib.FP4_OK                          # bad block
        assert call(name, a, b, cfg(), qq=None) == _lib.FP4_EINVAL                    # NULL payload
        assert call(name, a, b, cfg(), ss=None) == _lib.FP4_EINVAL                    # NULL scales
        assert call(name, a, b, cfg(), qq=P(4100)) == _lib.FP4_EALIGN                 # payload alignment
        assert call(name, a, b, cfg(), amx=None) == _lib.FP4_EINVAL                   # UE5M3 without amax
        assert call(name, a, op(rows=72), cfg()) == _lib.FP4_EINVAL                   # N % 16
        assert call(name, op(k=0), op(k=0), cfg()) == _lib.FP4_EUNSUPPORTED           # K = 0
        assert call(name, a, op(k=192), cfg()) == _lib.FP4_EINVAL                     # K mismatch
    assert call("fp4_gemm_dgrad_q", a, op(layout=1), cfg()) == _lib.FP4_EUNSUPPORTED  # weight's forward view
    assert call("fp4_gemm_fprop_q", a, op(layout=2), cfg()) == _lib.FP4_EUNSUPPORTED  # weight's dgrad view


def test_decode_once_entry_points_reject_bad_arguments(lib):
    """fp4_decode_f16 / fp4_gemm_f16: argument errors return before any launch."""
    P = ctypes.c_void_p
    out, a16, b16, c = P(4096), P(8192), P(12288), P(16384)
    mx = op(fmt=2, block=32)
    assert lib.fp4_decode_f16(ctypes.byref(mx), out, None) == _lib.FP4_EUNSUPPORTED      # MXFP4 runs natively
    assert lib.fp4_decode_f16(ctypes.byref(op()), None, None) == _lib.FP4_EINVAL
    assert lib.fp4_decode_f16(ctypes.byref(op()), P(4104), None) == _lib.FP4_EALIGN
    assert lib.fp4_decode_f16(None, out, None) == _lib.FP4_EINVAL
    assert lib.fp4_decode_f16(ctypes.byref(op(k=96)), out, None) == _lib.FP4_EINVAL      # K % 64
    a, b = op(), op()
    f = lib.fp4_gemm_f16
    assert f(ctypes.byref(mx), a16, ctypes.byref(op(fmt=2, block=32)), b16, c, 0, 0, None) == _lib.FP4_EUNSUPPORTED
    assert f(ctypes.byref(a), None, ctypes.byref(b), b16, c, 0, 0, None) == _lib.FP4_EINVAL
    assert f(ctypes.byref(a), a16, ctypes.byref(b), P(12296), c, 0, 0, None) == _lib.FP4_EALIGN
    assert f(ctypes.byref(a), a16, ctypes.byref(b), b16, c, 8, 0, None) == _lib.FP4_EINVAL
    assert f(ctypes.byref(a), a16, ctypes.byref(op(k=192)), b16, c, 0, 0, None) == _lib.FP4_EINVAL
    assert f(ctypes.byref(a), a16, ctypes.byref(b), b16, None, 0, 0, None) == _lib.FP4_EINVAL
    assert f(ctypes.byref(a), a16, ctypes.byref(b), b16, c, 0, 2, None) == _lib.FP4_EINVAL   # canon 0/1
    assert f(ctypes.byref(op(rows=0)), None, ctypes.byref(b), None, None, 0, 0, None) == _lib.FP4_OK   # empty: no-op
