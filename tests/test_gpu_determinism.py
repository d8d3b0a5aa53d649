"""Determinism at full size: the same call gives the same bits on every run, and different
kernels, tilings and grids over the same operands give the same bits.

Inputs are the up-projection shapes of an 8B model (8192 tokens, hidden 4096, MLP 14336) in
bf16, seeded Gaussian. Stochastic rounding draws from a counter-based generator keyed by
(seed, offset, element index), and every reduction (amax, health counts, the GEMMs'
K-ordered group accumulation) is order-fixed or order-free (max, integer adds), so repeats
must be bit-identical. Across routes: the UE5M3 GEMM runs either with a per-workgroup decode
or on operands decoded once to fp16, with different tiles; a GEMM on a row slice of A runs a
different grid with a ragged tail. All must agree bit for bit (the values themselves are
checked against the oracle elsewhere).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")

M, N, K = 8192, 14336, 4096


def _gauss(shape, std, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16).cuda()


@pytest.fixture(scope="module")
def data():
    return {"x": _gauss((M, K), 1.0, 1), "w": _gauss((N, K), 0.02, 2), "dy": _gauss((M, N), 1e-3, 3)}


def _same(a: torch.Tensor, b: torch.Tensor, what: str):
    torch.cuda.synchronize()
    assert a.shape == b.shape and a.dtype == b.dtype, what
    if a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    ne = int((a != b).sum())
    assert ne == 0, f"{what}: {ne} of {a.numel()} differ"


def _same_q(p, q, what):
    for f in ("q", "s", "g"):
        _same(getattr(p, f), getattr(q, f), f"{what} {f}")


def test_quantizers_repeat_bit_identical(data):
    x, w, dy = data["x"], data["w"], data["dy"]
    ax, aw, ad = fp4.tensor_amax(x), fp4.tensor_amax(w), fp4.tensor_amax(dy, hadamard_n=16)

    def run():
        st = [fp4.new_stats() for _ in range(5)]
        obs = [torch.zeros(1, dtype=torch.float32, device="cuda") for _ in range(3)]
        xr = fp4.quantize(x, fp4.UE5M3, 16, fp4.ROW, amax=ax, T=448, stats=st[0], amax_obs=obs[0])
        xc = fp4.quantize(x, fp4.UE5M3, 16, fp4.COL, amax=ax, T=448, stochastic=True, seed=7, offset=3,
                          hadamard_n=16, stats=st[1])
        wf, wt = fp4.quantize(w, fp4.UE5M3, 16, fp4.TILE2D, amax=aw, T=448, stats=st[2], amax_obs=obs[1])
        dr, dc = fp4.quantize_rowcol(dy, fp4.UE5M3, 16, amax_row=ad, amax_col=ad, T_col=2048.0, stochastic_row=True,
                                     stochastic_col=True, seed_row=11, seed_col=12, offset_row=5, offset_col=6,
                                     hadamard_n=16, stats_row=st[3], stats_col=st[4], amax_obs_row=obs[2])
        mx = fp4.quantize(x, fp4.E8M0, 32, fp4.ROW, stochastic=True, seed=9, offset=1)
        return [xr, xc, wf, wt, dr, dc, mx], st, obs

    q1, s1, o1 = run()
    q2, s2, o2 = run()
    names = ["x ROW", "x COL H16 SR", "w 2D", "w 2D^T", "dY ROW SR", "dY COL H16 SR", "x MXFP4 SR"]
    for name, a, b in zip(names, q1, q2):
        _same_q(a, b, name)
    for i, (a, b) in enumerate(zip(s1, s2)):
        _same(a, b, f"stats {i}")
    for i, (a, b) in enumerate(zip(o1, o2)):
        _same(a, b, f"amax_obs {i}")


@pytest.mark.parametrize("fmt", ["ue5m3", "mxfp4"])
def test_gemm_repeats_routes_and_grids_bit_identical(data, fmt):
    x, w = data["x"], data["w"]
    if fmt == "mxfp4":
        qx = fp4.quantize(x, fp4.E8M0, 32, fp4.ROW)
        qw = fp4.quantize(w, fp4.E8M0, 32, fp4.ROW)
    else:
        qx = fp4.quantize(x, fp4.UE5M3, 16, fp4.ROW, amax=fp4.tensor_amax(x), T=448)
        qw, _ = fp4.quantize(w, fp4.UE5M3, 16, fp4.TILE2D, amax=fp4.tensor_amax(w), T=448)
    y1 = fp4.gemm_fprop(qx, qw)
    y2 = fp4.gemm_fprop(qx, qw)
    _same(y1, y2, f"{fmt} fprop repeat")
    del y2
    if fmt == "ue5m3":
        y3 = fp4.gemm_f16(qx, qw)          # decode-once route: other kernel, other tiles
        _same(y1, y3, "ue5m3 fprop vs decode-once")
        del y3
    # a row slice of A: a smaller grid with a ragged tail (1000 = 7 x 128 + 104 rows)
    m0, m1 = 3072, 4072
    qs = fp4.QTensor(qx.q[m0:m1], qx.s[m0:m1], qx.g, qx.fmt, qx.block, fp4.FP4_SCALES_1D, m1 - m0, qx.k)
    ys = fp4.gemm_fprop(qs, qw)
    _same(ys, y1[m0:m1], f"{fmt} fprop row slice")
    if fmt == "ue5m3":
        _same(fp4.gemm_f16(qs, qw), y1[m0:m1], "ue5m3 decode-once row slice")


def test_backward_routes_bit_identical(data):
    """dgrad and wgrad (H16): the per-workgroup-decode and the decode-once kernels agree."""
    x, w, dy = data["x"], data["w"], data["dy"]
    aw, ad, ax16 = fp4.tensor_amax(w), fp4.tensor_amax(dy, hadamard_n=16), fp4.tensor_amax(x, hadamard_n=16)
    _, wt = fp4.quantize(w, fp4.UE5M3, 16, fp4.TILE2D, amax=aw, T=448)
    dr, dc = fp4.quantize_rowcol(dy, fp4.UE5M3, 16, amax_row=ad, amax_col=ad, stochastic_row=True,
                                 stochastic_col=True, seed_row=1, seed_col=2, hadamard_n=16)
    xc = fp4.quantize(x, fp4.UE5M3, 16, fp4.COL, amax=ax16, T=448, hadamard_n=16)
    dx = fp4.gemm_dgrad(dr, wt)
    _same(dx, fp4.gemm_f16(dr, wt), "dgrad vs decode-once")
    del dx
    dw = fp4.gemm_wgrad(dc, xc, hadamard_n=16)
    _same(dw, fp4.gemm_f16(dc, xc, hadamard_n=16), "wgrad H16 vs decode-once")
    _same(dw, fp4.gemm_wgrad(dc, xc, hadamard_n=16), "wgrad H16 repeat")
