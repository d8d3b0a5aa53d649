"""Parity at the remaining workloads' real shapes, against the oracle.

- Nemotron-H-8B down_proj backward (dY [8192 x 4096], W [4096 x 21504], X [8192 x 21504]):
  the fused ROW+COL quantizer for dY (SR, T = 448 / 2048), the weight's dgrad view, and
  dgrad and wgrad computed in full on the GPU; sampled output blocks (row slices x column
  slices) against the oracle's group model, whose operands are quantized from the matching
  slices (the SR draws indexed by the slices' logical positions, 2D tiles aligned to 16).
- 8B layer linear set (qkv, o, gate+up, down) over steps 0, 1 and 50 of a D = 50 amax
  cache per operand, with and without H16 on the wgrad operands, at 256 tokens: the device
  caches against the oracle's, every activation / gradient byte, and sampled output blocks
  of the three GEMMs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, assert_f32_bits_equal, dev_input, dev_scalar

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _block(qa, qb, va="1d", vb="1d", hadamard_n=0):
    a, sa = oracle.operand_from_quant(qa, va)
    b, sb = oracle.operand_from_quant(qb, vb)
    return oracle.gemm_model(a, sa, b, sb, qa.block, alpha=oracle.output_scale(qa.g, qb.g, hadamard_n))


def _row_slices(x, fmt, block, slices, **kw):
    """Oracle ROW view of the given row slices of x (SR index base = each slice's first row)."""
    return [oracle.quantize_1d(x[r0:r1], fmt, block, row0=r0, **kw) for r0, r1 in slices]


def _col_slices(x, fmt, block, slices, hadamard_n=0, **kw):
    """Oracle COL view (rows = features of x) of the given feature slices."""
    return [oracle.quantize_1d(oracle.transposed_view(x[:, f0:f1], hadamard_n), fmt, block, row0=f0, **kw)
            for f0, f1 in slices]


def _w_slices_2d(w, fmt, amax, slices, axis):
    """Oracle 2D quantization of 16-aligned slices of W along rows (axis 0, forward view rows)
    or columns (axis 1, dgrad view rows) with the whole tensor's amax."""
    out = []
    for a0, a1 in slices:
        assert a0 % 16 == 0 and a1 % 16 == 0
        part = w[a0:a1] if axis == 0 else w[:, a0:a1]
        out.append(oracle.quantize_2d(part, fmt, amax=amax, T=448))
    return out


def _rows(t, slices):
    return torch.cat([t[r0:r1] for r0, r1 in slices]).cpu().numpy()


@pytest.fixture(scope="module")
def down_proj():
    cfg = synth.make_config(4)
    return cfg, {k: dev_input(v) for k, v in cfg.items()}


@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E8M0], ids=["ue5m3", "mxfp4"])
def test_down_proj_backward_full_size_sampled(down_proj, fmt):
    cfg, dev = down_proj
    dY, W, X = cfg["dY"].values, cfg["W"].values, cfg["X"].values
    E8 = fmt == OF.E8M0
    B = 32 if E8 else 16
    Ady = None if E8 else oracle.tensor_amax(dY)
    Ax = None if E8 else oracle.tensor_amax(X)
    Aw = None if E8 else oracle.tensor_amax(W)
    am = (lambda A: None) if E8 else dev_scalar
    qdy, qdyt = fp4.quantize_rowcol(dev["dY"], fmt, B, amax_row=am(Ady), amax_col=am(Ady), T_row=448, T_col=2048,
                                    stochastic_row=True, stochastic_col=True, seed_row=42, offset_row=0, seed_col=42,
                                    offset_col=1)
    if E8:
        _, qwt = fp4.quantize_rowcol(dev["W"], fmt, B)
    else:
        _, qwt = fp4.quantize(dev["W"], fmt, 16, fp4.TILE2D, amax=dev_scalar(Aw), T=448)
    qxt = fp4.quantize(dev["X"], fmt, B, fp4.COL, amax=am(Ax), T=448)
    dx = fp4.gemm_dgrad(qdy, qwt)           # [8192 x 21504], K = 4096
    dw = fp4.gemm_wgrad(qdyt, qxt)          # [4096 x 21504], K = 8192
    torch.cuda.synchronize()

    tok = [(0, 4), (4096, 4100), (8188, 8192)]
    feat_out = [(0, 4), (2000, 2004), (4092, 4096)]
    feat_in = [(0, 64), (10752, 10816), (21440, 21504)]
    sr_row = dict(amax=Ady, T=448, rounding="sr", seed=42, offset=0)
    sr_col = dict(amax=Ady, T=2048, rounding="sr", seed=42, offset=1)
    # quantized bytes of the sampled slices
    for (r0, r1), rq in zip(tok, _row_slices(dY, fmt, B, tok, **sr_row)):
        assert_bytes_equal(qdy.q[r0:r1], rq.packed, f"dY ROW rows {r0}")
        assert_bytes_equal(qdy.s[r0:r1], rq.scales, f"dY ROW scales rows {r0}")
    for (f0, f1), rq in zip(feat_out, _col_slices(dY, fmt, B, feat_out, **sr_col)):
        assert_bytes_equal(qdyt.q[f0:f1], rq.packed, f"dY COL features {f0}")
        assert_bytes_equal(qdyt.s[f0:f1], rq.scales, f"dY COL scales features {f0}")
    # dgrad blocks: rows = token slices, cols = input-feature slices (rows of the W^T view)
    a_parts = _row_slices(dY, fmt, B, tok, **sr_row)
    if E8:
        b_parts = _col_slices(W, fmt, B, feat_in)
    else:
        b_parts = _w_slices_2d(W, fmt, Aw, feat_in, axis=1)
    got = _rows(dx, tok)
    for (c0, c1), bq in zip(feat_in, b_parts):
        want = np.concatenate([_block(aq, bq, vb="1d" if E8 else "2dT") for aq in a_parts])
        assert_f32_bits_equal(got[:, c0:c1], want, f"dgrad cols {c0}:{c1}")
    # wgrad blocks: rows = output-feature slices, cols = input-feature slices (rows of X^T)
    a_parts = _col_slices(dY, fmt, B, feat_out, **sr_col)
    b_parts = _col_slices(X, fmt, B, feat_in, amax=Ax, T=448)
    got = _rows(dw, feat_out)
    for (c0, c1), bq in zip(feat_in, b_parts):
        want = np.concatenate([_block(aq, bq) for aq in a_parts])
        assert_f32_bits_equal(got[:, c0:c1], want, f"wgrad cols {c0}:{c1}")


TOKENS = 256
STEPS = (0, 1, 50)


@pytest.mark.parametrize("layer", range(len(synth.LINEARS_8B)), ids=[n for n, _, _ in synth.LINEARS_8B])
def test_layer_set_steps_with_amax_caches(layer):
    name, in_f, out_f = synth.LINEARS_8B[layer]
    U = OF.UE5M3
    Wt = synth.layer_weight(layer, out_f, in_f)
    W = Wt.values
    Wd = dev_input(Wt)
    HNS = (0, 16)
    gpu = {k: fp4.AmaxCache(50) for k in ("x", "w", "dy")}
    ref = {k: oracle.AmaxCache(50) for k in ("x", "w", "dy")}
    for hn in HNS:
        gpu[f"xh{hn}"], gpu[f"dyh{hn}"] = fp4.AmaxCache(50), fp4.AmaxCache(50)
        ref[f"xh{hn}"], ref[f"dyh{hn}"] = oracle.AmaxCache(50), oracle.AmaxCache(50)
    obs = torch.empty(1, dtype=torch.float32, device="cuda")

    def sample(key, xd, x, step, hn=0):
        if gpu[key].needs_sample(step):
            fp4.tensor_amax(xd, hn, out=obs)
            gpu[key].update(step, obs)
        ref[key].update(step, oracle.tensor_amax(x, hn))
        torch.cuda.synchronize()
        assert gpu[key].amax.item() == ref[key].amax, f"{name} step {step} cache {key}"
        return gpu[key].amax, ref[key].amax

    rows_n = [(0, 16), (out_f - 16, out_f)]        # forward-view W rows = output columns
    rows_k = [(0, 16), (in_f - 16, in_f)]          # dgrad-view W rows = input columns
    for step in STEPS:
        inp = synth.layer_step_inputs(layer, step, TOKENS, in_f, out_f)
        X, dY = inp["X"].values, inp["dY"].values
        Xd, dYd = dev_input(inp["X"]), dev_input(inp["dY"])
        gx, rx_a = sample("x", Xd, X, step)
        gw, rw_a = sample("w", Wd, W, step)
        gdy, rdy_a = sample("dy", dYd, dY, step)
        # forward
        qx = fp4.quantize(Xd, U, 16, fp4.ROW, amax=gx, T=448)
        qw, qwt = fp4.quantize(Wd, U, 16, fp4.TILE2D, amax=gw, T=448)
        y = fp4.gemm_fprop(qx, qw)
        # dgrad (SR dY, offsets separate steps and views)
        qdy = fp4.quantize(dYd, U, 16, fp4.ROW, amax=gdy, T=448, stochastic=True, seed=42, offset=step * 8)
        dx = fp4.gemm_dgrad(qdy, qwt)
        torch.cuda.synchronize()
        rx = oracle.quantize_1d(X, U, 16, amax=rx_a, T=448)
        rdy = oracle.quantize_1d(dY, U, 16, amax=rdy_a, T=448, rounding="sr", seed=42, offset=step * 8)
        assert_bytes_equal(qx.q, rx.packed, f"{name} step {step} X payload")
        assert_bytes_equal(qx.s, rx.scales, f"{name} step {step} X scales")
        assert_bytes_equal(qdy.q, rdy.packed, f"{name} step {step} dY payload")
        assert_bytes_equal(qdy.s, rdy.scales, f"{name} step {step} dY scales")
        tok = slice(0, 8)
        for (n0, n1), rwq in zip(rows_n, _w_slices_2d(W, U, rw_a, rows_n, axis=0)):
            assert_bytes_equal(qw.q[n0:n1], rwq.packed, f"{name} step {step} W rows {n0}")
            rxs = oracle.quantize_1d(X[tok], U, 16, amax=rx_a, T=448)
            assert_f32_bits_equal(y[tok, n0:n1], _block(rxs, rwq, vb="2d"), f"{name} step {step} fprop cols {n0}")
        for (k0, k1), rwq in zip(rows_k, _w_slices_2d(W, U, rw_a, rows_k, axis=1)):
            rdys = oracle.quantize_1d(dY[tok], U, 16, amax=rdy_a, T=448, rounding="sr", seed=42, offset=step * 8)
            assert_f32_bits_equal(dx[tok, k0:k1], _block(rdys, rwq, vb="2dT"), f"{name} step {step} dgrad cols {k0}")
        # wgrad, with and without H16 on both operands (their own caches)
        for hn in HNS:
            gdyh, rdyh_a = sample(f"dyh{hn}", dYd, dY, step, hn)
            gxh, rxh_a = sample(f"xh{hn}", Xd, X, step, hn)
            qdyt = fp4.quantize(dYd, U, 16, fp4.COL, amax=gdyh, T=2048, stochastic=True, seed=42, offset=step * 8 + 1,
                                hadamard_n=hn)
            qxt = fp4.quantize(Xd, U, 16, fp4.COL, amax=gxh, T=448, hadamard_n=hn)
            dw = fp4.gemm_wgrad(qdyt, qxt, hadamard_n=hn)
            torch.cuda.synchronize()
            rdyt = oracle.quantize_col(dY, U, 16, amax=rdyh_a, T=2048, rounding="sr", seed=42, offset=step * 8 + 1,
                                       hadamard_n=hn)
            rxt = oracle.quantize_col(X, U, 16, amax=rxh_a, T=448, hadamard_n=hn)
            assert_bytes_equal(qdyt.q, rdyt.packed, f"{name} step {step} H{hn} dY^T payload")
            assert_bytes_equal(qxt.q, rxt.packed, f"{name} step {step} H{hn} X^T payload")
            assert_bytes_equal(qxt.s, rxt.scales, f"{name} step {step} H{hn} X^T scales")
            fo = slice(0, 8)
            a, sa = oracle.operand_from_quant(rdyt)
            b, sb = oracle.operand_from_quant(rxt)
            want = oracle.gemm_model(a[fo], sa[fo], b[:64], sb[:64], 16,
                                     alpha=oracle.output_scale(rdyt.g, rxt.g, hn))
            assert_f32_bits_equal(dw[fo, :64], want, f"{name} step {step} H{hn} wgrad")
