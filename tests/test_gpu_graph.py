"""Quantize + GEMM captured in a HIP graph: every replay, with eager work and synchronisations
between replays, gives the same bytes as the eager calls (the library launches only kernels on
the caller's stream: no allocation, memset or host synchronisation inside the captured calls)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt_name", ["ue5m3", "mxfp4"])
def test_graph_replays_match_eager(fmt_name):
    import fp4_block_scaled_tensor_amd as fp4
    fmt = {"ue5m3": fp4.UE5M3, "mxfp4": fp4.E8M0}[fmt_name]
    block = 32 if fmt == fp4.E8M0 else 16
    xs = synth.student_t((512, 1024), 3.0, 911)
    ws = synth.normal((384, 1024), 0.02, 912)
    X = torch.from_numpy(synth.f32_to_bf16_bits(xs).view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(synth.f32_to_bf16_bits(ws).view(np.int16)).view(torch.bfloat16).cuda()
    amax_x = fp4.tensor_amax(X)
    amax_w = fp4.tensor_amax(W)
    kw_x = {} if fmt == fp4.E8M0 else dict(amax=amax_x, T=448)
    kw_w = {} if fmt == fp4.E8M0 else dict(amax=amax_w, T=448)
    y_out = torch.empty((512, 384), dtype=torch.float32, device="cuda")

    def step():
        qx = fp4.quantize(X, fmt, block, fp4.ROW, **kw_x)
        qw = fp4.quantize(W, fmt, block, fp4.ROW, **kw_w)
        fp4.gemm_fprop(qx, qw, out=y_out)
        return qx, qw

    qx_e, qw_e = step()
    y_e = y_out.clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qx_g, qw_g = step()
    for rep in range(3):
        y_out.fill_(float("nan"))             # eager work between replays
        qx_g.q.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qx_g.q, qx_e.q) and torch.equal(qx_g.s, qx_e.s), f"replay {rep}: X payload/scales"
        assert torch.equal(qw_g.q, qw_e.q) and torch.equal(qw_g.s, qw_e.s), f"replay {rep}: W payload/scales"
        assert torch.equal(qx_g.g, qx_e.g), f"replay {rep}: g"
        assert torch.equal(y_out.view(torch.int32), y_e.view(torch.int32)), f"replay {rep}: GEMM output"
