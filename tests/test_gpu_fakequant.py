"""Inference fake quantization and operand decode: bit-exact against the oracle (float32
and bfloat16 outputs), and the activation-scale policies over an ordered request stream."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, dev_input, dev_scalar, qtensor_from_oracle

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _tensor(rows, cols, dtype, seed, scale=1.0):
    x = synth.student_t((rows, cols), 3.0, seed) * np.float32(scale)
    x, _ = synth.scale_channels(x, max(1, cols // 100), 100.0, seed + 1)
    if dtype == "bf16":
        return synth.Tensor("x", synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), "bf16")
    return synth.Tensor("x", x.astype(np.float32), dtype)


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


CASES = [
    # name, rows, cols, in dtype, fmt, block, T
    ("ue5m3", 256, 512, "bf16", OF.UE5M3, 16, 448),
    ("ue5m3_ragged", 200, 208, "bf16", OF.UE5M3, 16, 448),
    ("e4m3_b32_fp32", 96, 160, "fp32", OF.E4M3, 32, 448),
    ("mx", 130, 96, "bf16", OF.E8M0, 32, 0),
    ("ue5m3_T2048", 64, 1024, "bf16", OF.UE5M3, 16, 2048),
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("name,rows,cols,dtype,fmt,block,T", CASES, ids=[c[0] for c in CASES])
def test_fake_quant_matches_oracle(name, rows, cols, dtype, fmt, block, T, out):
    t = _tensor(rows, cols, dtype, 7000 + rows + cols)
    A = oracle.tensor_amax(t.values)
    want = oracle.fake_quant(t.values, fmt, block, amax=A, T=T, out=out)
    y = fp4.fake_quant(dev_input(t), fmt, block, amax=dev_scalar(A), T=T,
                       out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    got = _bits(y)
    want_bits = want.view(np.uint32) if out == "f32" else want
    assert_bytes_equal(torch.from_numpy(got.view(np.uint8)), want_bits.view(np.uint8), f"{name} {out}")


def test_fake_quant_stale_amax_saturates_like_oracle():
    t = _tensor(64, 256, "bf16", 71)
    for A in (oracle.tensor_amax(t.values) * np.float32(1e-3), np.float32(0.0)):
        want = oracle.fake_quant(t.values, OF.UE5M3, 16, amax=A, T=448)
        y = fp4.fake_quant(dev_input(t), fp4.UE5M3, 16, amax=dev_scalar(A), T=448)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32)), A


def test_fake_quant_strided_into_wider_output():
    t = _tensor(128, 320, "bf16", 72)
    full = dev_input(t)
    x = full[:, 64:256]
    A = oracle.tensor_amax(t.values[:, 64:256])
    outbuf = torch.full((128, 256), -7.0, dtype=torch.float32, device="cuda")
    fp4.fake_quant(x, fp4.UE5M3, 16, amax=dev_scalar(A), out=outbuf[:, 32:224])
    torch.cuda.synchronize()
    want = oracle.fake_quant(t.values[:, 64:256], OF.UE5M3, 16, amax=A)
    got = outbuf.cpu().numpy()
    assert np.array_equal(got[:, 32:224].view(np.uint32), want.view(np.uint32))
    assert np.all(got[:, :32] == -7.0) and np.all(got[:, 224:] == -7.0)


def test_fake_quant_full_size_activation_sampled():
    """8192 x 4096 activation (Student-t, outlier channels), bf16 out, the launch the bench
    times; 256 rows checked against the oracle."""
    X = synth.make_config(3, rows=8192)["X"]
    A = oracle.tensor_amax(X.values)
    y = fp4.fake_quant(dev_input(X), fp4.UE5M3, 16, amax=dev_scalar(A), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.r_[0:128, 8064:8192]
    want = oracle.fake_quant(X.values[rows], OF.UE5M3, 16, amax=A, out="bf16")
    assert np.array_equal(_bits(y[torch.from_numpy(rows).cuda()]), want)


@pytest.mark.parametrize("view", ["1d", "2d", "2dT"])
@pytest.mark.parametrize("fmt", [OF.UE5M3, OF.E4M3, OF.E8M0])
def test_dequantize_matches_oracle(view, fmt):
    if fmt == OF.E8M0 and view != "1d":
        pytest.skip("2D tiles use UE5M3 or E4M3 scales")
    x = _tensor(192, 256, "fp32", 73).values
    A = oracle.tensor_amax(x)
    block = 32 if fmt == OF.E8M0 else 16
    qr = oracle.quantize_1d(x, fmt, block, amax=A) if view == "1d" else oracle.quantize_2d(x, fmt, amax=A)
    if view == "2dT":
        qr_view = oracle.QuantResult(np.ascontiguousarray(qr.codes.T), qr.scales, qr.g, qr.fmt, 16)
    else:
        qr_view = qr
    qt = qtensor_from_oracle(qr, view)
    for dt, conv in ((torch.float32, lambda a: a.view(np.uint32)), (torch.bfloat16, oracle.f32_to_bf16_bits)):
        y = fp4.dequantize(qt, out_dtype=dt)
        torch.cuda.synchronize()
        want = conv(oracle.dequantize(qr_view, view))
        assert np.array_equal(_bits(y), want), (view, dt)


def test_dequantize_of_library_quantization_equals_fake_quant():
    t = _tensor(256, 512, "bf16", 74)
    x = dev_input(t)
    A = dev_scalar(oracle.tensor_amax(t.values))
    q = fp4.quantize(x, fp4.UE5M3, 16, fp4.ROW, amax=A)
    d = fp4.dequantize(q)
    f = fp4.fake_quant(x, fp4.UE5M3, 16, amax=A)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int32), f.view(torch.int32))


@pytest.mark.parametrize("kind,D", [("delayed", 2), ("current", None), ("frozen", None)])
def test_policy_request_stream_matches_oracle(kind, D):
    reqs = [_tensor(64, 256, "bf16", 80 + i, scale=s).values for i, s in enumerate([1.0, 300.0, 0.01, 1.0, 50.0])]
    kw = dict(amax=3.0) if kind == "frozen" else {}
    ref = oracle.FakeQuantPolicy(kind, D=D, **kw)
    pol = fp4.FakeQuantPolicy(kind, fp4.UE5M3, 16, D=D, **kw)
    for i, x in enumerate(reqs):
        want = ref(i, x, OF.UE5M3, 16)
        got = pol(i, torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), (kind, i)
