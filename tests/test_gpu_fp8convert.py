"""MXFP4 -> FP8 E4M3 conversion (row-major and transposed): bit-exact against the oracle,
including stress operands whose blocks span wide exponent ranges and ragged row counts."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests._helpers import assert_bytes_equal, dev_input, random_operand

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("fp4_block_scaled_tensor_amd")


def _qtensor(codes, scales):
    rows, k = codes.shape
    q = torch.from_numpy(oracle.pack_codes(codes)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    return fp4.QTensor(q, s, g, fp4.E8M0, 32, fp4.FP4_SCALES_1D, rows, k)


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("rows,k,spread", [(128, 256, 2), (208, 384, 10), (48, 128, 30), (16, 1024, 0)])
def test_random_operands_match_oracle(rows, k, spread, transpose):
    rng = np.random.default_rng(900 + rows + k + spread)
    qr = random_operand(rng, rows, k, OF.E8M0, 32, spread, zero_frac=0.1)
    codes, scales = qr.codes, qr.scales
    want_y, want_s = oracle.mxfp4_to_fp8(codes, scales, transpose=transpose)
    y, s8 = fp4.mxfp4_to_fp8(_qtensor(codes, scales), transpose=transpose)
    torch.cuda.synchronize()
    assert_bytes_equal(y, want_y, "fp8 codes")
    assert_bytes_equal(s8, want_s, "chunk scales")


def test_extreme_block_codes():
    """Block codes at 0 and 254 and every gap 0..20 to the chunk maximum."""
    rng = np.random.default_rng(91)
    rows, k = 64, 128 * 8
    codes = rng.integers(0, 16, (rows, k)).astype(np.uint8)
    scales = np.empty((rows, k // 32), np.uint8)
    for r in range(rows):
        for c in range(k // 128):
            top = [254, 3, 127, 20][(r + c) % 4]
            gaps = [0, (r * 3 + c) % 21, (r + 5 * c) % 17, r % 9]
            scales[r, 4 * c:4 * c + 4] = np.clip(top - np.array(gaps), 0, 254)
    for transpose in (False, True):
        want_y, want_s = oracle.mxfp4_to_fp8(codes, scales, transpose=transpose)
        y, s8 = fp4.mxfp4_to_fp8(_qtensor(codes, scales), transpose=transpose)
        torch.cuda.synchronize()
        assert_bytes_equal(y, want_y, f"fp8 codes T={transpose}")
        assert_bytes_equal(s8, want_s, "chunk scales")


def test_library_quantized_activation_full_size_sampled():
    """The 8192 x 4096 activation quantized to MXFP4 by the library, converted (transposed,
    the backward form); 2 x 128 rows of the result checked against the oracle applied to
    the library's own MXFP4 bytes."""
    X = synth.make_config(3, rows=8192)["X"]
    qx = fp4.quantize(dev_input(X), fp4.E8M0, 32, fp4.ROW)
    yt, s8 = fp4.mxfp4_to_fp8(qx, transpose=True)
    torch.cuda.synchronize()
    for r0 in (0, 8064):
        codes = oracle.unpack_codes(qx.q[r0:r0 + 128].cpu().numpy())
        scales = qx.s[r0:r0 + 128].cpu().numpy()
        want_y, want_s = oracle.mxfp4_to_fp8(codes, scales, transpose=True)
        assert_bytes_equal(yt[:, r0:r0 + 128], want_y, "transposed fp8 rows")
        assert_bytes_equal(s8[r0:r0 + 128], want_s, "chunk scales")
