"""GPU parity of vq_verify_linear_mx (the scaled MXFP4 matrix instruction with E4M3
activations, an approximation of W x) against the oracle of the same approximation:
  * the activation conversion (E4M3 codes, E8M0 block scales) is bit-exact against the
    oracle's OCP MX conversion, over every finite fp16 value and wide-range random blocks;
  * y against the oracle's fp64 W x_hat (x_hat = the E4M3-rounded activations) within
    1e-3 * sum |w x_hat| per output, on ragged shapes and the full-size matrices;
  * how far the approximation is from the exact W x is reported, not bounded."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_rows, need_gpu, report, say

pytestmark = pytest.mark.gpu


def _run(m, x):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    W = vq.DeviceMatrix.from_host(m)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    K = x.shape[0]
    ws = torch.empty(vq.workspace_bytes(vq.OP_LINEAR_MX, W.desc, K), dtype=torch.uint8, device="cuda")
    y = torch.full((K, m.rows), float("nan"), dtype=torch.float32, device="cuda")
    vq.verify_linear_mx(W, xd, y=y, ws=ws)
    torch.cuda.synchronize()
    # the workspace holds the converted activations: codes [16][cols], then scales [16][cols/32]
    cols = m.cols
    off = -(-16 * cols // 256) * 256
    w = ws.cpu().numpy()
    codes = w[:16 * cols].reshape(16, cols)[:K]
    scales = w[off:off + 16 * (cols // 32)].reshape(16, cols // 32)[:K]
    return y.cpu().numpy(), codes, scales


def test_activation_conversion_every_fp16_value():
    """All 63,488 finite fp16 patterns (in blocks of 32 consecutive patterns, so that block
    maxima span the whole range), then random blocks over 2^-24 .. 2^15: codes and scales
    equal the oracle's, bit for bit."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = pats.view(np.float16)
    h = np.where(np.isfinite(h), h, np.float16(0)).astype(np.float16)
    x = h.reshape(16, 4096)
    m = synth.weight_matrix(synth.FMT_MXFP4, 0, 0, 0, 16, 4096)
    _, codes, scales = _run(m, x)
    oc, osc = oracle.mx_quant(x)
    bad = int((codes != oc).sum()) + int((scales != osc).sum())
    report(f"E4M3 conversion, every finite fp16 value: {bad} codes or scales differ from the oracle")
    assert bad == 0
    rng = np.random.default_rng(2)
    xr = (rng.standard_normal((16, 2048)) * np.exp2(rng.uniform(-20, 14, (16, 2048)))).astype(np.float16)
    xr[3, 64:96] = 0
    xr[5, 100] = -0.0
    _, codes, scales = _run(synth.weight_matrix(synth.FMT_MXFP4, 0, 0, 0, 16, 2048), xr)
    oc, osc = oracle.mx_quant(xr)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)


SHAPES = [(77, 128), (300, 5120), (1000, 1024), (16, 17408), (2177, 384)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("K", [1, 3, 16])
def test_mx_linear_vs_oracle(rows, cols, K):
    m = synth.weight_matrix(synth.FMT_MXFP4, 3, 0, 1, rows, cols)
    x = synth.activations(3, K, cols)
    y, codes, scales = _run(m, x)
    oc, osc = oracle.mx_quant(x)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)
    xh = oracle.mx_dequant(oc, osc)
    y_ref, a_ref = oracle.linear_x64(m, xh, threads=8)
    ratio = check_rows(y, y_ref, a_ref, f"mx {rows}x{cols} K {K}")
    # distance from the exact W x (informational)
    y_ex, a_ex = oracle.linear(m, x, threads=8)
    dev = float(np.max(np.abs(y - y_ex) / np.maximum(a_ex, 1e-300)))
    report(f"mx {rows}x{cols} K {K}: parity {ratio:.2e} of sum|w x_hat|; E4M3 approximation "
           f"max |y - W x| / sum|w x| = {dev:.2e}")


@pytest.mark.parametrize("rows,cols", [(151936, 5120), (5120, 17408)])
def test_mx_full_size_sampled_rows(rows, cols):
    """The lm_head and down shapes at K = 16, 40 sampled rows against the oracle."""
    torch = need_gpu()
    m = synth.weight_matrix(synth.FMT_MXFP4, 0, 0, synth.MAT_LM_HEAD if rows == 151936 else synth.MAT_DOWN,
                            rows, cols, threads=16)
    x = synth.activations(0, 16, cols)
    y, codes, scales = _run(m, x)
    rng = np.random.default_rng(1)
    pick = np.unique(np.concatenate([rng.integers(0, rows, 38), [0, rows - 1]]))
    sub = synth.Q4Matrix(m.fmt, len(pick), cols, m.qs[pick], m.scales[pick], None)
    oc, osc = oracle.mx_quant(x)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)
    xh = oracle.mx_dequant(oc, osc)
    y_ref, a_ref = oracle.linear_x64(sub, xh, threads=8)
    check_rows(y[:, pick], y_ref, a_ref, f"mx {rows}x{cols} K 16 sampled rows")
