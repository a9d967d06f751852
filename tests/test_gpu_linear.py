"""GPU parity of vq_verify_linear against the fp64 oracle: |gpu - oracle| <= 1e-3 * sum|w x|
per output, for every format, K = 1..16 and ragged shapes (partial row tiles, partial
column groups, a single block; for Q4_K, odd numbers of super-blocks)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_guard, check_rows, guarded_buffer, need_gpu, say

pytestmark = pytest.mark.gpu


def _run(m, x, y_dtype=0):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    W = vq.DeviceMatrix.from_host(m)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = vq.verify_linear(W, xd, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_c1_tiny_step():
    """1024 x 1024 Q4 (no min), fp16 scales ~U(0.005, 0.02), K = 4 activations ~N(0,1)."""
    c = synth.C1
    m = synth.weight_matrix(c["fmt"], c["seed"], 0, 0, c["rows"], c["cols"])
    x = synth.activations(c["seed"], c["K"], c["cols"])
    y_ref, a_ref = oracle.linear(m, x, threads=8)
    check_rows(_run(m, x), y_ref, a_ref, "C1")


# rows not a multiple of 16 (partial tile), cols with 33, 1 and 3 blocks (partial group of
# 4 blocks), and column counts that split into 5, 16 and 40 groups; more tiles than
# workgroups, so that tiles are split between workgroups (and, at K = 16 with 5120
# columns, between column windows of the activations)
SHAPES = [(1000, 1056), (77, 32), (64, 2048), (300, 5120), (129, 256), (16, 96), (5, 4096),
          (4200, 256), (4136, 1056), (4400, 5120)]


@pytest.mark.parametrize("fmt", [synth.FMT_Q4, synth.FMT_Q4_MIN, synth.FMT_MXFP4])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_shapes_formats_k(fmt, rows, cols):
    m = synth.weight_matrix(fmt, 11, 1, 2, rows, cols)
    worst = 0.0
    for K in (1, 2, 3, 4, 5, 8, 13, 16):
        x = synth.activations(12, K, cols)
        y_ref, a_ref = oracle.linear(m, x, threads=8)
        worst = max(worst, check_rows(_run(m, x), y_ref, a_ref, f"fmt {fmt} {rows}x{cols} K {K}"))
    say(f"fmt {fmt} {rows}x{cols}: worst |err| / sum|w x| over K = {worst:.3e}")


# Q4_K needs cols % 256 == 0: odd numbers of super-blocks (3, 5, 17, 20) instead of
# partial groups; partial row tiles and tiles split between workgroups as above
SHAPES_Q4K = [(1000, 768), (77, 256), (64, 2048), (300, 5120), (129, 1280), (16, 512), (5, 4352),
              (4200, 256), (4136, 1280), (4400, 5120)]


@pytest.mark.parametrize("rows,cols", SHAPES_Q4K)
def test_q4k_shapes_k(rows, cols):
    fmt = synth.FMT_Q4_K
    m = synth.weight_matrix(fmt, 11, 1, 2, rows, cols)
    worst = 0.0
    for K in (1, 2, 3, 4, 5, 8, 13, 16):
        x = synth.activations(12, K, cols)
        y_ref, a_ref = oracle.linear(m, x, threads=8)
        worst = max(worst, check_rows(_run(m, x), y_ref, a_ref, f"Q4_K {rows}x{cols} K {K}"))
    say(f"Q4_K {rows}x{cols}: worst |err| / sum|w x| over K = {worst:.3e}")


def test_q4k_degenerate_rows_and_extreme_scales():
    """Rows whose sub-block scales and mins are all 0, or whose super-block D and Dmin are 0,
    give exactly 0; 6-bit extremes (s = m = 63, bytes up to 255) and a large D stay within
    the tolerance."""
    m = synth.weight_matrix(synth.FMT_Q4_K, 5, 0, 0, 192, 1024)
    m.scales[7] = 0
    m.mins[7] = 0
    m.supers[9] = 0
    m.scales[11] = 63
    m.mins[11] = 63
    m.scales[12] = 255
    m.mins[12] = 255
    m.supers[13, :, 0] = np.float16(0.5)
    for K in (1, 4, 8, 16):
        x = synth.activations(6, K, 1024)
        y = _run(m, x)
        assert np.all(y[:, 7] == 0.0) and np.all(y[:, 9] == 0.0), f"K {K}"
        y_ref, a_ref = oracle.linear(m, x, threads=8)
        check_rows(y, y_ref, a_ref, f"Q4_K degenerate K {K}")


def test_zero_rows_are_exactly_zero_and_f16_output():
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 5, 0, 0, 192, 512)
    m.qs[7] = 0x88          # q = 0 everywhere in row 7
    m.mins[7] = 0
    m.scales[9] = 0         # d = 0 and m = 0 in row 9
    m.mins[9] = 0
    for K in (1, 4, 8, 16):
        x = synth.activations(6, K, 512)
        y = _run(m, x)
        assert np.all(y[:, 7] == 0.0) and np.all(y[:, 9] == 0.0), f"K {K}"
        y16 = _run(m, x, y_dtype=vq.DTYPE_F16)
        assert y16.dtype == np.float16
        assert np.array_equal(y16, y.astype(np.float16)), f"K {K}: fp16 output is not the rounded fp32 one"


@pytest.mark.parametrize("fmt", [synth.FMT_Q4_MIN, synth.FMT_Q4, synth.FMT_Q4_K])
def test_large_same_sign_activations(fmt):
    """A block of 32 large activations of one sign (32 x 4096 sums to 131072, beyond fp16):
    the min term and the block sums stay fp32, finite and within the tolerance."""
    m = synth.weight_matrix(fmt, 31, 0, 1, 64, 1024)
    for K in (1, 4, 8, 16):
        x = synth.activations(32, K, 1024)
        x[:, 64:96] = np.float16(4096.0)
        x[0, 512:544] = np.float16(-60000.0)
        y_ref, a_ref = oracle.linear(m, x, threads=8)
        y = _run(m, x)
        assert np.isfinite(y).all(), f"K {K}: non-finite outputs"
        check_rows(y, y_ref, a_ref, f"large activations fmt {fmt} K {K}")


def test_bitwise_reproducible():
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 8, 0, 0, 1000, 2048)
    for K in (1, 4, 16):
        x = synth.activations(9, K, 2048)
        assert np.array_equal(_run(m, x), _run(m, x)), f"K {K}"


@pytest.mark.parametrize("rows,cols", [(300, 5120), (96, 17408), (1000, 1056)])
def test_output_stays_in_bounds(rows, cols):
    """Nothing is written past y (a guard band of 0xA5 bytes behind it); results match."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 21, 0, 6, rows, cols)
    W = vq.DeviceMatrix.from_host(m)
    for K in (1, 4, 8, 16):
        for dt, es in ((vq.DTYPE_F32, 4), (vq.DTYPE_F16, 2)):
            x = synth.activations(22, K, cols)
            ny = K * rows * es
            yb, y_whole = guarded_buffer(ny)
            y = yb.view(torch.float32 if es == 4 else torch.float16).view(K, rows)
            say(f"guarded {rows}x{cols} K {K} dtype {dt}")
            vq.verify_linear(W, torch.from_numpy(x).cuda(), y=y, y_dtype=dt)
            torch.cuda.synchronize()
            check_guard(y_whole, ny, f"y, K {K} dtype {dt}")
            if dt == vq.DTYPE_F32:
                y_ref, a_ref = oracle.linear(m, x, threads=8)
                check_rows(y.cpu().numpy(), y_ref, a_ref, f"guarded {rows}x{cols} K {K}")


@pytest.mark.parametrize("mid", [synth.MAT_DOWN, synth.MAT_LM_HEAD])
def test_full_size_sampled_rows(mid):
    """27B-class shapes (down 5120 x 17408, lm_head 151936 x 5120) at K = 1, 4, 8, 16, checked
    on 48 sampled rows each (the oracle regenerates just those rows)."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape = synth.SHAPE_27B
    rows, cols = shape.mat_shape(mid)
    for fmt in (synth.FMT_Q4_MIN, synth.FMT_MXFP4, synth.FMT_Q4_K):
        m = synth.weight_matrix(fmt, 0, 3, mid, rows, cols, threads=16)
        W = vq.DeviceMatrix.from_host(m)
        rng = np.random.default_rng(mid)
        pick = np.unique(np.concatenate([rng.integers(0, rows, 46), [0, rows - 1]]))
        sub = m.take(pick)
        del m
        for K in (1, 4, 8, 16):
            x = synth.activations(0, K, cols)
            xd = torch.from_numpy(x).cuda()
            y = vq.verify_linear(W, xd).cpu().numpy()
            y_ref, a_ref = oracle.linear(sub, x, threads=8)
            check_rows(y[:, pick], y_ref, a_ref, f"mat {mid} fmt {fmt} K {K}")
        del W
        torch.cuda.empty_cache()
