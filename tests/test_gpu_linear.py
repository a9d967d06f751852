"""GPU parity of vq_verify_linear against the fp64 oracle: |gpu - oracle| <= 1e-3 * sum|w x|."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_guard, check_rows, guarded_buffer, need_gpu, say

pytestmark = pytest.mark.gpu


def _run(m, x, path, y_dtype=0):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    W = vq.DeviceMatrix.from_host(m)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = vq.verify_linear(W, xd, y_dtype=y_dtype, path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_c1_tiny_step_both_paths():
    """1024 x 1024 Q4 (no min), fp16 scales ~U(0.005, 0.02), K = 4 activations ~N(0,1)."""
    import speculative_decoding_verification_bit_amd as vq
    c = synth.C1
    m = synth.weight_matrix(c["fmt"], c["seed"], 0, 0, c["rows"], c["cols"])
    x = synth.activations(c["seed"], c["K"], c["cols"])
    y_ref, a_ref = oracle.linear(m, x, threads=8)
    for path in (vq.PATH_VALU, vq.PATH_MFMA, vq.PATH_AUTO):
        say(f"C1 path {path}")
        check_rows(_run(m, x, path), y_ref, a_ref, f"C1 path {path}")


SHAPES = [(1000, 1056), (77, 32), (64, 2048), (300, 5120), (129, 256)]


@pytest.mark.parametrize("fmt", [synth.FMT_Q4, synth.FMT_Q4_MIN, synth.FMT_MXFP4])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_shapes_formats_paths(fmt, rows, cols):
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(fmt, 11, 1, 2, rows, cols)
    for path, Ks in ((vq.PATH_VALU, (1, 2, 3, 8)), (vq.PATH_MFMA, (1, 5, 16)), (vq.PATH_ROWS, (1, 2, 3, 4))):
        for K in Ks:
            x = synth.activations(12, K, cols)
            y_ref, a_ref = oracle.linear(m, x, threads=8)
            say(f"fmt {fmt} {rows}x{cols} path {path} K {K}")
            check_rows(_run(m, x, path), y_ref, a_ref, f"fmt {fmt} {rows}x{cols} path {path} K {K}")


def test_zero_rows_are_exactly_zero_and_f16_output():
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 5, 0, 0, 192, 512)
    m.qs[7] = 0x88          # q = 0 everywhere in row 7
    m.mins[7] = 0
    m.scales[9] = 0         # d = 0 and m = 0 in row 9
    m.mins[9] = 0
    x = synth.activations(6, 8, 512)
    for path in (vq.PATH_VALU, vq.PATH_MFMA, vq.PATH_ROWS):
        y = _run(m, x[:4] if path == vq.PATH_ROWS else x, path)
        assert np.all(y[:, 7] == 0.0) and np.all(y[:, 9] == 0.0)
        y16 = _run(m, x[:4] if path == vq.PATH_ROWS else x, path, y_dtype=vq.DTYPE_F16)
        assert y16.dtype == np.float16
        assert np.array_equal(y16, y.astype(np.float16))


def test_bitwise_reproducible():
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 8, 0, 0, 1000, 2048)
    x = synth.activations(9, 4, 2048)
    for path in (vq.PATH_VALU, vq.PATH_MFMA, vq.PATH_ROWS):
        assert np.array_equal(_run(m, x, path), _run(m, x, path))


@pytest.mark.parametrize("rows,cols", [(300, 5120), (96, 17408), (1000, 1056)])
def test_workspace_and_output_stay_in_bounds(rows, cols):
    """Every path and K writes nothing past the workspace the library asked for, nor past
    y (guard bands of 0xA5 bytes behind both); the results still match the oracle."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 21, 0, 6, rows, cols)
    W = vq.DeviceMatrix.from_host(m)
    for path, Ks in ((vq.PATH_VALU, (1, 4, 8)), (vq.PATH_MFMA, (1, 8, 16)), (vq.PATH_ROWS, (1, 4)),
                     (vq.PATH_AUTO, (1, 16))):
        for K in Ks:
            x = synth.activations(22, K, cols)
            need = vq.workspace_bytes(vq.OP_LINEAR, W.desc, K)
            ws, ws_whole = guarded_buffer(need)
            ny = K * rows * 4
            yb, y_whole = guarded_buffer(ny)
            y = yb.view(torch.float32).view(K, rows)
            say(f"guarded {rows}x{cols} path {path} K {K}: workspace {need} B")
            vq.verify_linear(W, torch.from_numpy(x).cuda(), y=y, path=path, ws=ws)
            torch.cuda.synchronize()
            check_guard(ws_whole, need, f"workspace, path {path} K {K}")
            check_guard(y_whole, ny, f"y, path {path} K {K}")
            y_ref, a_ref = oracle.linear(m, x, threads=8)
            check_rows(y.cpu().numpy(), y_ref, a_ref, f"guarded {rows}x{cols} path {path} K {K}")


@pytest.mark.parametrize("mid", [synth.MAT_DOWN, synth.MAT_LM_HEAD])
def test_full_size_sampled_rows(mid):
    """27B-class shapes (down 5120 x 17408, lm_head 151936 x 5120) at K = 1, 4, 8, 16, checked
    on 48 sampled rows each (the oracle regenerates just those rows)."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape = synth.SHAPE_27B
    rows, cols = shape.mat_shape(mid)
    for fmt in (synth.FMT_Q4_MIN, synth.FMT_MXFP4):
        m = synth.weight_matrix(fmt, 0, 3, mid, rows, cols, threads=16)
        W = vq.DeviceMatrix.from_host(m)
        rng = np.random.default_rng(mid)
        pick = np.unique(np.concatenate([rng.integers(0, rows, 46), [0, rows - 1]]))
        sub = synth.Q4Matrix(fmt, len(pick), cols, m.qs[pick], m.scales[pick],
                             None if m.mins is None else m.mins[pick])
        del m
        for K, path in ((1, vq.PATH_AUTO), (4, vq.PATH_AUTO), (8, vq.PATH_AUTO), (16, vq.PATH_AUTO),
                        (1, vq.PATH_ROWS), (2, vq.PATH_ROWS)):
            x = synth.activations(0, K, cols)
            xd = torch.from_numpy(x).cuda()
            y = vq.verify_linear(W, xd, path=path).cpu().numpy()
            y_ref, a_ref = oracle.linear(sub, x, threads=8)
            check_rows(y[:, pick], y_ref, a_ref, f"mat {mid} fmt {fmt} K {K} path {path}")
        del W
        torch.cuda.empty_cache()
