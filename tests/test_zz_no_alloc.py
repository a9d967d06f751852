"""vq_verify_linear_noalloc (the entry point that allocates nothing, for callers that cannot
allocate) against vq_verify_linear on the same inputs: bit-identical outputs, on two calls
in a row, the second with a smaller matrix and a smaller K, and back again; plus the limits
it rejects and the oracle bound on one case."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_rows, need_gpu, say

pytestmark = pytest.mark.gpu


def _pair(vq, torch, fmt, rows, cols, K, seed, y_dtype=0):
    m = synth.weight_matrix(fmt, seed, 0, 0, rows, cols)
    x = synth.activations(seed, K, cols)
    W = vq.DeviceMatrix.from_host(m)
    xd = torch.from_numpy(x).cuda()
    say(f"noalloc vs linear: fmt {fmt} {rows}x{cols} K {K} seed {seed} dtype {y_dtype}")
    y0 = vq.verify_linear(W, xd, y_dtype=y_dtype)
    # the output buffer holds garbage first: every element must be written
    y1 = torch.full_like(y0, float("nan"))
    vq.verify_linear_noalloc(W, xd, y=y1, y_dtype=y_dtype)
    torch.cuda.synchronize()
    a, b = y0.cpu().numpy(), y1.cpu().numpy()
    assert a.shape == b.shape
    same = a.view(np.uint32 if a.dtype == np.float32 else np.uint16) == b.view(np.uint32 if b.dtype == np.float32
                                                                               else np.uint16)
    assert same.all(), f"{int((~same).sum())} of {same.size} outputs differ from vq_verify_linear"
    return m, x, b


def test_noalloc_matches_linear_twice_then_smaller():
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    # the lm_head shape at K = 8, then a smaller one (split tiles, partial groups) at K = 3,
    # then the first again with other inputs (the scratch array keeps the last call's lists)
    m, x, y = _pair(vq, torch, synth.FMT_Q4_MIN, 151936, 5120, 8, 1)
    _pair(vq, torch, synth.FMT_Q4_MIN, 4136, 1056, 3, 2)
    _pair(vq, torch, synth.FMT_Q4_MIN, 151936, 5120, 8, 3)
    # oracle bound on sampled rows of the first call
    rows = np.arange(0, 151936, 997)
    sub = synth.weight_rows(synth.FMT_Q4_MIN, 1, 0, 0, 151936, 5120, rows)
    y_ref, a_ref = oracle.linear(sub, x, threads=8)
    check_rows(y[:, rows], y_ref, a_ref, "noalloc lm_head K 8 sampled rows")


@pytest.mark.parametrize("fmt", [synth.FMT_Q4, synth.FMT_MXFP4])
def test_noalloc_other_formats_and_f16(fmt):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    _pair(vq, torch, fmt, 1000, 1056, 4, 5, y_dtype=1)
    _pair(vq, torch, fmt, 77, 32, 1, 6)


def test_noalloc_rejects_windowed_shapes():
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    # K = 16 over 5120 columns needs column windows: refused with a clear error
    m = synth.weight_matrix(synth.FMT_Q4_MIN, 0, 0, 0, 64, 5120)
    W = vq.DeviceMatrix.from_host(m)
    xd = torch.from_numpy(synth.activations(0, 16, 5120)).cuda()
    with pytest.raises(vq.VqError) as e:
        vq.verify_linear_noalloc(W, xd)
    assert e.value.code == -2, e.value
    assert "column windows" in str(e.value)
