"""Helpers shared by the GPU parity tests (uploading synthetic inputs, tolerance checks)."""
import sys

import numpy as np
import pytest

import synth


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def report(line: str):
    """say(), and keep the line for the end-of-session summary (shown by quiet runs too)."""
    say(line)
    import conftest
    conftest.REPORT.append(line)


def f32(v: float) -> float:
    """The float32 value the C ABI receives for a sampler setting, as a double."""
    return float(np.float32(v))


def check_rows(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, what: str):
    """|y_gpu - y_ref| <= 1e-3 * sum_j |w_ij x_j| for every element (zero rows exactly 0)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > 1e-3 * a_ref
    ratio = float(np.max(err / np.maximum(a_ref, 1e-300))) if err.size else 0.0
    say(f"{what}: max |err| / sum|w x| = {ratio:.3e} over {err.size} outputs")
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside 1e-3 * sum|w x| (worst {ratio:.3e})"
    return ratio


def upload_model(shape: synth.ModelShape, fmt: int, seed: int, threads: int = 16):
    """The whole stack on the device, matrix by matrix (host memory stays small)."""
    import speculative_decoding_verification_bit_amd as vq
    layers = []
    for l in range(shape.n_layers):
        L = {}
        for mid, name in enumerate(synth.LAYER_MATS):
            r, c = shape.mat_shape(mid)
            L[name] = vq.DeviceMatrix.from_host(synth.weight_matrix(fmt, seed, l, mid, r, c, threads=threads))
        layers.append(L)
    r, c = shape.mat_shape(synth.MAT_LM_HEAD)
    lm = vq.DeviceMatrix.from_host(synth.weight_matrix(fmt, seed, shape.n_layers, synth.MAT_LM_HEAD, r, c,
                                                       threads=threads))
    return vq.DeviceModel(layers, lm)


GUARD_BYTES = 1 << 20
GUARD_FILL = 0xA5


def guarded_buffer(nbytes: int):
    """A device byte buffer of exactly nbytes followed by a 1 MiB guard band of 0xA5 bytes:
    returns (buffer view, whole allocation)."""
    import torch
    whole = torch.full((nbytes + GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device="cuda")
    return whole[:nbytes], whole


def check_guard(whole, nbytes: int, what: str):
    """No byte past the first nbytes of `whole` was written."""
    tail = whole[nbytes:]
    bad = int((tail != GUARD_FILL).sum().item())
    assert bad == 0, f"{what}: {bad} bytes written past the end of the {nbytes}-byte buffer"
