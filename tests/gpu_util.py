"""Helpers shared by the GPU parity tests: bit marshalling and the tolerance rule.

Tolerance (floats): |gpu - ref| <= 1e-2 |ref| + 1e-3 rms(ref), rms over the
whole output tensor of the stage.  Argmax: the index must equal the oracle's
lowest-index argmax unless the oracle's top-2 logits lie within that tolerance
(then any index whose oracle logit is within tolerance of the maximum passes).
"""
import sys

import numpy as np
import torch

from oracle import oracle as O
from synth.gen import bf16_bits_to_numpy, f16_bits_to_numpy  # noqa: F401

RTOL, ATOL_RMS = 1e-2, 1e-3


def say(msg: str) -> None:
    print("[gpu-test] " + msg, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_numpy(t)
    if t.dtype == torch.float16:
        return f16_bits_to_numpy(t)
    raise TypeError(t.dtype)


def tol_of(ref: np.ndarray) -> np.ndarray:
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return RTOL * np.abs(ref) + ATOL_RMS * rms


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str) -> float:
    """gpu, ref: float64 arrays of the same shape.  Returns worst |d|/tol."""
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what + ": non-finite GPU output"
    tol = tol_of(ref)
    d = np.abs(gpu - ref)
    bad = d > tol
    if bad.any():
        i = np.argmax(d - tol)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %d: gpu %r ref %r tol %r"
                             % (what, bad.sum(), bad.size, i, gpu.flat[i], ref.flat[i], tol.flat[i]))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(tol > 0, d / tol, 0.0)
    return float(np.max(r)) if r.size else 0.0


def assert_close_bf16(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str) -> float:
    return assert_close(O.bf16_array_to_f64(gpu_bits), O.bf16_array_to_f64(ref_bits), what)


def f16_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def check_argmax(gpu_idx: int, logits: np.ndarray, what: str) -> None:
    """logits: oracle binary64 logits of one batch row."""
    top = int(np.argmax(logits))  # numpy returns the first (lowest) index of the max
    if gpu_idx == top:
        return
    top1 = logits[top]
    second = np.max(np.delete(logits, top))
    rms = float(np.sqrt(np.mean(logits * logits)))
    tol = RTOL * abs(top1) + ATOL_RMS * rms
    assert top1 - second <= tol, "%s: argmax %d != oracle %d (gap %g > tol %g)" % (
        what, gpu_idx, top, top1 - second, tol)
    assert 0 <= gpu_idx < logits.size and logits[gpu_idx] >= top1 - tol, (
        "%s: waived argmax %d is not a near-maximum" % (what, gpu_idx))
