"""Helpers for the GPU parity tests: tolerance checks and host copies for the oracle."""

import sys

import numpy as np
import torch

from long_context_sparse_index_amd import inputs as I

# Attention outputs and gradients: max |x - ref| <= 2e-2 RMS(ref), mean |x - ref| <= 2e-3 RMS(ref).
MAX_REL = 2e-2
MEAN_REL = 2e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_errors(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(x - ref)
    if rms == 0.0:
        return float(err.max(initial=0.0)), float(err.mean() if err.size else 0.0), rms
    return float(err.max() / rms), float(err.mean() / rms), rms


def assert_close(x, ref, what: str, max_rel=MAX_REL, mean_rel=MEAN_REL):
    mx, mn, rms = rel_errors(x, ref)
    say("  %s: max/rms %.3g  mean/rms %.3g  (rms %.3g)" % (what, mx, mn, rms))
    assert mx <= max_rel and mn <= mean_rel, "%s out of tolerance: max %.3g mean %.3g" % (
        what, mx, mn)


def f32_bits_equal(a, b) -> bool:
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.int32), b.view(np.int32))


def host_bits(t: torch.Tensor) -> np.ndarray:
    return I.index_bits(t) if t.dtype != torch.bfloat16 else I.bits_u16(t)
