"""Shared helpers of the GPU parity tests."""
import sys

import numpy as np
import pytest
import torch

# Output tolerance for bf16-input, fp32-accumulated results against the fp64 oracle:
# max-abs 1e-2 and mean-abs 1e-3; LSE max-abs 1e-2.
OUT_MAX, OUT_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still leaves the name)."""
    print(*a, flush=True)
    sys.stdout.flush()


def as_bf16_for_oracle(t: torch.Tensor) -> np.ndarray:
    """The exact values the kernels consume: fp32 inputs are rounded to bf16 on load."""
    return t.detach().to(torch.bfloat16).contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def check_close(got, ref, what, max_abs=OUT_MAX, mean_abs=OUT_MEAN):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    say("  %s: max-abs %.3e mean-abs %.3e" % (what, mx, mn))
    assert mx <= max_abs and mn <= mean_abs, "%s: max-abs %.3g (<= %g), mean-abs %.3g (<= %g)" % (
        what, mx, max_abs, mn, mean_abs)
    return mx, mn
