"""Shared helpers for the GPU parity tests (device copies, comparisons)."""
import sys

import numpy as np
import torch

BF16_TOL = 2e-2  # max-abs bound for bf16 inputs against the float64 oracle
F32_TOL = 1e-5   # max-abs bound for the float32 path


def dev(t):
    return None if t is None else t.to("cuda")


def host64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(a, b):
    a = a if isinstance(a, np.ndarray) else host64(a)
    b = b if isinstance(b, np.ndarray) else host64(b)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
