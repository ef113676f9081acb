"""Shared helpers of the GPU parity tests (comparison metrics, device plumbing)."""
import sys

import numpy as np
import pytest

# fp32 outputs: max over elements of |y - ref| / max(|ref|, 1e-2 * rms(ref)),
# which is the plain relative error except for the ~0.1% of outputs close to
# zero, where relative error is not meaningful.
FP32_TOL = 1e-3
FP16_TOL = 1e-2


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), 1e-2 * rms + 1e-300)
    return float(np.max(np.abs(y - ref) / den)) if ref.size else 0.0


def norm_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import bit_weight_streaming_q4_amd as mk
    mk.lib()  # raises if the HIP library is missing: there is no fallback
    return torch


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def to_np(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()
