"""Shared helpers of the GPU parity tests (plumbing only)."""
import os
import sys

import numpy as np
import pytest


def gpu_ok() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


needs_gpu = pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| over the tensor."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(gpu - ref))) / max(den, 1e-30) if ref.size else 0.0


def host64(t) -> np.ndarray:
    """torch tensor (bf16 / f32 / int) -> float64 numpy on the host."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_tensor_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# tolerances (max relative error, per tensor) for the two storage formats
TOL = {"bf16": 2e-2, "f32": 1e-4}
