"""Shared helpers for the GPU parity tests (host <-> device plumbing and the
error checks)."""
import sys

import numpy as np
import torch

BF16_TOL = 2e-2   # max abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4    # max abs error, fp32


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        t = t.view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to("cuda")


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tol(dtype: str) -> float:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault points at it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def max_abs_err(a: np.ndarray, b: np.ndarray) -> float:
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite values in the GPU result"
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def assert_discriminating(ref: np.ndarray, dtype: str) -> None:
    """The expected output is far from zero against the tolerance, so that a
    result that skipped rows or tiles cannot pass by being near zero."""
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    assert rms > 10 * tol(dtype), rms
