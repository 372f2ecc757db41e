"""Shared helpers for the GPU parity tests (error metrics, sampling, devices)."""
import sys

import numpy as np
import torch

# Relative L2 bars: fp32 I/O, and fp16/bf16 I/O with fp32 accumulation.
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(got, ref) -> float:
    got = np.asarray(got)
    ref = np.asarray(ref)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def cplx(t: torch.Tensor) -> np.ndarray:
    """[..., 2] float tensor -> complex128 numpy."""
    a = t.detach().to("cpu", torch.float64).numpy()
    return a[..., 0] + 1j * a[..., 1]


def row_rel_l2(got, ref) -> np.ndarray:
    """Relative L2 error of every row (last axis) of got against ref; rows
    whose reference is all zero report their absolute norm."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.where(den > 0, den, 1.0)
