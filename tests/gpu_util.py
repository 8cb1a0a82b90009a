"""Shared helpers for the GPU tests: host<->device bit transfers and tolerances."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

# |gpu - ref| <= TOL * (|ref| + 1) against the unrounded fp64 oracle.
BF16_TOL = 1e-2     # bf16 outputs; their own rounding costs <= 2^-8 |ref|
F32_TOL = 1e-5      # fp32 shrink output; floored so that outputs near zero are judged fairly


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device torch.bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def check_bf16(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    g = oracle.bf16_decode(gpu_bits)
    err = np.abs(g - ref)
    bound = BF16_TOL * (np.abs(ref) + 1.0)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3g}, max ratio {(err / bound).max():.3g}")
    return float((err / bound).max())


def check_f32(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = F32_TOL * (np.abs(ref) + 1.0)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3g}")
    return float((err / bound).max())


def say(msg: str):
    print(msg, flush=True)
