"""Seeded synthetic inputs, shared by the tests, the benchmark and the harness.

This module holds no arithmetic of the method itself (no sums, norms or
products).  It only draws random numbers and converts them to bf16 bit patterns
with torch's own float32 -> bfloat16 cast (round to nearest, ties to even),
so that the oracle and the HIP path receive the very same bits.

Distributions follow the workloads the pages talk about (LLM activations and
weights); none of the pages' datasets is reproduced.  Host generators use
numpy's PCG64 with an explicit seed; inputs of a GiB or more are drawn on the
device with torch's seeded generator (``device_normal_bf16``), and whatever
checks them on the host copies back the slices it needs.
"""
from __future__ import annotations

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's bfloat16 cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, seed: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(mean, std^2) samples (std is the standard deviation)."""
    g = rng(seed)
    v = g.standard_normal(size=shape) * std + mean
    return f32_to_bf16_bits(v.astype(np.float32))


def device_normal_bf16(shape, seed: int, mean: float = 0.0, std: float = 1.0,
                       device: str = "cuda", dtype=torch.bfloat16) -> torch.Tensor:
    """N(mean, std^2) samples drawn on the device by torch's seeded generator,
    cast to ``dtype`` (bf16 by default, round to nearest even)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return (t * std + mean).to(dtype)


def int_bf16(shape, seed: int, lo: int, hi: int) -> np.ndarray:
    """bf16 bits of uniform integers in [lo, hi]; exact in bf16 while |v| <= 256."""
    if max(abs(lo), abs(hi)) > 256:
        raise ValueError("integers above 256 in magnitude are not all exact in bf16")
    g = rng(seed)
    v = g.integers(lo, hi, endpoint=True, size=shape)
    return f32_to_bf16_bits(v.astype(np.float32))


def permutation(n: int, seed: int) -> np.ndarray:
    return rng(seed).permutation(n)


def batch_stream(n_batches: int, m_max: int, pool_rows: int, n_probes: int,
                 seed_m: int, seed_probe: int):
    """A dynamic-batch stream: ``n_batches`` batches with M ~ U{1..m_max}.

    Returns ``(probe_pool_index, batches)``; each batch is a dict with
    ``rows`` (int64 indices into the row pool, length M) and ``probe_pos``
    (positions of the probes inside the batch, -1 where a probe is absent
    because M is smaller than the probe count).  The probes sit at distinct
    random positions; the other rows are drawn from the pool with replacement.
    """
    gp = rng(seed_probe)
    probes = gp.choice(pool_rows, size=n_probes, replace=False)
    gm = rng(seed_m)
    batches = []
    for _ in range(n_batches):
        M = int(gm.integers(1, m_max, endpoint=True))
        rows = gm.integers(0, pool_rows, size=M).astype(np.int64)
        n_in = min(M, n_probes)
        pos = gm.choice(M, size=n_in, replace=False)
        probe_pos = np.full(n_probes, -1, dtype=np.int64)
        for p in range(n_in):
            rows[pos[p]] = probes[p]
            probe_pos[p] = pos[p]
        batches.append({"rows": rows, "probe_pos": probe_pos})
    return probes.astype(np.int64), batches
