"""Rewrite the expected bits in ``fixed_order_pins.txt`` from the oracle alone.

Usage: ``python tests/golden/make_fixed_order_pins.py`` (from the repo root).

For each pin, the per-step terms are exact (each matrix-core step holds at most
one non-zero product, and every product is a power of two), so the documented
order's fp32 result is the oracle's fp32 left fold of those terms.  The bf16
output of the GEMM pin is the oracle's round-to-nearest-even of that fp32 value.
"""
from __future__ import annotations

import itertools
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

OUT = os.path.join(HERE, "fixed_order_pins.txt")


def f32_bits(v) -> str:
    return "0x%08X" % int(np.asarray(v, dtype=np.float32).view(np.uint32))


def bf16_bits_of_f32(v) -> str:
    return "0x%04X" % int(oracle.bf16_round(np.array([float(np.float32(v))]))[0])


def pins():
    rows = []
    # GEMM K-order pin: one ascending pass over K = 4096 in matrix-core steps
    # (32 k per bf16 16x16x32 step).  Every non-zero product falls in a step of
    # its own for steps of 16 k as well, so the pin does not depend on which
    # bf16 instruction form runs the pass.
    k_terms = [(0, 1.0, 1.0), (64, 1.0, 2.0 ** -8), (2112, 1.0, 2.0 ** -24),
               (4032, 1.0, 2.0 ** -24)]
    for step in (16, 32):
        steps = [k // step for k, _, _ in k_terms]
        assert len(set(steps)) == len(steps)
    terms = np.array([x * w for _, x, w in k_terms], dtype=np.float32)
    asc = oracle.combine_f32(terms.reshape(-1, 1))[0]
    desc = oracle.combine_f32(terms[::-1].copy().reshape(-1, 1))[0]
    nz = ",".join(f"{k}:{x:g}*{w:.17g}" for k, x, w in k_terms)
    rows.append(("gemm_korder_ascending", 4096, nz, f32_bits(asc), bf16_bits_of_f32(asc)))
    rows.append(("gemm_korder_descending_is_wrong", 4096, nz, f32_bits(desc),
                 bf16_bits_of_f32(desc)))
    # The same input through a fixed split-K of 2 (chunks [0, 2048), [2048, 4096)):
    # each chunk folds its steps, then the partials fold in order.
    p = []
    for c in range(2):
        t = np.array([x * w for k, x, w in k_terms if c * 2048 <= k < (c + 1) * 2048], np.float32)
        p.append(oracle.combine_f32(t.reshape(-1, 1))[0] if len(t) else np.float32(0))
    sk = oracle.combine_f32(np.array(p, np.float32).reshape(-1, 1))[0]
    rows.append(("gemm_splitk2_korder", 4096, nz, f32_bits(sk), bf16_bits_of_f32(sk)))

    # LoRA shrink combine-order pin: K = 4096, split into 8 chunks of 512.
    s_terms = [(0, 1.0, 1.0), (512, 1.0, 2.0 ** -24), (1024, 1.0, 2.0 ** -24)]
    nz = ",".join(f"{k}:{x:g}*{w:.17g}" for k, x, w in s_terms)
    partials = np.zeros(8, dtype=np.float32)
    for k, x, w in s_terms:
        partials[k // 512] += np.float32(x * w)   # one term per chunk: exact
    det = oracle.combine_f32(partials.reshape(8, 1))[0]
    rows.append(("shrink_split8_fixed_order", 4096, nz, f32_bits(det), f32_bits(det)))
    # Unsplit: one ascending pass, 32 k per 16x16x32 step; the terms fall in
    # steps 0, 16 and 32.
    uns_terms = np.array([x * w for _, x, w in s_terms], dtype=np.float32)
    uns = oracle.combine_f32(uns_terms.reshape(-1, 1))[0]
    rows.append(("shrink_unsplit", 4096, nz, f32_bits(uns), f32_bits(uns)))
    # Atomic control: out starts at 0 and the 8 partials arrive in any order.
    seen = set()
    for perm in set(itertools.permutations(partials.tolist())):
        seq = np.array([0.0, *perm], dtype=np.float32).reshape(-1, 1)
        seen.add(f32_bits(oracle.combine_f32(seq)[0]))
    rows.append(("shrink_atomic_any_of", 4096, nz, "-", ",".join(sorted(seen))))
    return rows


def main():
    with open(OUT) as f:
        header = [ln for ln in f if ln.startswith("#")]
    with open(OUT, "w") as f:
        f.writelines(header)
        for r in pins():
            f.write(" | ".join(str(c) for c in r) + "\n")
    print(open(OUT).read())


if __name__ == "__main__":
    main()
