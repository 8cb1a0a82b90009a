"""Invariance harness: bitwise comparison of outputs across batch contexts,
reruns and identical-input replays, counted on the device by bi_row_bitdiff.

What it checks ("God Does Not Play Dice: Enforcing Batch Invariance in Agentic
Kernel Generation", abstract: dynamic validation of bitwise consistency across
batch contexts; the forum thread "You think you are measuring intelligence...",
first comment: the same prompt alone and pad-batched must agree; "Reproducible
LoRA Inference Through Deterministic Split-K Reduction", abstract:
identical-input replay):

  * batch invariance -- a probe row's output computed alone (M = 1) against the
    same row's output inside batches of other sizes, at other positions;
  * run-to-run determinism -- the same batch computed again;
  * replay variation -- one input replayed N times; a replay "differs" when any
    bit of its output differs from replay 0.

``run`` is any callable mapping a device input batch [M, K] to a device output
[M, C] (2- or 4-byte elements).  Gathering batch rows from a pool is test
set-up (torch indexing); the comparison itself runs in the HIP kernel.
"""
from __future__ import annotations

from typing import Callable, Iterable

import torch

from . import binding


def solo_outputs(run: Callable[[torch.Tensor], torch.Tensor], pool: torch.Tensor,
                 probes: Iterable[int]) -> torch.Tensor:
    """Each probe row computed alone: [P, C]."""
    outs = [run(pool[int(p):int(p) + 1]).clone() for p in probes]
    return torch.cat(outs, dim=0)


def compare_rows(y: torch.Tensor, y_rows: torch.Tensor, ref: torch.Tensor,
                 ref_rows: torch.Tensor) -> tuple[int, int]:
    """Total (differing bits, differing elements) between y[y_rows] and ref[ref_rows]."""
    if y_rows.numel() == 0:
        return 0, 0
    c = binding.bi_row_bitdiff(y, ref, y_rows, ref_rows)
    s = c.sum(dim=0).tolist()
    return int(s[0]), int(s[1])


def batch_invariance(run, pool: torch.Tensor, probes, batches) -> dict:
    """Run each batch (a device int64 index vector into ``pool``) and compare
    every output row that holds a probe with that probe's solo output.

    Returns totals: batches, rows compared, differing bits and elements, and
    the worst batch's differing bits."""
    probes = [int(p) for p in probes]
    solo = solo_outputs(run, pool, probes)
    pid = {p: i for i, p in enumerate(probes)}
    total = dict(batches=0, rows=0, diff_bits=0, diff_elems=0, worst_batch_bits=0)
    for idx in batches:
        idx = idx.to(device=pool.device, dtype=torch.int64)
        y = run(pool.index_select(0, idx))
        host = idx.tolist()
        pos = [j for j, r in enumerate(host) if r in pid]
        ids = [pid[host[j]] for j in pos]
        t_pos = torch.tensor(pos, dtype=torch.int64, device=pool.device)
        t_ids = torch.tensor(ids, dtype=torch.int64, device=pool.device)
        bits, elems = compare_rows(y, t_pos, solo, t_ids)
        total["batches"] += 1
        total["rows"] += len(pos)
        total["diff_bits"] += bits
        total["diff_elems"] += elems
        total["worst_batch_bits"] = max(total["worst_batch_bits"], bits)
    return total


def prefix_and_permuted_batches(Ms, pool_rows: int, perm: torch.Tensor, device) -> list:
    """For each M: the first M pool rows in order, and the same M rows in a
    permuted order (so every row also moves position)."""
    out = []
    for M in Ms:
        pre = torch.arange(M, dtype=torch.int64)
        p = perm[perm < M][:M] if M <= pool_rows else None
        out.append(pre.to(device))
        if p is not None and M > 1:
            out.append(p.to(device=device, dtype=torch.int64))
    return out


def rerun_determinism(run, x: torch.Tensor, reruns: int) -> dict:
    """Compute ``run(x)`` ``reruns`` more times; compare each with the first."""
    ref = run(x).clone()
    rows = torch.arange(ref.shape[0], dtype=torch.int64, device=x.device)
    diff_runs = bits_total = 0
    for _ in range(reruns):
        bits, _ = compare_rows(run(x), rows, ref, rows)
        bits_total += bits
        diff_runs += bits > 0
    return dict(reruns=reruns, differing_reruns=diff_runs, diff_bits=bits_total)


def replay_variation(run, x: torch.Tensor, replays: int) -> dict:
    """Replay one input ``replays`` times on the same buffers; count replays
    whose output differs in any bit from replay 0, and differing elements."""
    ref = run(x).clone()
    rows = torch.arange(ref.shape[0], dtype=torch.int64, device=x.device)
    counts = torch.zeros((replays - 1, 2), dtype=torch.int64, device=x.device)
    for r in range(1, replays):
        c = binding.bi_row_bitdiff(run(x), ref, None, None)
        counts[r - 1] = c.sum(dim=0)
    c = counts.cpu()
    differing = int((c[:, 0] > 0).sum())
    return dict(replays=replays, comparisons=replays - 1, differing=differing,
                frac_differing=differing / max(1, replays - 1),
                diff_elems=int(c[:, 1].sum()), elems_per_replay=int(ref.numel()))
