"""GPU parity and batch invariance of bi_decode_attention against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth
from tests.gpu_util import check_bf16, dev_bf16, host_u16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    need_gpu()
    from invariant_deterministic_amd import binding
    return binding


def _inputs(B, H, Hkv, D, Tmax, seed):
    q = synth.normal_bf16((B, H, D), seed)
    k = synth.normal_bf16((B, Tmax, Hkv, D), seed + 1)
    v = synth.normal_bf16((B, Tmax, Hkv, D), seed + 2)
    return q, k, v


def _run(bi, q, k, v, lens, split):
    Q, Kc, Vc = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    L = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    return host_u16(bi.bi_decode_attention(Q, Kc, Vc, L, split_size=split))


@pytest.mark.parametrize("H,Hkv,D,split", [(32, 8, 128, 256), (8, 8, 64, 128), (16, 2, 128, 512),
                                           (4, 1, 64, 256), (8, 4, 128, 128), (6, 2, 64, 512),
                                           (14, 2, 128, 256)])
def test_attention_parity(bi, H, Hkv, D, split):
    B, Tmax = 5, 1100
    q, k, v = _inputs(B, H, Hkv, D, Tmax, 700 + H)
    lens = [1, split - 1, split, split + 1, Tmax]        # ragged against the split size
    say(f"attention H={H} Hkv={Hkv} D={D} split={split}")
    o = _run(bi, q, k, v, lens, split)
    check_bf16(o, oracle.decode_attention(q, k, v, lens), f"H={H} D={D} split={split}")


def test_attention_single_token_returns_value_exactly(bi):
    B, H, Hkv, D, Tmax = 3, 8, 2, 128, 64
    q, k, v = _inputs(B, H, Hkv, D, Tmax, 720)
    o = _run(bi, q, k, v, [1, 1, 1], 256)
    for h in range(H):
        assert np.array_equal(o[:, h], v[:, 0, h // 4])


def test_attention_masked_tail_is_never_read(bi):
    B, H, Hkv, D, Tmax = 3, 8, 8, 64, 600
    q, k, v = _inputs(B, H, Hkv, D, Tmax, 730)
    lens = [300, 513, 1]
    ref = oracle.decode_attention(q, k, v, lens)
    for b, T in enumerate(lens):       # NaN garbage past each sequence's length
        k[b, T:] = 0x7FC0
        v[b, T:] = 0x7FC0
    o = _run(bi, q, k, v, lens, 256)
    assert np.all((o & 0x7F80) != 0x7F80), "a NaN leaked in"
    check_bf16(o, ref, "masked")


def test_attention_batch_invariance(bi):
    """Each sequence alone (B = 1) and inside batches of different sizes, at
    different positions, beside sequences of other lengths: identical bits."""
    H, Hkv, D, Tmax, split = 32, 8, 128, 1024, 256
    pool = 12
    q, k, v = _inputs(pool, H, Hkv, D, Tmax, 740)
    lens = synth.rng(741).integers(1, Tmax + 1, size=pool).astype(np.int32)
    solo = np.stack([_run(bi, q[i:i + 1], k[i:i + 1], v[i:i + 1], lens[i:i + 1], split)[0]
                     for i in range(pool)])
    g = synth.rng(742)
    total = 0
    for B in (2, 5, 12):
        for _ in range(3):
            idx = g.choice(pool, size=B, replace=False)
            o = _run(bi, q[idx], k[idx], v[idx], lens[idx], split)
            for j, i in enumerate(idx):
                assert np.array_equal(o[j], solo[i]), (B, j, i)
                total += 1
    say(f"attention invariance: {total} sequence placements, 0 differing bits")
    check_bf16(solo, oracle.decode_attention(q, k, v, lens), "solo vs oracle")


def test_attention_split_sizes_agree_within_tolerance(bi):
    B, H, Hkv, D, Tmax = 2, 8, 2, 128, 1500
    q, k, v = _inputs(B, H, Hkv, D, Tmax, 750)
    lens = [1500, 777]
    ref = oracle.decode_attention(q, k, v, lens)
    for split in (128, 256, 512):
        check_bf16(_run(bi, q, k, v, lens, split), ref, f"split {split}")


def test_attention_lengths_outside_range_are_clamped(bi):
    """lens below 1 act as 1 and above Tmax as Tmax (as the header says)."""
    B, H, Hkv, D, Tmax = 3, 8, 2, 64, 300
    q, k, v = _inputs(B, H, Hkv, D, Tmax, 760)
    o = _run(bi, q, k, v, [0, Tmax + 7, -5], 128)
    want = _run(bi, q, k, v, [1, Tmax, 1], 128)
    assert np.array_equal(o, want)
