"""GPU parity and invariance of bi_lora_expand, alone and after the shrink."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import check_bf16, dev_bf16, host_u16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    need_gpu()
    from invariant_deterministic_amd import binding
    return binding


def test_expand_integer_inputs_bitwise(bi):
    g = synth.rng(901)
    for M, N in ((1, 8), (70, 264), (200, 4096)):
        l = g.integers(-20, 20, size=(M, 16)).astype(np.float32)
        b = synth.int_bf16((N, 16), M + 902, -4, 4)
        base = synth.int_bf16((M, N), M + 903, -64, 64)
        for scale, bs in ((1.0, base), (2.0, None)):
            want = oracle.bf16_round(oracle.lora_expand(l, b, bs, scale=scale))
            y = bi.bi_lora_expand(torch.from_numpy(l).cuda(), dev_bf16(b),
                                  None if bs is None else dev_bf16(bs), scale=scale)
            assert np.array_equal(host_u16(y), want), (M, N, scale)


def test_expand_parity_and_in_place(bi):
    M, N = 300, 4096
    l = (synth.rng(904).standard_normal((M, 16)) * 0.5).astype(np.float32)
    b = synth.normal_bf16((N, 16), 905, std=0.02)
    base = synth.normal_bf16((M, N), 906)
    ref = oracle.lora_expand(l, b, base, scale=0.5)
    L, B, Y = torch.from_numpy(l).cuda(), dev_bf16(b), dev_bf16(base)
    out = host_u16(bi.bi_lora_expand(L, B, Y, scale=0.5))
    check_bf16(out, ref, "expand")
    bi.bi_lora_expand(L, B, Y, y=Y, scale=0.5)          # in place
    assert np.array_equal(host_u16(Y), out)


def test_expand_batch_invariance(bi):
    from invariant_deterministic_amd import harness
    N, pool = 1032, 600
    l = synth.rng(907).standard_normal((pool, 16)).astype(np.float32)
    b = synth.normal_bf16((N, 16), 908, std=0.05)
    L, B = torch.from_numpy(l).cuda(), dev_bf16(b)
    perm = torch.from_numpy(synth.permutation(pool, 909))
    batches = harness.prefix_and_permuted_batches((1, 3, 64, 65, 599), pool, perm, "cuda")
    r = harness.batch_invariance(lambda lb: bi.bi_lora_expand(lb, B, scale=2.0), L,
                                 [0, 1, 2, 63, 64, 598], batches)
    assert r["rows"] > 10 and r["diff_bits"] == 0, r


def test_shrink_then_expand_end_to_end(bi):
    """y = base + scale * (x . A^T) . B^T with the deterministic split-K shrink:
    within tolerance of the oracle and bitwise batch-invariant."""
    x, a = workloads.lora_inputs(257)
    N = 4096
    b = synth.normal_bf16((N, 16), 910, std=0.02)
    base = synth.normal_bf16((257, N), 911)
    X, A, B, BASE = dev_bf16(x), dev_bf16(a), dev_bf16(b), dev_bf16(base)

    def run(rows):
        idx = torch.from_numpy(np.asarray(rows, np.int64)).cuda()
        l = bi.bi_lora_shrink(X.index_select(0, idx), A, split_k=8)
        return host_u16(bi.bi_lora_expand(l, B, BASE.index_select(0, idx), scale=2.0))

    full = run(range(257))
    l_ref = oracle.lora_shrink(x, a).astype(np.float32)
    check_bf16(full, oracle.lora_expand(l_ref, b, base, scale=2.0), "shrink+expand")
    for i in (0, 100, 256):
        assert np.array_equal(run([i])[0], full[i])
    say("shrink -> expand: parity and single-row invariance ok")


@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_shrink_expand_fused_equals_two_calls(bi, split):
    """One launch gives the bits of bi_lora_shrink followed by bi_lora_expand
    (y and the optional l), with and without base, at ragged M and N."""
    K = 4096
    a = dev_bf16(synth.normal_bf16((16, K), 941, std=0.01))
    for M, N in ((1, 8), (17, 520), (300, 4096), (1000, 5000)):
        say(f"shrink_expand split={split} M={M} N={N}")
        x = dev_bf16(synth.normal_bf16((M, K), 942 + M))
        b = dev_bf16(synth.normal_bf16((N, 16), 943 + N, std=0.02))
        base = dev_bf16(synth.normal_bf16((M, N), 944 + M))
        for bs, scale in ((base, 0.5), (None, 2.0)):
            l_ref = bi.bi_lora_shrink(x, a, split_k=split)
            y_ref = bi.bi_lora_expand(l_ref, b, base=bs, scale=scale)
            l = torch.empty_like(l_ref)
            y = bi.bi_lora_shrink_expand(x, a, b, base=bs, l=l, scale=scale, split_k=split)
            assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32)), (M, N)
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (M, N, bs is None)


def test_shrink_expand_parity_invariance_and_in_place(bi):
    M, K, N = 300, 4096, 4096
    x = synth.normal_bf16((M, K), 951)
    a = synth.normal_bf16((16, K), 952, std=0.01)
    b = synth.normal_bf16((N, 16), 953, std=0.02)
    base = synth.normal_bf16((M, N), 954)
    X, A, B, BASE = dev_bf16(x), dev_bf16(a), dev_bf16(b), dev_bf16(base)
    y = host_u16(bi.bi_lora_shrink_expand(X, A, B, base=BASE, scale=0.5))
    l64 = oracle.lora_shrink(x, a)
    check_bf16(y, oracle.lora_expand(l64.astype(np.float32), b, base, scale=0.5), "shrink_expand")
    for r in (0, 1, 15, 16, 299):
        solo = host_u16(bi.bi_lora_shrink_expand(X[r:r + 1], A, B, base=BASE[r:r + 1], scale=0.5))
        assert np.array_equal(solo[0], y[r]), r
    inplace = BASE.clone()
    bi.bi_lora_shrink_expand(X, A, B, base=inplace, y=inplace, scale=0.5)
    assert np.array_equal(host_u16(inplace), y)


@pytest.mark.parametrize("N", [1032, 4096])
def test_expand_strided_operands_same_bits(bi, N):
    """l, b, base and y as slices of wider buffers (row strides 20, 24, N + 8
    and N + 16 elements): the same bits as with contiguous operands.  N = 1032
    leaves a last column slice of 8 columns, whose b rows past N are never
    used."""
    M = 77
    l = synth.rng(910).standard_normal((M, 16)).astype(np.float32)
    b = synth.normal_bf16((N, 16), 911, std=0.05)
    base = synth.normal_bf16((M, N), 912)
    L, B, BASE = torch.from_numpy(l).cuda(), dev_bf16(b), dev_bf16(base)
    dense = host_u16(bi.bi_lora_expand(L, B, BASE, scale=0.75))
    Lw = torch.zeros((M, 20), dtype=torch.float32, device="cuda")
    Bw = torch.zeros((N, 24), dtype=B.dtype, device="cuda")
    Basew = torch.zeros((M, N + 8), dtype=BASE.dtype, device="cuda")
    Yw = torch.full((M, N + 16), 3.0, dtype=BASE.dtype, device="cuda")
    Lw[:, :16] = L
    Bw[:, 8:24] = B
    Basew[:, :N] = BASE
    say(f"expand strided N={N}")
    bi.bi_lora_expand(Lw[:, :16], Bw[:, 8:24], Basew[:, :N], y=Yw[:, :N], scale=0.75)
    yw = host_u16(Yw)
    assert np.array_equal(yw[:, :N], dense)
    assert np.all(yw[:, N:] == host_u16(torch.full((1,), 3.0, dtype=BASE.dtype))[0])
    check_bf16(dense, oracle.lora_expand(l, b, base, scale=0.75), f"expand N={N}")
