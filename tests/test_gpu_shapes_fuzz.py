"""Seeded random shapes through every entry point: sampled rows against the
fp64 oracle, and the bit-for-bit agreements the design promises (every GEMM
configuration, bi_gemm_fill, the shrink variants, the fused LoRA pair)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import check_bf16, check_f32, dev_bf16, host_f32, host_u16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    need_gpu()
    from invariant_deterministic_amd import binding
    return binding


def _sample(M, g, n=12):
    return np.unique(np.concatenate([[0, M - 1], g.integers(0, M, size=n)])).astype(np.int64)


@pytest.mark.parametrize("seed", range(10))
def test_fuzz_gemm(bi, seed):
    g = synth.rng(7000 + seed)
    M = int(g.integers(1, 3000))
    N = 8 * int(g.integers(1, 700))
    K = 32 * int(g.integers(1, 200))
    say(f"fuzz gemm seed={seed} M={M} N={N} K={K}")
    x = synth.normal_bf16((M, K), 7100 + seed)
    w = synth.normal_bf16((N, K), 7200 + seed, std=0.05)
    X, Wt = dev_bf16(x), dev_bf16(w)
    y = bi.bi_gemm(X, Wt)
    rows = _sample(M, g)
    check_bf16(host_u16(y[torch.from_numpy(rows).cuda()]), oracle.gemm(x[rows], w), "fuzz gemm")
    for cfg in range(bi.bi_gemm_num_configs()):
        assert torch.equal(bi.bi_gemm_with_config(cfg, X, Wt).view(torch.int16), y.view(torch.int16)), cfg
    assert torch.equal(bi.bi_gemm_fill(X, Wt).view(torch.int16), y.view(torch.int16))
    splits = [s for s in (1, 2, 4, 8, 16) if K % (32 * s) == 0]
    S = splits[int(g.integers(0, len(splits)))]
    ys = bi.bi_gemm_splitk(X[:64], Wt, split_k=S)
    check_bf16(host_u16(ys), oracle.gemm(x[:64], w), f"fuzz splitk S={S}")


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_rmsnorm_shrink_expand(bi, seed):
    g = synth.rng(7300 + seed)
    M = int(g.integers(1, 2500))
    K = 8 * int(g.integers(1, 2048))
    say(f"fuzz rmsnorm seed={seed} M={M} K={K}")
    x = synth.normal_bf16((M, K), 7400 + seed)
    w = synth.normal_bf16((K,), 7500 + seed, mean=1.0, std=0.1)
    y = bi.bi_rmsnorm(dev_bf16(x), dev_bf16(w), eps=workloads.EPS)
    rows = _sample(M, g)
    check_bf16(host_u16(y[torch.from_numpy(rows).cuda()]), oracle.rmsnorm(x[rows], w, workloads.EPS),
               "fuzz rmsnorm")

    S = int(g.choice([1, 2, 4, 8, 16]))
    Ks = 32 * S * int(g.integers(1, 40))
    N = 8 * int(g.integers(1, 900))
    say(f"fuzz shrink/expand seed={seed} M={M} K={Ks} S={S} N={N}")
    xs = synth.normal_bf16((M, Ks), 7600 + seed)
    a = synth.normal_bf16((16, Ks), 7700 + seed, std=0.01)
    X, A = dev_bf16(xs), dev_bf16(a)
    l = bi.bi_lora_shrink(X, A, split_k=S)
    assert torch.equal(bi.bi_lora_shrink_two_pass(X, A, split_k=S).view(torch.int32), l.view(torch.int32))
    check_f32(host_f32(l[torch.from_numpy(rows).cuda()]), oracle.lora_shrink(xs[rows], a), "fuzz shrink")
    check_f32(host_f32(bi.bi_lora_shrink_atomic(X, A, split_k=S)[torch.from_numpy(rows).cuda()]),
              oracle.lora_shrink(xs[rows], a), "fuzz shrink atomic")
    b = dev_bf16(synth.normal_bf16((N, 16), 7800 + seed, std=0.02))
    base = dev_bf16(synth.normal_bf16((M, N), 7900 + seed))
    ye = bi.bi_lora_expand(l, b, base=base, scale=0.75)
    if S <= 8:
        yf = bi.bi_lora_shrink_expand(X, A, b, base=base, scale=0.75, split_k=S)
        assert torch.equal(yf.view(torch.int16), ye.view(torch.int16))
    ref = oracle.lora_expand(host_f32(l[torch.from_numpy(rows).cuda()]), host_u16(b),
                             host_u16(base[torch.from_numpy(rows).cuda()]), 0.75)
    check_bf16(host_u16(ye[torch.from_numpy(rows).cuda()]), ref, "fuzz expand")


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_attention(bi, seed):
    g = synth.rng(8000 + seed)
    B = int(g.integers(1, 9))
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.integers(1, 9))
    D = int(g.choice([64, 128]))
    split = int(g.choice([128, 256, 512]))
    Tmax = int(g.integers(1, 1600))
    H = Hkv * G
    lens = g.integers(1, Tmax + 1, size=B).astype(np.int32)
    say(f"fuzz attention seed={seed} B={B} H={H} Hkv={Hkv} D={D} split={split} Tmax={Tmax}")
    q = synth.normal_bf16((B, H, D), 8100 + seed)
    k = synth.normal_bf16((B, Tmax, Hkv, D), 8200 + seed)
    v = synth.normal_bf16((B, Tmax, Hkv, D), 8300 + seed)
    o = bi.bi_decode_attention(dev_bf16(q), dev_bf16(k), dev_bf16(v),
                               torch.from_numpy(lens).cuda(), split_size=split)
    check_bf16(host_u16(o), oracle.decode_attention(q, k, v, lens), "fuzz attention")
