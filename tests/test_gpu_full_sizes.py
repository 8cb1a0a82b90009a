"""Sampled parity at the largest sizes the bench sweep times, in the same
launch configurations: decode attention at B = 64, T = 4096 (split 256); LoRA
expand at M = 16384; the shrink variants and RMSNorm at M = 65536.  The oracle
computes sampled rows (sequences) one by one; each sampled row is also run
alone and must match its row of the big batch bit for bit."""
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


def _rows(M, seed, n=16):
    edges = [0, 1, 15, 16, 255, 256, M // 2, M - 2, M - 1]
    r = synth.rng(seed).integers(0, M, size=n)
    return np.unique(np.concatenate([np.array(edges), r])).astype(np.int64)


def test_attention_b64_t4096_sampled(bi):
    B, H, Hkv, D, T, split = 64, 32, 8, 128, 4096, 256
    q = synth.device_normal_bf16((B, H, D), 901)
    k = synth.device_normal_bf16((B, T, Hkv, D), 902)
    v = synth.device_normal_bf16((B, T, Hkv, D), 903)
    lens = np.full(B, T, np.int32)
    lens[[3, 10, 17, 40, 63]] = [1, 255, 256, 257, 4095]     # ragged against the split
    L = torch.from_numpy(lens).cuda()
    say("attention B=64 T=4096 split=256")
    o = host_u16(bi.bi_decode_attention(q, k, v, L, split_size=split))
    for b in (0, 3, 10, 17, 31, 40, 63):
        kb, vb = host_u16(k[b:b + 1]), host_u16(v[b:b + 1])
        ref = oracle.decode_attention(host_u16(q[b:b + 1]), kb, vb, lens[b:b + 1])
        check_bf16(o[b:b + 1], ref, f"attention b={b} T={lens[b]}")
        solo = host_u16(bi.bi_decode_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], L[b:b + 1],
                                               split_size=split))
        assert np.array_equal(solo, o[b:b + 1]), b


def test_expand_m16384_sampled(bi):
    M, N, R = 16384, 4096, 16
    lt = synth.device_normal_bf16((M, R), 911, std=0.5, dtype=torch.float32)
    bw = synth.device_normal_bf16((N, R), 912, std=0.01)
    base = synth.device_normal_bf16((M, N), 913)
    say("expand M=16384")
    y = bi.bi_lora_expand(lt, bw, base=base, scale=0.5)
    rows = _rows(M, 914)
    idx = torch.from_numpy(rows).cuda()
    ys = host_u16(y[idx])
    ref = oracle.lora_expand(host_f32(lt[idx]), host_u16(bw), host_u16(base[idx]), 0.5)
    check_bf16(ys, ref, "expand M=16384")
    for j, r in enumerate(rows[:6]):
        solo = host_u16(bi.bi_lora_expand(lt[r:r + 1], bw, base=base[r:r + 1], scale=0.5))
        assert np.array_equal(solo[0], ys[j]), int(r)


def test_shrink_m65536_sampled(bi):
    M, K = 65536, 4096
    x = synth.device_normal_bf16((M, K), 921)
    a = synth.normal_bf16((16, K), 922, std=0.01)
    A = dev_bf16(a)
    rows = _rows(M, 923)
    idx = torch.from_numpy(rows).cuda()
    xs = host_u16(x[idx])
    ref = oracle.lora_shrink(xs, a)
    for name, fn in (("det8", lambda t: bi.bi_lora_shrink(t, A, split_k=8)),
                     ("unsplit", lambda t: bi.bi_lora_shrink(t, A, split_k=1)),
                     ("atomic8", lambda t: bi.bi_lora_shrink_atomic(t, A, split_k=8))):
        say(f"shrink {name} M=65536")
        y = fn(x)
        ys = host_f32(y[idx])
        check_f32(ys, ref, f"shrink {name} M=65536")
        if name != "atomic8":
            for j, r in enumerate(rows[:6]):
                solo = host_f32(fn(x[r:r + 1]))
                assert np.array_equal(solo[0].view(np.uint32), ys[j].view(np.uint32)), (name, int(r))


def test_rmsnorm_m65536_sampled(bi):
    M, K = 65536, 4096
    x = synth.device_normal_bf16((M, K), 931)
    w = synth.normal_bf16((K,), 932, mean=1.0, std=0.1)
    W = dev_bf16(w)
    say("rmsnorm M=65536")
    y = bi.bi_rmsnorm(x, W, eps=workloads.EPS)
    rows = _rows(M, 933)
    idx = torch.from_numpy(rows).cuda()
    ys = host_u16(y[idx])
    check_bf16(ys, oracle.rmsnorm(host_u16(x[idx]), w, workloads.EPS), "rmsnorm M=65536")
    for j, r in enumerate(rows[:6]):
        solo = host_u16(bi.bi_rmsnorm(x[r:r + 1], W, eps=workloads.EPS))
        assert np.array_equal(solo[0], ys[j]), int(r)
