"""The entry points launch on the caller's stream and allocate nothing, so a
chain of them can run on a side stream and be captured in a HIP graph.  Every
replay (with eager work in between) must reproduce the eager bits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import dev_bf16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bi():
    need_gpu()
    from invariant_deterministic_amd import binding
    return binding


def _inputs():
    M, K, N = 300, 4096, 1024
    X = dev_bf16(synth.normal_bf16((M, K), 9001))
    G = dev_bf16(synth.normal_bf16((K,), 9002, mean=1.0, std=0.1))
    W = dev_bf16(synth.normal_bf16((N, K), 9003, std=0.02))
    A = dev_bf16(synth.normal_bf16((16, K), 9004, std=0.01))
    B = dev_bf16(synth.normal_bf16((N, 16), 9005, std=0.02))
    return X, G, W, A, B


def _chain(bi, X, G, W, A, B, H, Y, L, Z, Ya):
    bi.bi_rmsnorm(X, G, y=H, eps=workloads.EPS)
    bi.bi_gemm(H, W, y=Y)
    bi.bi_lora_shrink(H, A, y=L, split_k=8)
    bi.bi_lora_expand(L, B, base=Y, y=Z, scale=0.5)
    bi.bi_lora_shrink_atomic(H, A, y=Ya, split_k=8)


def _buffers(X, W):
    M, N = X.shape[0], W.shape[0]
    dev = X.device
    return (torch.empty_like(X), torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 16), dtype=torch.float32, device=dev),
            torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 16), dtype=torch.float32, device=dev))


def test_side_stream_matches_default_stream(bi):
    X, G, W, A, B = _inputs()
    ref = _buffers(X, W)
    _chain(bi, X, G, W, A, B, *ref)
    torch.cuda.synchronize()
    out = _buffers(X, W)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _chain(bi, X, G, W, A, B, *out)
    s.synchronize()
    for r, o in list(zip(ref, out))[:4]:
        assert torch.equal(r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32),
                           o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32))
    assert torch.allclose(ref[4], out[4], rtol=1e-5, atol=1e-5)   # the atomic control: values only


def test_graph_replays_reproduce_eager_bits(bi):
    X, G, W, A, B = _inputs()
    ref = _buffers(X, W)
    _chain(bi, X, G, W, A, B, *ref)
    torch.cuda.synchronize()
    out = _buffers(X, W)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _chain(bi, X, G, W, A, B, *out)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _chain(bi, X, G, W, A, B, *out)
    for rep in range(3):
        for t in out:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        for r, o in list(zip(ref, out))[:4]:
            if r.dtype == torch.bfloat16:
                assert torch.equal(r.view(torch.int16), o.view(torch.int16)), rep
            else:
                assert torch.equal(r.view(torch.int32), o.view(torch.int32)), rep
        assert torch.allclose(ref[4], out[4], rtol=1e-5, atol=1e-5), rep
        _chain(bi, X, G, W, A, B, *_buffers(X, W))   # eager work between replays
        torch.cuda.synchronize()


def test_graph_decode_step_follows_device_lengths(bi):
    """A decode step (RMSNorm over a batch of 4096 rows, which takes the
    several-rows-per-workgroup path, then attention over a paged-free cache)
    captured once; the sequence lengths live in device memory, so each replay
    after the lengths grow in place must give the bits an eager call with those
    lengths gives."""
    M, K = 4096, 4096
    X = dev_bf16(synth.normal_bf16((M, K), 9101))
    G = dev_bf16(synth.normal_bf16((K,), 9102, mean=1.0, std=0.1))
    B, H, Hkv, D, Tmax, split = 4, 32, 8, 128, 1100, 256
    q = dev_bf16(synth.normal_bf16((B, H, D), 9103))
    kc = dev_bf16(synth.normal_bf16((B, Tmax, Hkv, D), 9104))
    vc = dev_bf16(synth.normal_bf16((B, Tmax, Hkv, D), 9105))
    lens = torch.tensor([1, 255, 700, 1000], dtype=torch.int32, device=X.device)
    need = bi.bi_decode_attention_workspace_bytes(B, H, Tmax, D, split)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device)
    Hn = torch.empty_like(X)
    o = torch.empty((B, H, D), dtype=torch.bfloat16, device=X.device)

    def step():
        bi.bi_rmsnorm(X, G, y=Hn, eps=workloads.EPS)
        bi.bi_decode_attention(q, kc, vc, lens, o=o, split_size=split, ws=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    prev = None
    for rep in range(3):
        lens.add_(rep * 33)                      # the cache grows between steps
        torch.cuda.synchronize()
        Hn.zero_()
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"decode graph replay {rep} lens {lens.tolist()}")
        got_h, got_o = Hn.clone(), o.clone()
        step()                                   # eager with the same lengths
        torch.cuda.synchronize()
        assert torch.equal(got_h.view(torch.int16), Hn.view(torch.int16)), rep
        assert torch.equal(got_o.view(torch.int16), o.view(torch.int16)), rep
        assert int(got_o.view(torch.int16).ne(0).sum()) > 0, rep
        if prev is not None:                     # the replay read the new lengths
            assert not torch.equal(prev[0].view(torch.int16), got_o[0].view(torch.int16)), rep
        prev = got_o


def test_graph_replays_split_k_both_launch_forms(bi):
    """The fixed split-K GEMM in a graph: a 4-row batch (one launch, chunks
    folded in LDS) and a 40-row batch (partial kernel, then the fold), each
    with its own workspace.  Every replay, with eager work between, gives the
    eager bits and the eager partials."""
    K, N = 4096, 1024
    S = bi.bi_gemm_splitk_for(N, K)
    W = dev_bf16(synth.normal_bf16((N, K), 9011, std=0.02))
    cases = []
    for M in (4, 40):
        X = dev_bf16(synth.normal_bf16((M, K), 9012 + M))
        ws_e = torch.zeros(bi.bi_gemm_splitk_workspace_bytes(M, N, S), dtype=torch.uint8, device="cuda")
        y_e = bi.bi_gemm_splitk(X, W, split_k=S, ws=ws_e)
        ws_g = torch.zeros_like(ws_e)
        y_g = torch.empty_like(y_e)
        cases.append((X, ws_e, y_e, ws_g, y_g))
    torch.cuda.synchronize()

    def run():
        for X, _, _, ws_g, y_g in cases:
            bi.bi_gemm_splitk(X, W, y=y_g, split_k=S, ws=ws_g)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for _, _, _, ws_g, y_g in cases:
            ws_g.zero_()
            y_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"split-K graph replay {rep}")
        for X, ws_e, y_e, ws_g, y_g in cases:
            assert torch.equal(y_e.view(torch.int16), y_g.view(torch.int16)), (rep, X.shape[0])
            assert torch.equal(ws_e, ws_g), (rep, X.shape[0])
        for X, *_ in cases:                        # eager work between replays
            bi.bi_gemm_splitk(X, W, split_k=S)
        torch.cuda.synchronize()


def test_graph_replays_fill_mixed_launch(bi):
    """bi_gemm_fill at a shape where it takes the mixed launch (272 tiles of
    256 x 256: each XCD's last two run as 256 x 128 halves), captured in a
    graph: every replay, with eager work in between, reproduces the eager
    bits, which are bi_gemm's."""
    M, N, K = 4200, 4096, 256
    mixed = bi.bi_gemm_num_configs() - 1
    assert bi.bi_gemm_fill_config_id(M, N, K) == mixed
    X = dev_bf16(synth.normal_bf16((M, K), 9101))
    W = dev_bf16(synth.normal_bf16((N, K), 9102, std=0.02))
    ref = bi.bi_gemm(X, W)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bi.bi_gemm_fill(X, W, y=out)             # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bi.bi_gemm_fill(X, W, y=out)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"graph replay of the mixed fill launch {rep}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        bi.bi_gemm(X, W)                          # eager work between replays
        torch.cuda.synchronize()
