"""GPU parity, pins, replays and invariance of the LoRA shrink variants."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import check_f32, dev_bf16, host_f32, host_u32, need_gpu, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def bi():
    need_gpu()
    from invariant_deterministic_amd import binding
    return binding


def _golden(name):
    with open(os.path.join(GOLDEN, "fixed_order_pins.txt")) as f:
        for ln in f:
            if ln.startswith(name + " |"):
                return [c.strip() for c in ln.split("|")]
    raise KeyError(name)


VARIANTS = ("det8", "det8_two_pass", "unsplit", "atomic8")


def run_variant(bi, name, X, A, y=None, ws=None):
    if name == "det8":
        return bi.bi_lora_shrink(X, A, y=y, split_k=8)
    if name == "det8_two_pass":
        return bi.bi_lora_shrink_two_pass(X, A, y=y, split_k=8, ws=ws)
    if name == "unsplit":
        return bi.bi_lora_shrink(X, A, y=y, split_k=1)
    return bi.bi_lora_shrink_atomic(X, A, y=y, split_k=8)


def test_shrink_parity_all_sizes_all_variants(bi):
    x, a = workloads.lora_inputs()
    X, A = dev_bf16(x), dev_bf16(a)
    for M in workloads.LORA["Ms"]:
        ref = oracle.lora_shrink(x[:M], a)
        for v in VARIANTS:
            say(f"shrink {v} M={M}")
            check_f32(host_f32(run_variant(bi, v, X[:M], A)), ref, f"{v} M={M}")


@pytest.mark.parametrize("split", [1, 2, 4, 8, 16])
def test_shrink_integer_inputs_bitwise(bi, split):
    """Integer inputs: exact in every order, so every variant -- the atomic one
    included -- equals the exact value bit for bit."""
    for M in (1, 17, 130):
        x = synth.int_bf16((M, 4096), 7 + M, -4, 4)
        a = synth.int_bf16((16, 4096), 8 + M, -4, 4)
        want = oracle.lora_shrink(x, a).astype(np.float32)
        X, A = dev_bf16(x), dev_bf16(a)
        say(f"shrink int split={split} M={M}")
        assert np.array_equal(host_f32(bi.bi_lora_shrink(X, A, split_k=split)), want)
        assert np.array_equal(host_f32(bi.bi_lora_shrink_two_pass(X, A, split_k=split)), want)
        assert np.array_equal(host_f32(bi.bi_lora_shrink_atomic(X, A, split_k=split)), want)


def _assoc_rows(M, positions):
    """Rows carrying the combine-order pin at the given positions; others random."""
    row = _golden("shrink_split8_fixed_order")
    K = int(row[1])
    x = synth.normal_bf16((M, K), 4100 + M)
    a = np.zeros((16, K), np.float32)
    pin = np.zeros(K, np.float32)
    for term in row[2].split(","):
        k, xv_w = term.split(":")
        xv, wv = xv_w.split("*")
        pin[int(k)] = float(xv)
        a[:, int(k)] = float(wv)
    for p in positions:
        x[p] = synth.f32_to_bf16_bits(pin)
    return x, synth.f32_to_bf16_bits(a), row


def test_shrink_combine_order_pin(bi):
    """p0 = 1, p1 = p2 = 2^-24: the fixed order gives exactly 1.0f; the unsplit
    pass also gives 1.0f; the atomic control may give 1.0f or 1.0f + 1 ulp."""
    M = 64
    pos = [0, 5, 17, 63]
    x, a, row = _assoc_rows(M, pos)
    X, A = dev_bf16(x), dev_bf16(a)
    det = host_u32(bi.bi_lora_shrink(X, A, split_k=8))
    two = host_u32(bi.bi_lora_shrink_two_pass(X, A, split_k=8))
    uns = host_u32(bi.bi_lora_shrink(X, A, split_k=1))
    want = int(row[4], 16)
    assert np.all(det[pos] == want), [hex(v) for v in det[pos].ravel()]
    assert np.all(two[pos] == want)
    assert np.all(uns[pos] == int(_golden("shrink_unsplit")[4], 16))
    allowed = {int(v, 16) for v in _golden("shrink_atomic_any_of")[4].split(",")}
    for _ in range(20):
        at = host_u32(bi.bi_lora_shrink_atomic(X, A, split_k=8))
        assert set(at[pos].ravel().tolist()) <= allowed
    check_f32(host_f32(bi.bi_lora_shrink(X, A, split_k=8)), oracle.lora_shrink(x, a), "pin rows")


@pytest.mark.parametrize("split", [1, 2, 4, 8, 16])
def test_shrink_fused_equals_two_pass_bitwise(bi, split):
    """The single-kernel (LDS) combine and the two-pass (HBM workspace) combine
    compute the same partials and fold them in the same order: same bits."""
    for M in (1, 5, 64, 1000):
        x, a = workloads.lora_inputs(M)
        X, A = dev_bf16(x), dev_bf16(a)
        f = host_u32(bi.bi_lora_shrink(X, A, split_k=split))
        t = host_u32(bi.bi_lora_shrink_two_pass(X, A, split_k=split))
        assert np.array_equal(f, t), (split, M)


def test_shrink_workspace_partials_and_exact_combine(bi):
    """The det-8 workspace holds p_s; each p_s matches the oracle over its chunk,
    and y is bit-exactly the oracle's fp32 left fold of those partials."""
    x, a = workloads.lora_inputs(512)
    M, K = x.shape
    X, A = dev_bf16(x), dev_bf16(a)
    ws = torch.zeros(bi.bi_lora_shrink_workspace_bytes(M, 16, 8), dtype=torch.uint8, device="cuda")
    y = host_f32(bi.bi_lora_shrink(X, A, split_k=8, ws=ws))
    p = host_f32(ws.view(torch.float32)[: 8 * M * 16]).reshape(8, M, 16)
    ws2 = torch.zeros_like(ws)
    y2 = host_f32(bi.bi_lora_shrink_two_pass(X, A, split_k=8, ws=ws2))
    assert np.array_equal(host_u32(ws2), host_u32(ws)) and np.array_equal(y2.view(np.uint32), y.view(np.uint32))
    ch = K // 8
    for s in range(8):
        check_f32(p[s], oracle.gemm(x[:, s * ch:(s + 1) * ch].copy(), a[:, s * ch:(s + 1) * ch].copy()),
                  f"partial {s}")
    assert np.array_equal(y.view(np.uint32), oracle.combine_f32(p).view(np.uint32))


def test_shrink_replays(bi):
    """1000 identical-input replays on the same buffers: the deterministic
    split-K and the unsplit pass never vary; the atomic control does."""
    from invariant_deterministic_amd import harness
    c = workloads.LORA
    x, a = workloads.lora_inputs()
    X, A = dev_bf16(x), dev_bf16(a)
    results = {}
    for M in c["Ms"]:
        Xm = X[:M]
        y = torch.empty((M, 16), dtype=torch.float32, device="cuda")
        ws = torch.empty(bi.bi_lora_shrink_workspace_bytes(M, 16, 8), dtype=torch.uint8,
                         device="cuda")
        for v in VARIANTS:
            say(f"replays {v} M={M}")
            r = harness.replay_variation(lambda xb: run_variant(bi, v, xb, A, y=y, ws=ws), Xm,
                                         c["replays"])
            results[(v, M)] = r
            if v != "atomic8":
                assert r["differing"] == 0, (v, M, r)
    for M in c["Ms"]:
        r = results[("atomic8", M)]
        say(f"atomic8 M={M}: {r['differing']}/{r['comparisons']} replays differ "
            f"({100 * r['frac_differing']:.2f}%), {r['diff_elems']} elements")
    assert results[("atomic8", 4096)]["differing"] > 0, "the atomic control never varied"


def test_shrink_batch_invariance(bi):
    from invariant_deterministic_amd import harness
    c = workloads.LORA
    x, a = workloads.lora_inputs()
    X, A = dev_bf16(x), dev_bf16(a)
    perm = torch.from_numpy(synth.permutation(x.shape[0], c["pos_seed"]))
    probes = [0, 1, 7, 15, 16, 63, 64, 511, 4095]
    batches = harness.prefix_and_permuted_batches(c["Ms"] + (3, 100, 1000), x.shape[0], perm, "cuda")
    for split in (8, 1):
        say(f"shrink invariance split={split}")
        r = harness.batch_invariance(lambda xb: bi.bi_lora_shrink(xb, A, split_k=split), X,
                                     probes, batches)
        assert r["rows"] > 20 and r["diff_bits"] == 0, (split, r)


def test_shrink_strided_output(bi):
    x, a = workloads.lora_inputs(40)
    X, A = dev_bf16(x), dev_bf16(a)
    out = torch.full((40, 24), 7.0, dtype=torch.float32, device="cuda")
    bi.bi_lora_shrink(X, A, y=out[:, :16], split_k=8)
    o = host_f32(out)
    check_f32(o[:, :16], oracle.lora_shrink(x, a), "strided")
    assert np.all(o[:, 16:] == 7.0)
    out[:] = 7.0
    bi.bi_lora_shrink_atomic(X, A, y=out[:, :16], split_k=8)
    o = host_f32(out)
    check_f32(o[:, :16], oracle.lora_shrink(x, a), "strided atomic")
    assert np.all(o[:, 16:] == 7.0)


@pytest.mark.parametrize("K", [512, 1024, 2048, 8192, 14336])
def test_shrink_other_k_every_path(bi, K):
    """K other than 4096 reaches the other kernels: the staged kernel only at 16
    (S = 8) or 8/16 (S = 16) steps a chunk; the streamed kernel at the other
    compiled step counts (8, 32, 64, 128); the one-step-at-a-time loop at run-time
    counts (K = 14336: 56 steps a chunk at S = 8).  Exact integer inputs, every
    split that divides K, the three variants."""
    for split in (1, 2, 4, 8, 16):
        if K % (32 * split):
            continue
        for M in (1, 33):
            x = synth.int_bf16((M, K), K + M, -4, 4)
            a = synth.int_bf16((16, K), K + M + 1, -4, 4)
            want = oracle.lora_shrink(x, a).astype(np.float32)
            X, A = dev_bf16(x), dev_bf16(a)
            say(f"shrink K={K} split={split} M={M}")
            assert np.array_equal(host_f32(bi.bi_lora_shrink(X, A, split_k=split)), want), split
            assert np.array_equal(host_f32(bi.bi_lora_shrink_two_pass(X, A, split_k=split)), want)
            assert np.array_equal(host_f32(bi.bi_lora_shrink_atomic(X, A, split_k=split)), want)


@pytest.mark.parametrize("K,split", [(4096, 8), (4096, 16), (8192, 16)])
def test_shrink_staged_persistent_blocks(bi, K, split):
    """The staged kernel is persistent: with more 16-row blocks than
    workgroups each workgroup runs several blocks, its loads running one block
    ahead.  M = 8209 gives 514 blocks (two or three per workgroup on 256 CUs)
    and a ragged last block; exact integer inputs."""
    M = 8209
    x = synth.int_bf16((M, K), K + split, -4, 4)
    a = synth.int_bf16((16, K), K + split + 1, -4, 4)
    want = oracle.lora_shrink(x, a).astype(np.float32)
    X, A = dev_bf16(x), dev_bf16(a)
    say(f"shrink staged K={K} split={split} M={M}")
    assert np.array_equal(host_f32(bi.bi_lora_shrink(X, A, split_k=split)), want)


@pytest.mark.parametrize("M", [100, 3000])
def test_shrink_strided_inputs_same_bits(bi, M):
    """x and a as column slices of wider buffers (row strides K + 64 and K + 8
    elements): every path reads rows through the stride, so the bits equal
    those of the contiguous inputs.  M = 100 runs the 8-row blocks of the
    staged kernel, M = 3000 the 16-row ones; split 4 and the unsplit pass run
    the streamed kernel."""
    x, a = workloads.lora_inputs(M)
    K = x.shape[1]
    X, A = dev_bf16(x), dev_bf16(a)
    Xw = torch.zeros((M, K + 64), dtype=X.dtype, device="cuda")
    Aw = torch.zeros((a.shape[0], K + 8), dtype=A.dtype, device="cuda")
    Xw[:, 32:32 + K] = X
    Aw[:, :K] = A
    Xs, As = Xw[:, 32:32 + K], Aw[:, :K]
    assert Xs.stride(0) == K + 64 and As.stride(0) == K + 8
    ref = oracle.lora_shrink(x, a)
    for name, fn in (("det8", lambda xx, aa: bi.bi_lora_shrink(xx, aa, split_k=8)),
                     ("split4", lambda xx, aa: bi.bi_lora_shrink(xx, aa, split_k=4)),
                     ("unsplit", lambda xx, aa: bi.bi_lora_shrink(xx, aa, split_k=1)),
                     ("two_pass", lambda xx, aa: bi.bi_lora_shrink_two_pass(xx, aa, split_k=8))):
        say(f"shrink strided inputs {name} M={M}")
        dense = host_u32(fn(X, A))
        strided = host_u32(fn(Xs, As))
        assert np.array_equal(dense, strided), name
        check_f32(strided.view(np.float32), ref, f"strided {name} M={M}")
