"""GPU parity and invariance of bi_rmsnorm against the fp64 oracle."""
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


def test_rmsnorm_tiny_config_parity_and_invariance(bi):
    x, _, ones = workloads.tiny_inputs()
    c = workloads.TINY
    X, Wn = dev_bf16(x), dev_bf16(ones)
    solo = [host_u16(bi.bi_rmsnorm(X[i:i + 1], Wn, eps=workloads.EPS))[0] for i in range(64)]
    for M in c["Ms"]:
        y = host_u16(bi.bi_rmsnorm(X[:M], Wn, eps=workloads.EPS))
        say(f"rmsnorm tiny M={M}")
        check_bf16(y, oracle.rmsnorm(x[:M], ones, workloads.EPS), f"tiny M={M}")
        for i in range(M):
            assert np.array_equal(y[i], solo[i]), f"row {i} differs between M=1 and M={M}"
    # unit-weight rows: mean(y^2) = ms / (ms + eps)
    y = oracle.bf16_decode(host_u16(bi.bi_rmsnorm(X, Wn, eps=workloads.EPS)))
    xd = oracle.bf16_decode(x)
    ms = (xd * xd).mean(axis=1)
    assert np.allclose((y * y).mean(axis=1), ms / (ms + workloads.EPS), rtol=1e-2)


def test_rmsnorm_k4096_parity_all_sizes(bi):
    x, w = workloads.rmsnorm_inputs()
    X, Wt = dev_bf16(x), dev_bf16(w)
    for M in workloads.RMSNORM["Ms"]:
        say(f"rmsnorm K=4096 M={M}")
        y = host_u16(bi.bi_rmsnorm(X[:M], Wt, eps=workloads.EPS))
        check_bf16(y, oracle.rmsnorm(x[:M], w, workloads.EPS), f"M={M}")


def test_rmsnorm_batch_invariance_prefix_permuted_reruns(bi):
    from invariant_deterministic_amd import harness
    c = workloads.RMSNORM
    x, w = workloads.rmsnorm_inputs()
    X, Wt = dev_bf16(x), dev_bf16(w)
    run = lambda xb: bi.bi_rmsnorm(xb, Wt, eps=workloads.EPS)
    perm = torch.from_numpy(synth.permutation(x.shape[0], c["perm_seed"]))
    probes = [0, 1, 6, 7, 127, 128, 2047, 4095, 8191] + list(range(200, 8192, 997))
    # beyond the configured sizes (256 CUs): 1, 7 and 128 run one row per
    # 256-thread workgroup, 2048 and 3000 one row per wavefront, 4096 four rows
    # per workgroup, 4097 and 8192 four rows per wavefront (4097 with a partly
    # filled last wavefront), so rows meet every launch shape
    batches = harness.prefix_and_permuted_batches(tuple(c["Ms"]) + (3000, 4096, 4097), x.shape[0],
                                                  perm, "cuda")
    say("rmsnorm batch invariance")
    r = harness.batch_invariance(run, X, probes, batches)
    assert r["rows"] > 20 and r["diff_bits"] == 0, r
    r = harness.rerun_determinism(run, X, 10)
    assert r["diff_bits"] == 0, r


def test_rmsnorm_ragged_k_and_limits(bi):
    eps = workloads.EPS
    for K, M in ((8, 5), (1032, 3), (2056, 9), (16384, 2), (4104, 1)):
        say(f"rmsnorm K={K} M={M}")
        x = synth.normal_bf16((M, K), 10 + K)
        w = synth.normal_bf16((K,), 20 + K, mean=1.0, std=0.1)
        y = host_u16(bi.bi_rmsnorm(dev_bf16(x), dev_bf16(w), eps=eps))
        check_bf16(y, oracle.rmsnorm(x, w, eps), f"K={K}")
        # every row alone gives the same bits
        for i in range(M):
            yi = host_u16(bi.bi_rmsnorm(dev_bf16(x[i:i + 1]), dev_bf16(w), eps=eps))
            assert np.array_equal(yi[0], y[i])


@pytest.mark.parametrize("rows_per_cu", [10, 20])
def test_rmsnorm_one_wavefront_launches_ragged_k(bi, rows_per_cu):
    """The one-wavefront launches -- one row per wavefront at 6-12 rows per CU
    (8-12 at K <= 2048), four rows per wavefront at 16-32 (K > 2048) -- on
    ragged K, where some lanes of a virtual wavefront own no chunk, and with a
    partly filled last wavefront: oracle parity, and every sampled row equal
    to the same row alone (one row per 256-thread workgroup)."""
    eps = workloads.EPS
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = synth.rng(31 + rows_per_cu)
    for K in ((1032, 2056, 3080, 4096) if rows_per_cu == 10 else (2056, 3080, 4096)):
        M = rows_per_cu * cus + (3 if rows_per_cu == 20 else 0)
        say(f"rmsnorm one wavefront per row K={K} M={M}")
        x = synth.normal_bf16((M, K), 40 + K)
        w = synth.normal_bf16((K,), 50 + K, mean=1.0, std=0.1)
        X, Wt = dev_bf16(x), dev_bf16(w)
        y = host_u16(bi.bi_rmsnorm(X, Wt, eps=eps))
        rows = np.unique(np.concatenate([[0, 1, M - 1], g.integers(0, M, size=40)]))
        check_bf16(y[rows], oracle.rmsnorm(x[rows], w, eps), f"K={K}")
        for i in rows[:12]:
            yi = host_u16(bi.bi_rmsnorm(X[i:i + 1], Wt, eps=eps))
            assert np.array_equal(yi[0], y[i]), (K, int(i))


def test_rmsnorm_closed_forms(bi):
    K = 4096
    w = synth.normal_bf16((K,), 77, mean=1.0, std=0.1)
    rows = []
    for j in (-10, 0, 7):
        for s in (1.0, -1.0):
            rows.append(np.full(K, s * 2.0 ** j, np.float32))
    x = synth.f32_to_bf16_bits(np.stack(rows))
    x = np.vstack([x, np.zeros((1, K), np.uint16)])
    y = host_u16(bi.bi_rmsnorm(dev_bf16(x), dev_bf16(w), eps=0.0))
    ref = oracle.rmsnorm(x[:-1], w, 0.0)
    check_bf16(y[:-1], ref, "constant rows")
    # a zero row with eps > 0 gives exactly zero
    z = host_u16(bi.bi_rmsnorm(dev_bf16(x[-1:]), dev_bf16(w), eps=1e-6))
    assert np.all((z & 0x7FFF) == 0)


@pytest.mark.parametrize("M", [33, 2500, 4096])
def test_rmsnorm_in_place_and_strided(bi, M):
    """In place and with row strides: the bits of the plain call.  M = 2500 and
    4096 run two and four rows per workgroup (all of a workgroup's rows are
    read before any is written)."""
    x, w = workloads.rmsnorm_inputs()
    x = x[:M]
    ref = host_u16(bi.bi_rmsnorm(dev_bf16(x), dev_bf16(w), eps=workloads.EPS))
    X = dev_bf16(x)
    bi.bi_rmsnorm(X, dev_bf16(w), y=X, eps=workloads.EPS)
    assert np.array_equal(host_u16(X), ref)
    # strided input/output rows (ld > K)
    big = np.zeros((M, 4096 + 64), np.uint16)
    big[:, :4096] = x
    B = dev_bf16(big)
    out = torch.zeros((M, 4096 + 128), dtype=torch.bfloat16, device="cuda")
    bi.bi_rmsnorm(B[:, :4096], dev_bf16(w), y=out[:, :4096], eps=workloads.EPS)
    o = host_u16(out)
    assert np.array_equal(o[:, :4096], ref)
    assert np.all(o[:, 4096:] == 0)


def test_rmsnorm_m_zero_is_noop(bi):
    X = torch.zeros((0, 4096), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    y = bi.bi_rmsnorm(X, w)
    assert y.shape == (0, 4096)
