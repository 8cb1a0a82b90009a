"""GPU parity, pins and batch invariance of bi_gemm against the fp64 oracle."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import synth, workloads
from tests.gpu_util import check_bf16, dev_bf16, host_u16, need_gpu, say

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


@pytest.mark.parametrize("M,N,K", [(1, 1024, 1024), (33, 1032, 1024), (257, 520, 4096),
                                   (300, 4096, 640), (70, 264, 14336)])
def test_gemm_integer_inputs_bitwise_all_configs(bi, M, N, K):
    """Integer inputs: every fp32 partial sum is exact in any order, so each
    configuration must equal the oracle's exact result rounded to bf16, bit for
    bit (this pins indexing, layout, masking and the RNE epilogue)."""
    x = synth.int_bf16((M, K), M + N, -4, 4)
    w = synth.int_bf16((N, K), M * N, -4, 4)
    want = oracle.bf16_round(oracle.gemm(x, w))
    X, Wt = dev_bf16(x), dev_bf16(w)
    for cfg in range(bi.bi_gemm_num_configs()):
        say(f"gemm int M={M} N={N} K={K} cfg={cfg}")
        y = host_u16(bi.bi_gemm_with_config(cfg, X, Wt))
        assert np.array_equal(y, want), f"cfg {cfg}: {int((y != want).sum())} mismatches"
    assert np.array_equal(host_u16(bi.bi_gemm(X, Wt)), want)


def test_gemm_rne_ties_in_epilogue(bi):
    """Exact integer results 257..296 (bf16 quantum 2 there): the odd ones are
    exact ties and must go to the even neighbour."""
    K, N, M = 1024, 64, 40
    x = np.zeros((M, K), np.float32)
    x[:, 0] = 200.0
    x[:, 1] = 57.0 + np.arange(M)
    w = np.zeros((N, K), np.float32)
    w[:, 0] = 1.0
    w[:, 1] = 1.0
    xb, wb = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w)
    y = host_u16(bi.bi_gemm(dev_bf16(xb), dev_bf16(wb)))
    want = oracle.bf16_round(oracle.gemm(xb, wb))
    assert np.array_equal(oracle.gemm(xb, wb)[:, 0], 257.0 + np.arange(M))
    assert np.array_equal(y, want)


def test_gemm_k_order_pin(bi):
    """One ascending K pass with fp32 rounding between matrix-core steps gives
    0x3F80; a reversed or split reduction would give 0x3F81."""
    row = _golden("gemm_korder_ascending")
    K = int(row[1])
    x = np.zeros((5, K), np.float32)
    w = np.zeros((16, K), np.float32)
    for term in row[2].split(","):
        k, xv_w = term.split(":")
        xv, wv = xv_w.split("*")
        x[:, int(k)] = float(xv)
        w[3, int(k)] = float(wv)
    xb, wb = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w)
    X, Wt = dev_bf16(xb), dev_bf16(wb)
    for cfg in range(bi.bi_gemm_num_configs()):
        y = host_u16(bi.bi_gemm_with_config(cfg, X, Wt))
        assert np.all(y[:, 3] == int(row[4], 16)), [hex(v) for v in y[:, 3]]
    # the exact value lies within tolerance of the pinned bits too
    check_bf16(host_u16(bi.bi_gemm(X, Wt)), oracle.gemm(xb, wb), "k-order")


def test_gemm_identity_and_one_hot(bi):
    K = 1024
    x = synth.normal_bf16((70, K), 91)
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    y = host_u16(bi.bi_gemm(dev_bf16(x), dev_bf16(eye)))
    assert np.array_equal(y, x)
    w = synth.normal_bf16((520, K), 92)
    ks = np.array([0, 1, 15, 16, 63, 64, 511, 1023])
    oh = np.zeros((len(ks), K), np.uint16)
    oh[np.arange(len(ks)), ks] = 0x3F80
    y = host_u16(bi.bi_gemm(dev_bf16(oh), dev_bf16(w)))
    assert np.array_equal(y, w[:, ks].T)


def test_gemm_tiny_config_parity_and_invariance(bi):
    x, w, _ = workloads.tiny_inputs()
    X, Wt = dev_bf16(x), dev_bf16(w)
    solo = np.stack([host_u16(bi.bi_gemm(X[i:i + 1], Wt))[0] for i in range(64)])
    for M in workloads.TINY["Ms"]:
        say(f"gemm tiny M={M}")
        y = host_u16(bi.bi_gemm(X[:M], Wt))
        check_bf16(y, oracle.gemm(x[:M], w), f"tiny M={M}")
        assert np.array_equal(y, solo[:M])


@pytest.mark.parametrize("shape_index", [0, 1, 2, 3])
def test_gemm_llama8b_parity_sampled(bi, shape_index):
    """Full sizes, sampled rows: the oracle computes 24 rows (including tile
    edges) of each batch."""
    c = workloads.LLAMA8B
    K, N = c["shapes"][shape_index]
    x = workloads.llama8b_x(K)
    w = workloads.llama8b_w(shape_index)
    X, Wt = dev_bf16(x), dev_bf16(w)
    for M in (1, 127, 1000, 4096, 8192):
        say(f"gemm llama8b K={K} N={N} M={M}")
        y = bi.bi_gemm(X[:M], Wt)
        g = synth.rng(M)
        rows = np.unique(np.concatenate([np.array([0, M - 1], np.int64),
                                         np.array([r for r in (127, 128, 255, 256) if r < M], np.int64),
                                         g.integers(0, M, size=18)])).astype(np.int64)
        ys = host_u16(y[torch.from_numpy(rows).cuda()])
        check_bf16(ys, oracle.gemm(x[rows], w), f"K={K} N={N} M={M}")


def test_gemm_configs_agree_bitwise(bi):
    """All tile configurations run the same reduction order: identical bits."""
    x = synth.normal_bf16((300, 4096), 93)
    w = synth.normal_bf16((1024, 4096), 94, std=0.02)
    X, Wt = dev_bf16(x), dev_bf16(w)
    ref = host_u16(bi.bi_gemm_with_config(0, X, Wt))
    for cfg in range(1, bi.bi_gemm_num_configs()):
        assert np.array_equal(host_u16(bi.bi_gemm_with_config(cfg, X, Wt)), ref), cfg


def test_gemm_batch_invariance_sweep(bi):
    """Probe rows alone vs inside prefix and permuted batches over the M sweep,
    for every Llama-3-8B shape; plus reruns."""
    from invariant_deterministic_amd import harness
    c = workloads.LLAMA8B
    Ms = sorted(set(c["Ms"]) | set(c["extra_Ms"]))
    for si, (K, N) in enumerate(c["shapes"]):
        x = workloads.llama8b_x(K)
        X = dev_bf16(x)
        Wt = dev_bf16(workloads.llama8b_w(si))
        run = lambda xb: bi.bi_gemm(xb, Wt)
        perm = torch.from_numpy(synth.permutation(x.shape[0], c["perm_seed"]))
        probes = [0, 1, 4, 31, 32, 126, 127, 255, 256, 999, 2038, 4092, 4095, 8190, 8191]
        batches = harness.prefix_and_permuted_batches(Ms, x.shape[0], perm, "cuda")
        say(f"gemm invariance K={K} N={N}: {len(batches)} batches")
        r = harness.batch_invariance(run, X, probes, batches)
        assert r["rows"] > 50 and r["diff_bits"] == 0, r
        r = harness.rerun_determinism(run, X[:1000], 3)
        assert r["diff_bits"] == 0, r


def test_gemm_strided_and_m_zero(bi):
    x = synth.normal_bf16((40, 1024 + 64), 95)
    w = synth.normal_bf16((256, 1024 + 128), 96)
    X, Wt = dev_bf16(x), dev_bf16(w)
    out = torch.zeros((40, 256 + 8), dtype=torch.bfloat16, device="cuda")
    bi.bi_gemm(X[:, :1024], Wt[:, :1024], y=out[:, :256])
    o = host_u16(out)
    check_bf16(o[:, :256], oracle.gemm(x[:, :1024], w[:, :1024]), "strided")
    assert np.all(o[:, 256:] == 0)
    bi.bi_gemm(X[:0, :1024], Wt[:, :1024])


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320])
def test_gemm_wide_stages_short_k(bi, K):
    """K % 64 == 0 runs 64-k LDS stages: loops of one, two, three stages and
    ragged M and N edges give the same bits in every configuration, within
    tolerance of the oracle."""
    M, N = 300, 520
    x = synth.normal_bf16((M, K), 97 + K)
    w = synth.normal_bf16((N, K), 98 + K)
    X, Wt = dev_bf16(x), dev_bf16(w)
    say(f"gemm wide K={K}")
    y0 = host_u16(bi.bi_gemm_with_config(0, X, Wt))
    for cfg in range(1, bi.bi_gemm_num_configs()):
        assert np.array_equal(host_u16(bi.bi_gemm_with_config(cfg, X, Wt)), y0), cfg
    check_bf16(y0, oracle.gemm(x, w), f"wide K={K}")


@pytest.mark.parametrize("K", [32, 96, 1056])
def test_gemm_wide_and_narrow_stages_agree(bi, K):
    """K % 64 == 32 runs 32-k LDS stages.  Appending 32 zero columns to x and
    w (K + 32, a multiple of 64, so 64-k stages) adds exact zeros after the
    same ascending k steps: the two staging schemes must give the same bits,
    in every configuration."""
    M, N = 300, 520
    x = synth.normal_bf16((M, K), 99 + K)
    w = synth.normal_bf16((N, K), 100 + K)
    xp = np.zeros((M, K + 32), np.uint16)
    wp = np.zeros((N, K + 32), np.uint16)
    xp[:, :K], wp[:, :K] = x, w
    X, Wt, XP, WP = dev_bf16(x), dev_bf16(w), dev_bf16(xp), dev_bf16(wp)
    say(f"gemm narrow K={K} vs wide K={K + 32}")
    for cfg in range(bi.bi_gemm_num_configs()):
        narrow = host_u16(bi.bi_gemm_with_config(cfg, X, Wt))
        wide = host_u16(bi.bi_gemm_with_config(cfg, XP, WP))
        assert np.array_equal(narrow, wide), cfg
    check_bf16(narrow, oracle.gemm(x, w), f"narrow K={K}")


def test_gemm_fill_same_bits_as_bi_gemm(bi):
    """bi_gemm_fill picks its tile from M; every tile runs the same reduction
    order, so its bits equal bi_gemm's at every M and every projection, and
    rows stay batch-invariant across the sweep.  M = 2305 and 4200 end in a
    partly filled tile row."""
    from invariant_deterministic_amd import harness
    c = workloads.LLAMA8B
    for si, (K, N) in enumerate(c["shapes"]):
        x = workloads.llama8b_x(K)
        X = dev_bf16(x)
        Wt = dev_bf16(workloads.llama8b_w(si))
        for M in (1, 127, 512, 1000, 2048, 2305, 3000, 4096, 4200, 8192):
            say(f"gemm fill K={K} N={N} M={M} cfg={bi.bi_gemm_fill_config_id(M, N, K)}")
            assert torch.equal(bi.bi_gemm_fill(X[:M], Wt).view(torch.int16),
                               bi.bi_gemm(X[:M], Wt).view(torch.int16)), (K, N, M)
        perm = torch.from_numpy(synth.permutation(x.shape[0], c["perm_seed"]))
        probes = [0, 1, 127, 255, 999, 2047, 4095, 8191]
        batches = harness.prefix_and_permuted_batches((1, 500, 1000, 2048, 3000, 8192), x.shape[0],
                                                      perm, "cuda")
        r = harness.batch_invariance(lambda xb: bi.bi_gemm_fill(xb, Wt), X, probes, batches)
        assert r["rows"] > 20 and r["diff_bits"] == 0, r


@pytest.mark.parametrize("M,N", [(4096, 14336), (4200, 4096), (2305, 14336), (6144, 4096)])
def test_gemm_mixed_launch(bi, M, N):
    """The mixed launch (the last configuration) runs each XCD's full waves of
    256 x 256 tiles and cuts a tail of at most half a wave into 256 x 128
    halves; at M = 4200 and 2305 the last tile row is ragged, so some halves
    lie wholly past M and store nothing.  Its bits equal configuration 0's,
    and sampled columns match the oracle."""
    K = 256
    mixed = bi.bi_gemm_num_configs() - 1
    x = synth.normal_bf16((M, K), 411 + M)
    w = synth.normal_bf16((N, K), 412 + N, std=0.02)
    X, Wt = dev_bf16(x), dev_bf16(w)
    say(f"gemm mixed launch M={M} N={N} K={K}")
    y = host_u16(bi.bi_gemm_with_config(mixed, X, Wt))
    assert np.array_equal(y, host_u16(bi.bi_gemm_with_config(0, X, Wt)))
    cols = np.sort(np.random.default_rng(M + N).choice(N, 48, replace=False))
    check_bf16(y[:, cols], oracle.gemm(x, w[cols]), f"mixed M={M} N={N}")


def test_gemm_runs_one_config_at_every_m(bi):
    """bi_gemm's output equals that of its own configuration
    (bi_gemm_config_id(N, K), reported by bi_gemm_launch_plan) at every M: the
    dynamic half of the static check that M selects nothing but the number of
    workgroups."""
    for N, K in ((4096, 4096), (1024, 4096)):
        x = synth.normal_bf16((1000, K), 301 + N)
        w = synth.normal_bf16((N, K), 302 + N, std=0.02)
        X, Wt = dev_bf16(x), dev_bf16(w)
        cfg = bi.bi_gemm_config_id(N, K)
        kernels = {bi.bi_gemm_launch_plan(M, N, K)["kernel"] for M in (1, 33, 257, 1000)}
        assert len(kernels) == 1
        for M in (1, 33, 257, 1000):
            say(f"gemm planned config N={N} K={K} M={M} cfg={cfg}")
            assert torch.equal(bi.bi_gemm(X[:M], Wt).view(torch.int16),
                               bi.bi_gemm_with_config(cfg, X[:M], Wt).view(torch.int16)), (N, K, M)


def _two_term_sums(M: int, N: int, K: int, seed: int):
    """x rows with two ones (columns 0 and 1 + m) and w rows chosen so that
    every output y[m][n] = w[n][0] + w[n][1 + m] is a sum of two bf16 values
    1..15 binades apart, exact in fp32 (at most 24 significant bits), that
    then has to be rounded to bf16.  Mixed signs (cancellation), random
    significands (odd and even neighbours), exact ties (the second term half an
    output ulp), sums that carry into the next binade, and magnitudes from
    2^-100 to 2^125 (no fp32 subnormals)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = np.zeros((M, K), np.uint16)
    x[:, 0] = 0x3F80
    x[np.arange(M), 1 + np.arange(M)] = 0x3F80
    w = np.zeros((N, K), np.uint16)

    def bits(sign, e, mant):
        return ((sign.astype(np.uint32) << 15) | ((e + 127).astype(np.uint32) << 7)
                | mant.astype(np.uint32)).astype(np.uint16)

    E = g.integers(-100, 126, size=N)
    sa = g.integers(0, 2, size=N)
    ma = g.integers(0, 128, size=N)
    ma[: N // 8] = 127                         # 1.1111111: rounding up carries
    w[:, 0] = bits(sa, E, ma)
    d = g.integers(1, 16, size=(N, M))
    sb = g.integers(0, 2, size=(N, M))
    mb = g.integers(0, 128, size=(N, M))
    tie = g.random((N, M)) < 0.2                # b = +-2^(E-8): half an ulp of a
    d[tie], mb[tie] = 8, 0
    same = g.random((N, M)) < 0.5
    sb[same] = np.repeat(sa[:, None], M, axis=1)[same]
    w[:, 1:1 + M] = bits(sb, E[:, None] - d, mb)
    return x, w


def test_gemm_epilogue_rounds_arbitrary_fp32_sums(bi):
    """The fp32 -> bf16 rounding of the epilogue against the oracle's
    round-to-nearest-even, bit for bit, on 262,144 fp32 values that are not
    integers: every output is an exact two-term sum (see _two_term_sums), so
    its fp32 accumulator is exactly the fp64 oracle's value and only the final
    rounding can differ."""
    M, N, K = 64, 4096, 128
    x, w = _two_term_sums(M, N, K, 4242)
    exact = oracle.gemm(x, w)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)  # exact in fp32
    f32bits = exact.astype(np.float32).view(np.uint32)
    ties = ((f32bits & 0xFFFF) == 0x8000).sum()
    assert ties > 10000 and (exact != 0).all()
    want = oracle.bf16_round(exact)
    X, Wt = dev_bf16(x), dev_bf16(w)
    for cfg in range(bi.bi_gemm_num_configs()):
        say(f"gemm rounding of two-term sums cfg={cfg}")
        y = host_u16(bi.bi_gemm_with_config(cfg, X, Wt))
        bad = y != want
        assert not bad.any(), (cfg, int(bad.sum()), [hex(v) for v in f32bits[bad][:4]])
