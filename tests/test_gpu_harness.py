"""GPU tests of the invariance check itself (bi_row_bitdiff, exact against the
oracle's bit counts) and the dynamic-batch stream of the Llama-3-70B MLP shape."""
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


@pytest.mark.parametrize("dtype,nbits", [(np.uint16, 16), (np.uint32, 32)])
@pytest.mark.parametrize("cols", [1000, 1001, 4096])   # 16-byte vector path and element path
def test_bitdiff_matches_oracle_exactly(bi, dtype, nbits, cols):
    g = synth.rng(60 + nbits + cols)
    rows = 37
    a = g.integers(0, 1 << nbits, size=(rows, cols), dtype=np.uint64).astype(dtype)
    b = a.copy()
    flips = g.integers(0, rows * cols, size=300)
    bitsel = g.integers(0, nbits, size=300)
    bf = b.reshape(-1)
    for i, k in zip(flips, bitsel):
        bf[i] ^= dtype(1 << int(k))
    b[3, 5] = a[3, 5] ^ dtype(1 << (nbits - 1))          # sign bit only (+0 / -0 style)
    tdt = torch.int16 if nbits == 16 else torch.int32
    sdt = np.int16 if nbits == 16 else np.int32
    A = torch.from_numpy(a.view(sdt)).to("cuda")
    B = torch.from_numpy(b.view(sdt)).to("cuda")
    c = bi.bi_row_bitdiff(A, B).cpu().numpy()
    for r in range(rows):
        assert tuple(c[r]) == oracle.bitdiff(a[r], b[r]), r
    # gathered rows in both operands
    ar = np.array([5, 0, 36, 3], np.int64)
    br = np.array([2, 0, 36, 9], np.int64)
    c = bi.bi_row_bitdiff(A, B, torch.from_numpy(ar).cuda(), torch.from_numpy(br).cuda())
    c = c.cpu().numpy()
    for i in range(4):
        assert tuple(c[i]) == oracle.bitdiff(a[ar[i]], b[br[i]])
    assert tdt is not None


def test_bitdiff_signed_zero_and_nan_payload(bi):
    a = np.array([[0x0000, 0x7FC0, 0x3F80, 0x1234] * 4], np.uint16)
    b = np.array([[0x8000, 0x7FC1, 0x3F80, 0x1234] * 4], np.uint16)
    A, B = (torch.from_numpy(v.view(np.int16)).cuda() for v in (a, b))
    c = bi.bi_row_bitdiff(A, B).cpu().numpy()
    assert tuple(c[0]) == oracle.bitdiff(a[0], b[0]) == (8, 8)


def test_bitdiff_batch_equals_single_calls(bi):
    """bi_row_bitdiff_batch over items of both element sizes, with and without
    row index vectors, strided and contiguous: every item's counts equal the
    oracle's, hence those of one bi_row_bitdiff call per item."""
    g = synth.rng(71)
    items, want = [], []
    for k, (nbits, rows, cols, gather) in enumerate(((16, 9, 256, False), (32, 5, 64, True),
                                                       (16, 40, 4096, True), (32, 1, 16, False),
                                                       (16, 3, 8, False))):
        dtype = np.uint16 if nbits == 16 else np.uint32
        sdt = np.int16 if nbits == 16 else np.int32
        a = g.integers(0, 1 << nbits, size=(rows, cols + 8), dtype=np.uint64).astype(dtype)
        b = a.copy()
        for i, kk in zip(g.integers(0, rows * (cols + 8), size=50), g.integers(0, nbits, size=50)):
            b.reshape(-1)[i] ^= dtype(1 << int(kk))
        A = torch.from_numpy(a.view(sdt)).cuda()[:, :cols]        # strided views (row stride cols + 8)
        B = torch.from_numpy(b.view(sdt)).cuda()[:, :cols]
        if gather:
            ar = g.permutation(rows)[: max(1, rows // 2)].astype(np.int64)
            br = ar[::-1].copy()
            items.append((A, B, torch.from_numpy(ar).cuda(), torch.from_numpy(br).cuda(), None))
            want.append([oracle.bitdiff(a[ar[i], :cols], b[br[i], :cols]) for i in range(len(ar))])
        else:
            items.append((A, B, None, None, None))
            want.append([oracle.bitdiff(a[r, :cols], b[r, :cols]) for r in range(rows)])
    outs = bi.bi_row_bitdiff_batch(items)
    for k, (c, w) in enumerate(zip(outs, want)):
        c = c.cpu().numpy()
        assert [tuple(x) for x in c] == w, k
        single = bi.bi_row_bitdiff(*items[k][:4]).cpu().numpy()
        assert np.array_equal(c, single), k


def test_llama70b_dynamic_batch_stream(bi):
    """200 batches, M ~ U{1..4096}; 8 fixed probe rows at random positions must
    equal their solo outputs bit for bit; sampled rows match the oracle."""
    c = workloads.LLAMA70B
    probes, batches = workloads.llama70b_stream()
    say("70b: generating inputs")
    xpool = workloads.llama70b_x_pool()
    w = workloads.llama70b_w()
    X, Wt = dev_bf16(xpool), dev_bf16(w)
    solo = torch.cat([bi.bi_gemm(X[int(p):int(p) + 1], Wt) for p in probes], dim=0)
    check_bf16(host_u16(solo), oracle.gemm(xpool[probes], w), "probe rows solo")
    y = torch.empty((c["m_max"], c["N"]), dtype=torch.bfloat16, device="cuda")
    tot_rows = tot_bits = 0
    ms = []
    for bno, b in enumerate(batches):
        idx = torch.from_numpy(b["rows"]).cuda()
        M = idx.numel()
        ms.append(M)
        xb = X.index_select(0, idx)
        bi.bi_gemm(xb, Wt, y=y[:M])
        present = [p for p in range(len(probes)) if b["probe_pos"][p] >= 0]
        pos = torch.tensor([int(b["probe_pos"][p]) for p in present], dtype=torch.int64).cuda()
        pid = torch.tensor(present, dtype=torch.int64).cuda()
        cnt = bi.bi_row_bitdiff(y, solo, pos, pid).sum(dim=0).tolist()
        tot_rows += len(present)
        tot_bits += int(cnt[0])
        if bno % 50 == 0:
            say(f"70b batch {bno}: M={M} probes={len(present)} bits={int(cnt[0])}")
            r = np.array(sorted({0, M - 1, M // 2}))
            check_bf16(host_u16(y[:M][torch.from_numpy(r).cuda()]), oracle.gemm(xpool[b["rows"][r]], w),
                       f"batch {bno}")
    say(f"70b: {len(batches)} batches, M in [{min(ms)}, {max(ms)}], {tot_rows} probe rows, "
        f"{tot_bits} differing bits")
    assert tot_rows >= 8 * 150 and tot_bits == 0
