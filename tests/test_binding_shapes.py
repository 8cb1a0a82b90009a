"""The Python binding checks every tensor's shape before anything reaches the
library: the C ABI receives only pointers and strides, so an output with too
few rows or a weight with the wrong K would otherwise be written or read out of
bounds on the device.  These run on the CPU: shapes are checked before the
device check, so a wrong shape raises a shape error, and right shapes on host
tensors raise the device error -- neither reaches a launch."""
from __future__ import annotations

import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "invariant_deterministic_amd", "libbi.so")


@pytest.fixture(scope="module")
def bi():
    if not os.path.exists(LIB):
        pytest.skip("libbi.so not built")
    from invariant_deterministic_amd import binding
    return binding


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def shape_error(fn, *args, **kw):
    with pytest.raises(ValueError) as e:
        fn(*args, **kw)
    assert "device" not in str(e.value), str(e.value)
    return str(e.value)


def device_error(fn, *args, **kw):
    with pytest.raises(ValueError, match="device"):
        fn(*args, **kw)


def test_gemm_family_shapes(bi):
    x, w = bf(5, 64), bf(32, 64)
    for fn in (bi.bi_gemm, bi.bi_gemm_fill,
               lambda *a, **k: bi.bi_gemm_with_config(0, *a, **k),
               lambda *a, **k: bi.bi_gemm_splitk(*a, split_k=2, **k),
               bi.bi_gemm_mswitch_control):
        shape_error(fn, x, bf(32, 96))             # w has another K
        shape_error(fn, x, w, y=bf(4, 32))          # y has too few rows
        shape_error(fn, x, w, y=bf(5, 24))          # y has too few columns
        shape_error(fn, x, bf(32, 64, 1))           # w not 2-D
        device_error(fn, x, w)                      # right shapes, host tensors
        device_error(fn, x, w, y=bf(5, 32))


def test_shrink_family_shapes(bi):
    x, a = bf(7, 256), bf(16, 256)
    for fn in (bi.bi_lora_shrink, bi.bi_lora_shrink_two_pass, bi.bi_lora_shrink_atomic):
        shape_error(fn, x, bf(16, 512))             # a has another K
        shape_error(fn, x, a, y=f32(6, 16))         # y has too few rows
        shape_error(fn, x, a, y=f32(7, 8))          # y has too few ranks
        device_error(fn, x, a)
        device_error(fn, x, a, y=f32(7, 16))


def test_expand_and_pair_shapes(bi):
    l, b = f32(9, 16), bf(64, 16)
    shape_error(bi.bi_lora_expand, l, bf(64, 8))              # b has another R
    shape_error(bi.bi_lora_expand, l, b, base=bf(8, 64))      # base too short
    shape_error(bi.bi_lora_expand, l, b, y=bf(9, 56))         # y too narrow
    device_error(bi.bi_lora_expand, l, b)
    x, a = bf(9, 256), bf(16, 256)
    shape_error(bi.bi_lora_shrink_expand, x, bf(16, 128), b)  # a has another K
    shape_error(bi.bi_lora_shrink_expand, x, a, bf(64, 8))    # b has another R
    shape_error(bi.bi_lora_shrink_expand, x, a, b, y=bf(8, 64))
    shape_error(bi.bi_lora_shrink_expand, x, a, b, base=bf(9, 32))
    shape_error(bi.bi_lora_shrink_expand, x, a, b, l=f32(8, 16))
    device_error(bi.bi_lora_shrink_expand, x, a, b)


def test_rmsnorm_attention_bitdiff_shapes(bi):
    x = bf(3, 64)
    shape_error(bi.bi_rmsnorm, x, bf(32))                     # weight of another K
    shape_error(bi.bi_rmsnorm, x, bf(64), y=bf(2, 64))
    device_error(bi.bi_rmsnorm, x, bf(64))
    q, kc = bf(2, 8, 64), bf(2, 128, 2, 64)
    lens = torch.ones(2, dtype=torch.int32)
    shape_error(bi.bi_decode_attention, q, kc, bf(2, 128, 2, 32), lens)
    shape_error(bi.bi_decode_attention, q, kc, kc, torch.ones(3, dtype=torch.int32))
    shape_error(bi.bi_decode_attention, q, kc, kc, lens, o=bf(2, 8, 32))
    device_error(bi.bi_decode_attention, q, kc, kc, lens)
    a, b2 = bf(4, 16), bf(4, 16)
    shape_error(bi.bi_row_bitdiff, a, b2, counts=torch.zeros((3, 2), dtype=torch.int64))
    device_error(bi.bi_row_bitdiff, a, b2, counts=torch.zeros((4, 2), dtype=torch.int64))
