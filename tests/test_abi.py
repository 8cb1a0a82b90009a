"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything.

Every call here fails validation (or has M == 0), so no kernel is launched and
no pointer is dereferenced: the fake device addresses are never touched.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")
LIB = os.path.join(ROOT, "invariant_deterministic_amd", "libbi.so")

BI_OK, BI_ERR_NULL, BI_ERR_SHAPE, BI_ERR_ALIGN, BI_ERR_WORKSPACE, BI_ERR_ALIAS, BI_ERR_HIP, \
    BI_ERR_UNSUPPORTED = range(8)

# fake, never-dereferenced, 16-byte aligned "device" addresses far apart
X, W, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text)))


class _Guarded:
    """Wraps the library so that no call made here can reach a kernel launch:
    a call must either fail validation or have an empty batch (M == 0)."""

    # position of the batch-size argument in each launching entry point
    M_ARG = {"bi_rmsnorm": 3, "bi_gemm": 3, "bi_gemm_with_config": 4, "bi_gemm_fill": 3,
             "bi_lora_shrink": 3,
             "bi_gemm_splitk": 3, "bi_gemm_splitk_noalloc": 3, "bi_gemm_mswitch_control": 3, "bi_decode_attention": 5, "bi_lora_expand": 4, "bi_lora_shrink_expand": 6,
             "bi_lora_shrink_two_pass": 3, "bi_lora_shrink_atomic": 3, "bi_row_bitdiff": 6}

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        f = getattr(self._lib, name)
        if name not in self.M_ARG:
            return f

        def call(*args):
            r = f(*args)
            assert r != BI_ERR_HIP, f"{name}{args} reached a launch"
            assert r != BI_OK or args[self.M_ARG[name]] == 0, f"{name}{args} would launch"
            return r
        return call


def _gpu_visible() -> bool:
    """True when a GPU is visible.  The validation calls below pass fake device
    addresses; they must never run where a regression in validation could turn
    one of them into a real launch.  (Counting devices initialises nothing.)"""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return os.path.exists("/dev/kfd")


@pytest.fixture(scope="module")
def rawlib():
    if not os.path.exists(LIB):
        pytest.skip("libbi.so not built")
    return _load()


@pytest.fixture(scope="module")
def lib(rawlib):
    if _gpu_visible():
        pytest.skip("argument-validation calls with fake addresses run only where no GPU is visible")
    return _Guarded(rawlib)


def _load():
    L = ctypes.CDLL(LIB)
    p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bi_rmsnorm.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_float, p]
    L.bi_gemm.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, p]
    L.bi_gemm_with_config.argtypes = [i, p, p, p, i64, i64, i64, i64, i64, i64, p]
    L.bi_gemm_fill.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, p]
    L.bi_gemm_fill_config_id.argtypes = [i64, i64, i64]
    L.bi_gemm_config_id.argtypes = [i64, i64]
    L.bi_gemm_splitk.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p, ctypes.c_size_t, p]
    L.bi_gemm_splitk_workspace_bytes.argtypes = [i64, i64, i]
    L.bi_gemm_splitk_workspace_bytes.restype = ctypes.c_size_t
    L.bi_gemm_splitk_for.argtypes = [i64, i64]
    L.bi_gemm_splitk_noalloc.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p]
    L.bi_gemm_mswitch_control.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, p, ctypes.c_size_t, p]
    L.bi_lora_shrink.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p, ctypes.c_size_t, p]
    L.bi_lora_shrink_two_pass.argtypes = L.bi_lora_shrink.argtypes
    L.bi_lora_shrink_atomic.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, i, p]
    L.bi_lora_shrink_workspace_bytes.argtypes = [i64, i64, i]
    L.bi_lora_shrink_workspace_bytes.restype = ctypes.c_size_t
    L.bi_row_bitdiff.argtypes = [p, i64, p, p, i64, p, i64, i64, i, p, p]
    L.bi_decode_attention.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i, p, ctypes.c_size_t, p]
    L.bi_decode_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i]
    L.bi_decode_attention_workspace_bytes.restype = ctypes.c_size_t
    L.bi_lora_expand.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, i64, ctypes.c_float, p]
    L.bi_lora_shrink_expand.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                        i64, ctypes.c_float, i, p]
    L.bi_status_str.restype = ctypes.c_char_p
    return L


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("bi_rmsnorm", "bi_gemm", "bi_gemm_config_id", "bi_lora_shrink",
              "bi_lora_shrink_workspace_bytes", "bi_lora_shrink_atomic", "bi_row_bitdiff",
              "bi_status_str", "bi_abi_version"):
        assert n in names


def test_every_declared_function_is_exported(rawlib):
    for n in declared_functions():
        assert hasattr(rawlib, n), f"{n} declared in bi.h but not exported"


def test_binding_exports_match_header():
    import invariant_deterministic_amd.binding as b
    assert sorted(b.EXPORTS) == declared_functions()
    for n in b.EXPORTS:
        assert callable(getattr(b, n))


def test_version_and_status_strings(rawlib):
    assert rawlib.bi_abi_version() == 1
    for s in range(8):
        assert rawlib.bi_status_str(s).decode().startswith("BI_")
    assert rawlib.bi_status_str(99) == b"unknown bi_status"


def test_rmsnorm_validation(lib):
    f = lib.bi_rmsnorm
    assert f(None, W, Y, 4, 4096, 4096, 4096, 1e-6, None) == BI_ERR_NULL
    assert f(X, W, Y, -1, 4096, 4096, 4096, 1e-6, None) == BI_ERR_SHAPE
    assert f(X, W, Y, 4, 4, 8, 8, 1e-6, None) == BI_ERR_SHAPE          # K < 8
    assert f(X, W, Y, 4, 16392, 16392, 16392, 1e-6, None) == BI_ERR_SHAPE  # K too big
    assert f(X, W, Y, 4, 4096, 4000, 4096, 1e-6, None) == BI_ERR_SHAPE  # ldx < K
    assert f(X, W, Y, 4, 4096, 4096, 4096, -1.0, None) == BI_ERR_SHAPE
    assert f(X, W, Y, 4, 4100, 4100, 4100, 1e-6, None) == BI_ERR_ALIGN  # K % 8
    assert f(X + 8, W, Y, 4, 4096, 4096, 4096, 1e-6, None) == BI_ERR_ALIGN
    assert f(X, W, X + 2 * 4096, 4, 4096, 4096, 4096, 1e-6, None) == BI_ERR_ALIAS
    assert f(X, Y, Y, 4, 4096, 4096, 4096, 1e-6, None) == BI_ERR_ALIAS   # w overlaps y
    assert f(X, W, Y, 0, 4096, 4096, 4096, 1e-6, None) == BI_OK          # M == 0: no launch
    assert f(X, W, X, 0, 4096, 4096, 4096, 1e-6, None) == BI_OK          # in place
    assert f(None, W, None, 0, 4096, 4096, 4096, 1e-6, None) == BI_OK    # empty batch
    assert f(None, None, None, 0, 4096, 4096, 4096, 1e-6, None) == BI_ERR_NULL


def test_gemm_validation(lib):
    f = lib.bi_gemm
    assert f(X, None, Y, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_NULL
    assert f(X, W, Y, 4, 4096, 4008, 4008, 4008, 4096, None) == BI_ERR_SHAPE   # K % 32
    assert f(X, W, Y, 1 << 20, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_SHAPE  # x > 2^31
    assert f(X, W, Y, 4, 4, 4096, 4096, 4096, 4, None) == BI_ERR_SHAPE         # N < 8
    assert f(X, W, Y, 4, 4096, 4096, 4096, 4096, 4095, None) == BI_ERR_SHAPE   # ldy < N
    assert f(X, W, Y, 4, 4100, 4096, 4096, 4096, 4100, None) == BI_ERR_ALIGN   # N % 8
    assert f(X, W, Y + 2, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_ALIGN
    assert f(X, W, X, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_ALIAS
    assert f(X, W, W + 64, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_ALIAS
    assert f(X, W, Y, 0, 4096, 4096, 4096, 4096, 4096, None) == BI_OK
    assert f(None, W, None, 0, 4096, 4096, 4096, 4096, 4096, None) == BI_OK
    assert f(None, None, None, 0, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_NULL
    assert lib.bi_gemm_with_config(99, X, W, Y, 0, 4096, 4096, 4096, 4096, 4096, None) == \
        BI_ERR_UNSUPPORTED
    assert lib.bi_gemm_with_config(0, X, W, Y, 0, 4096, 4096, 4096, 4096, 4096, None) == BI_OK


def test_gemm_fill_validation_and_choice(lib):
    f = lib.bi_gemm_fill
    assert f(X, None, Y, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_NULL
    assert f(X, W, Y, 4, 4096, 4008, 4008, 4008, 4096, None) == BI_ERR_SHAPE
    assert f(X, W, Y + 2, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_ALIGN
    assert f(X, W, X, 4, 4096, 4096, 4096, 4096, 4096, None) == BI_ERR_ALIAS
    assert f(X, W, Y, 0, 4096, 4096, 4096, 4096, 4096, None) == BI_OK
    c = lib.bi_gemm_fill_config_id
    assert c(0, 4096, 4096) == -1 and c(4, 4100, 4096) == -1 and c(4, 4096, 100) == -1
    # with 256 CUs (the count assumed when no device answers): the big tile
    # once it fills the chip, smaller ones below, and never an id outside
    # bi_gemm_with_config's range
    if c(4096, 4096, 4096) == 0:
        assert c(2048, 4096, 4096) == 3 and c(1000, 4096, 4096) == 2
        # 256 x 256 tiles with each XCD's tail of at most half a wave cut into
        # 256 x 128 halves (5): 896, 560, 272 and 2688 tiles leave 16, 6, 2 and
        # 16 on each XCD after its full waves
        assert c(4096, 14336, 4096) == 5 and c(2305, 14336, 4096) == 5
        assert c(4200, 4096, 4096) == 5 and c(6144, 28672, 8192) == 5
        # 128 x 64 tiles (4) only where 128 x 128 tiles fill at most half the
        # CUs and 128 x 64 tiles fill them in one wave
        assert c(2048, 1024, 4096) == 4 and c(1024, 1024, 4096) == 4
        assert c(512, 4096, 4096) == 4 and c(3072, 1024, 4096) == 2
        # never for more tiles than CUs: Up at M = 520 would need four waves
        assert c(520, 14336, 4096) == 0 and c(576, 14336, 4096) == 0
        # whole waves (1792 tiles) or a tail of more than half a wave (448
        # tiles: 24 per XCD): the big tile alone
        assert c(8192, 14336, 4096) == 0 and c(2048, 14336, 4096) == 0
        # 32-k stages: no mixed launch
        assert c(4096, 14336, 4064) == 0
        assert c(8192, 1024, 4096) == 3 and c(4096, 1024, 4096) == 2


def _params(name):
    """Parameter list of ``name`` as declared in bi.h, comments removed."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    return [" ".join(p.split()) for p in m.group(1).split(",")]


def test_config_functions_take_no_batch_size():
    """The static half of the contract: the functions that choose the GEMM's
    reduction (tile configuration, split of K) are declared with exactly
    (N, K) -- there is no M for them to read."""
    for name in ("bi_gemm_config_id", "bi_gemm_splitk_for"):
        assert _params(name) == ["int64_t N", "int64_t K"], (name, _params(name))


SHAPES = ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (28672, 8192), (1024, 1024),
          (1032, 1024), (4096, 96))
SWEEP = (1, 2, 3, 5, 16, 33, 64, 127, 128, 129, 255, 256, 257, 1000, 2039, 2048, 4093, 4096,
         8191, 8192, 65536)


def test_gemm_launch_plan_ignores_m(rawlib):
    """bi_gemm builds its launch from the host function bi_gemm_launch_plan
    reports: for each (N, K) the configuration, compiled kernel, tile, K stage
    and workgroup size are one and the same at every M, and M changes only the
    number of tile rows."""
    buf = (ctypes.c_int64 * 7)()
    ptr = ctypes.cast(buf, ctypes.c_void_p)
    rawlib.bi_gemm_launch_plan.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    for N, K in SHAPES:
        cfg = rawlib.bi_gemm_config_id(N, K)
        assert 0 <= cfg < rawlib.bi_gemm_num_configs()
        seen = set()
        for M in SWEEP + (0,):
            assert rawlib.bi_gemm_launch_plan(M, N, K, ptr) == BI_OK
            p = list(buf)
            assert p[0] == cfg and p[1] >= 0 and p[5] in (256, 512)
            assert p[4] == (64 if K % 64 == 0 else 32)
            tm, tn = p[2], p[3]
            assert p[6] == (-(-M // tm)) * (-(-N // tn)), (M, N, K, p)
            seen.add(tuple(p[:6]))
        assert len(seen) == 1, (N, K, seen)
    assert rawlib.bi_gemm_launch_plan(4, 4096, 100, ptr) == BI_ERR_SHAPE
    assert rawlib.bi_gemm_launch_plan(-1, 4096, 4096, ptr) == BI_ERR_SHAPE
    assert rawlib.bi_gemm_launch_plan(4, 4096, 4096, None) == BI_ERR_NULL
    assert rawlib.bi_gemm_config_id(4096, 100) == -1
    assert rawlib.bi_gemm_config_id(4100, 4096) == -1


def test_gemm_splitk_validation(lib):
    f = lib.bi_gemm_splitk
    need = lib.bi_gemm_splitk_workspace_bytes(4, 4096, 8)
    assert need == 8 * 4 * 4096 * 4
    a = (4, 4096, 4096, 4096, 4096, 4096)
    assert f(X, W, Y, *a, 8, None, need, None) == BI_ERR_NULL
    assert f(X, W, Y, *a, 8, WS, need - 1, None) == BI_ERR_WORKSPACE
    assert f(X, W, Y, *a, 0, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, *a, 65, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, 4, 4096, 4064, 4064, 4064, 4096, 8, WS, need, None) == BI_ERR_SHAPE  # K % (32*8)
    assert f(X, W, Y, *a, 8, Y + 64, need, None) == BI_ERR_ALIAS
    assert f(X, W, Y, *a, 8, WS + 8, need, None) == BI_ERR_ALIGN
    assert f(None, W, None, 0, 4096, 4096, 4096, 4096, 4096, 8, None, 0, None) == BI_OK
    for N, K in ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (28672, 8192)):
        s = lib.bi_gemm_splitk_for(N, K)
        assert s >= 1 and (s & (s - 1)) == 0 and K % (32 * s) == 0
    assert [lib.bi_gemm_splitk_for(N, K) for N, K in ((4096, 4096), (1024, 4096), (14336, 4096),
                                                      (4096, 14336), (28672, 8192))] == [8, 16, 4, 8, 2]
    h = lib.bi_gemm_splitk_noalloc
    assert h(X, None, Y, *a, 8, None) == BI_ERR_NULL
    assert h(X, W, Y, *a, 0, None) == BI_ERR_UNSUPPORTED
    assert h(X, W, Y, 4, 4096, 4064, 4064, 4064, 4096, 8, None) == BI_ERR_SHAPE
    assert h(X, W, X, *a, 8, None) == BI_ERR_ALIAS
    # 8 * 128 * 4096 * 4 = 16 MiB fits the static scratch; one more row does not
    assert lib.bi_gemm_splitk_workspace_bytes(129, 4096, 8) > 16 << 20
    assert h(X, W, Y, 129, 4096, 4096, 4096, 4096, 4096, 8, None) == BI_ERR_WORKSPACE
    assert h(None, W, None, 0, 4096, 4096, 4096, 4096, 4096, 8, None) == BI_OK
    g = lib.bi_gemm_mswitch_control
    assert g(X, W, Y, *a, None, need, None) == BI_ERR_NULL              # small M needs ws
    assert g(X, W, Y, 0, 4096, 4096, 4096, 4096, 4096, None, 0, None) == BI_OK


def test_shrink_validation(lib):
    f = lib.bi_lora_shrink
    need = lib.bi_lora_shrink_workspace_bytes(4096, 16, 8)
    assert need == 8 * 4096 * 16 * 4
    assert lib.bi_lora_shrink_workspace_bytes(4096, 16, 1) == 0
    assert lib.bi_lora_shrink_workspace_bytes(3, 16, 8) == 1536   # 8*3*16*4 rounded to 256
    args = (4096, 4096, 16, 4096, 4096, 16)
    assert lib.bi_lora_shrink_two_pass(X, W, Y, *args, 8, None, need, None) == BI_ERR_NULL
    assert lib.bi_lora_shrink_two_pass(X, W, Y, *args, 8, WS, need - 1, None) == BI_ERR_WORKSPACE
    assert lib.bi_lora_shrink_two_pass(X, W, Y, 0, 4096, 16, 4096, 4096, 16, 8, None, 0, None) == BI_OK
    assert f(X, W, Y, *args, 8, WS, need - 1, None) == BI_ERR_WORKSPACE
    assert f(X, W, Y, 4096, 4096, 8, 4096, 4096, 16, 8, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, *args, 3, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, 4096, 4000, 16, 4096, 4096, 16, 8, WS, need, None) == BI_ERR_SHAPE
    assert f(X, W, Y, 4096, 4096, 16, 4096, 4096, 15, 8, WS, need, None) == BI_ERR_SHAPE
    assert f(X, W, Y + 4, *args, 8, WS, need, None) == BI_ERR_ALIGN
    assert f(X, W, Y, *args, 8, Y + 64, need, None) == BI_ERR_ALIAS
    assert f(X, W, X, *args, 8, WS, need, None) == BI_ERR_ALIAS
    assert f(X, W, Y, 0, 4096, 16, 4096, 4096, 16, 8, WS, 0, None) == BI_OK
    assert f(X, W, Y, 0, 4096, 16, 4096, 4096, 16, 1, None, 0, None) == BI_OK
    assert f(None, W, None, 0, 4096, 16, 4096, 4096, 16, 8, None, 0, None) == BI_OK
    g = lib.bi_lora_shrink_atomic
    assert g(X, None, Y, *args, 8, None) == BI_ERR_NULL
    assert g(X, W, Y, *args, 5, None) == BI_ERR_UNSUPPORTED
    assert g(X, W, Y, 0, 4096, 16, 4096, 4096, 16, 8, None) == BI_OK


def test_bitdiff_validation(lib):
    f = lib.bi_row_bitdiff
    assert f(None, 8, None, Y, 8, None, 1, 8, 2, WS, None) == BI_ERR_NULL
    assert f(X, 8, None, Y, 8, None, 1, 8, 3, WS, None) == BI_ERR_UNSUPPORTED
    assert f(X, 4, None, Y, 8, None, 1, 8, 2, WS, None) == BI_ERR_SHAPE
    assert f(X + 1, 8, None, Y, 8, None, 1, 8, 2, WS, None) == BI_ERR_ALIGN
    assert f(X, 8, None, Y, 8, None, 0, 8, 2, WS, None) == BI_OK


class _Item(ctypes.Structure):
    # bi_bitdiff_item as include/bi.h lays it out: ten 8-byte fields
    _fields_ = [("a", ctypes.c_void_p), ("lda", ctypes.c_int64), ("a_rows", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("b_rows", ctypes.c_void_p),
                ("nrows", ctypes.c_int64), ("ncols", ctypes.c_int64), ("elem_bytes", ctypes.c_int64),
                ("counts", ctypes.c_void_p)]


def test_bitdiff_batch_validation(rawlib):
    """Every rejected call is rejected before a launch; an all-empty batch
    returns BI_OK without one."""
    if _gpu_visible():
        pytest.skip("validation with fake addresses runs only where no GPU is visible")
    assert ctypes.sizeof(_Item) == 80
    f = rawlib.bi_row_bitdiff_batch
    f.argtypes = [ctypes.POINTER(_Item), ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def call(items, n=None):
        arr = (_Item * max(1, len(items)))(*items)
        r = f(arr, len(items) if n is None else n, None)
        assert r != BI_ERR_HIP
        return r

    good = _Item(X, 64, None, Y, 64, None, 3, 64, 2, WS)
    assert f(None, 1, None) == BI_ERR_NULL
    assert call([good], n=0) == BI_ERR_UNSUPPORTED
    assert call([good] * 17) == BI_ERR_UNSUPPORTED
    assert call([good, _Item(None, 64, None, Y, 64, None, 3, 64, 2, WS)]) == BI_ERR_NULL
    assert call([good, _Item(X, 64, None, Y, 64, None, 3, 64, 2, None)]) == BI_ERR_NULL
    assert call([_Item(X, 64, None, Y, 64, None, 3, 64, 8, WS), good]) == BI_ERR_UNSUPPORTED
    assert call([good, _Item(X, 32, None, Y, 64, None, 3, 64, 2, WS)]) == BI_ERR_SHAPE
    assert call([good, _Item(X, 64, None, Y, 64, None, -1, 64, 2, WS)]) == BI_ERR_SHAPE
    assert call([good, _Item(X + 8, 64, None, Y, 64, None, 3, 64, 2, WS)]) == BI_ERR_ALIGN
    assert call([good, _Item(X, 68, None, Y, 68, None, 3, 68, 2, WS)]) == BI_ERR_ALIGN  # 136-byte rows
    assert call([good, _Item(X, 64, None, Y, 64, None, 3, 64, 2, WS + 4)]) == BI_ERR_ALIGN
    empty = _Item(X, 64, None, Y, 64, None, 0, 64, 4, WS)
    assert call([empty, empty]) == BI_OK


def test_decode_attention_validation(lib):
    f = lib.bi_decode_attention
    need = lib.bi_decode_attention_workspace_bytes(2, 32, 1000, 128, 256)
    assert need == (2 * 32 * 4 * 130 * 4 + 255) // 256 * 256
    L = WS + (1 << 24)
    a = (2, 32, 8, 128, 1000)
    assert f(X, W, Y, L, None, *a, 256, WS, need, None) == BI_ERR_NULL
    assert f(X, W, Y, L, X + (1 << 26), 2, 32, 8, 96, 1000, 256, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, L, X + (1 << 26), 2, 32, 3, 128, 1000, 256, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, L, X + (1 << 26), 2, 32, 2, 128, 1000, 256, WS, need, None) == BI_ERR_UNSUPPORTED  # G=16
    assert f(X, W, Y, L, X + (1 << 26), *a, 100, WS, need, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, Y, L + 2, X + (1 << 26), *a, 256, WS, need, None) == BI_ERR_ALIGN
    assert f(X, W, Y, L, X + (1 << 26), *a, 256, WS, need - 1, None) == BI_ERR_WORKSPACE
    assert f(X, W, Y, L, X, *a, 256, WS, need, None) == BI_ERR_ALIAS
    assert f(None, None, None, None, None, 0, 32, 8, 128, 1000, 256, None, 0, None) == BI_OK


def test_lora_expand_validation(lib):
    f = lib.bi_lora_expand
    assert f(X, None, None, Y, 4, 4096, 16, 16, 16, 0, 4096, 1.0, None) == BI_ERR_NULL
    assert f(X, W, None, Y, 4, 4096, 8, 16, 16, 0, 4096, 1.0, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, None, Y, 4, 4100, 16, 16, 16, 0, 4100, 1.0, None) == BI_ERR_ALIGN
    assert f(X, W + 2, None, Y, 4, 4096, 16, 16, 16, 0, 4096, 1.0, None) == BI_ERR_ALIGN  # b
    assert f(X, W, None, Y, 4, 4096, 16, 16, 20, 0, 4096, 1.0, None) == BI_ERR_ALIGN     # ldb
    assert f(X, W, WS, Y, 4, 4096, 16, 16, 16, 4000, 4096, 1.0, None) == BI_ERR_SHAPE
    assert f(X, W, Y + 16, Y, 4, 4096, 16, 16, 16, 4096, 4096, 1.0, None) == BI_ERR_ALIAS
    assert f(X, W, None, X, 4, 4096, 16, 16, 16, 0, 4096, 1.0, None) == BI_ERR_ALIAS
    assert f(None, W, None, None, 0, 4096, 16, 16, 16, 0, 4096, 1.0, None) == BI_OK


def test_shrink_expand_validation(lib):
    f = lib.bi_lora_shrink_expand
    B, BASE, L = 0x50000000, 0x60000000, 0x70000000
    ok = (4096, 4096, 4096, 16, 4096, 4096, 16, 4096, 4096, 16)   # M K N R ldx lda ldb ldbase ldy ldl
    assert f(X, W, None, BASE, Y, L, *ok, 1.0, 8, None) == BI_ERR_NULL
    assert f(X, W, B, BASE, Y, L, 4096, 4096, 4096, 8, 4096, 4096, 16, 4096, 4096, 16, 1.0, 8,
             None) == BI_ERR_UNSUPPORTED                                            # R != 16
    assert f(X, W, B, BASE, Y, L, *ok, 1.0, 16, None) == BI_ERR_UNSUPPORTED          # split 16
    assert f(X, W, B, BASE, Y, L, *ok, 1.0, 3, None) == BI_ERR_UNSUPPORTED
    assert f(X, W, B, BASE, Y, L, 4096, 4064, 4096, 16, 4096, 4096, 16, 4096, 4096, 16, 1.0, 8,
             None) == BI_ERR_SHAPE                                                  # K % 256
    assert f(X, W, B, BASE, Y, L, 4096, 4096, 4100, 16, 4096, 4096, 16, 4100, 4100, 16, 1.0, 8,
             None) == BI_ERR_ALIGN                                                  # N % 8
    assert f(X, W, B, BASE, Y, L + 4, *ok, 1.0, 8, None) == BI_ERR_ALIGN
    assert f(X, W, B, BASE, X, L, *ok, 1.0, 8, None) == BI_ERR_ALIAS                 # y over x
    assert f(X, W, B, BASE, Y, Y, *ok, 1.0, 8, None) == BI_ERR_ALIAS                 # l over y
    assert f(X, W, B, Y, Y, L, 0, *ok[1:], 1.0, 8, None) == BI_OK                   # in place
    assert f(X, W, B, Y + 64, Y, L, 4096, *ok[1:], 1.0, 8, None) == BI_ERR_ALIAS     # base shifted onto y
    assert f(None, W, B, None, None, None, 0, 4096, 4096, 16, 4096, 4096, 16, 4096, 4096, 16, 1.0,
             8, None) == BI_OK
