"""Thin ctypes binding of libbi.so with the C ABI's own names.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libbi.so``.  Tensors are torch CUDA (ROCm) tensors -- torch
supplies device memory and the current stream, nothing else.  bf16 operands
may be given as ``torch.bfloat16`` or as 16-bit integer views of the same bits.

There is no fallback: importing this module raises if ``libbi.so`` has not
been built (``python -m invariant_deterministic_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbi.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python -m invariant_deterministic_amd.build); there is no CPU fallback")

_lib = ctypes.CDLL(_LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _sig(name, argtypes, restype=_int):
    f = getattr(_lib, name)
    f.argtypes = argtypes
    f.restype = restype
    return f


_lib_abi_version = _sig("bi_abi_version", [])
_lib_status_str = _sig("bi_status_str", [_int], ctypes.c_char_p)
_lib_rmsnorm = _sig("bi_rmsnorm", [_p, _p, _p, _i64, _i64, _i64, _i64, ctypes.c_float, _p])
_lib_gemm = _sig("bi_gemm", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p])
_lib_gemm_config_id = _sig("bi_gemm_config_id", [_i64, _i64])
_lib_gemm_num_configs = _sig("bi_gemm_num_configs", [])
_lib_gemm_launch_plan = _sig("bi_gemm_launch_plan", [_i64, _i64, _i64, _p])
_lib_gemm_fill = _sig("bi_gemm_fill", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p])
_lib_gemm_fill_config_id = _sig("bi_gemm_fill_config_id", [_i64, _i64, _i64])
_lib_gemm_with_config = _sig("bi_gemm_with_config",
                             [_int, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p])
_lib_gemm_splitk = _sig("bi_gemm_splitk", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _int, _p,
                                           ctypes.c_size_t, _p])
_lib_gemm_splitk_noalloc = _sig("bi_gemm_splitk_noalloc", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                                                           _i64, _int, _p])
_lib_gemm_splitk_ws = _sig("bi_gemm_splitk_workspace_bytes", [_i64, _i64, _int], ctypes.c_size_t)
_lib_gemm_splitk_for = _sig("bi_gemm_splitk_for", [_i64, _i64])
_lib_gemm_mswitch = _sig("bi_gemm_mswitch_control", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                                     _p, ctypes.c_size_t, _p])
_lib_attn = _sig("bi_decode_attention", [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _int, _p,
                                         ctypes.c_size_t, _p])
_lib_attn_ws = _sig("bi_decode_attention_workspace_bytes", [_i64, _i64, _i64, _i64, _int],
                    ctypes.c_size_t)
_lib_shrink_expand = _sig("bi_lora_shrink_expand",
                         [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                          _i64, _i64, ctypes.c_float, _int, _p])
_lib_expand = _sig("bi_lora_expand", [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      ctypes.c_float, _p])
_lib_ws_bytes = _sig("bi_lora_shrink_workspace_bytes", [_i64, _i64, _int], ctypes.c_size_t)
_lib_shrink = _sig("bi_lora_shrink", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                                      _p, ctypes.c_size_t, _p])
_lib_shrink_two_pass = _sig("bi_lora_shrink_two_pass", [_p, _p, _p, _i64, _i64, _i64, _i64, _i64,
                                                        _i64, _int, _p, ctypes.c_size_t, _p])
_lib_shrink_atomic = _sig("bi_lora_shrink_atomic",
                          [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _int, _p])
_lib_row_bitdiff = _sig("bi_row_bitdiff", [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _int, _p, _p])


class BitdiffItem(ctypes.Structure):
    """bi_bitdiff_item (include/bi.h): all fields 8 bytes wide."""
    _fields_ = [("a", _p), ("lda", _i64), ("a_rows", _p), ("b", _p), ("ldb", _i64),
                ("b_rows", _p), ("nrows", _i64), ("ncols", _i64), ("elem_bytes", _i64),
                ("counts", _p)]


BITDIFF_BATCH_MAX = 16   # BI_BITDIFF_BATCH_MAX
_lib_row_bitdiff_batch = _sig("bi_row_bitdiff_batch", [ctypes.POINTER(BitdiffItem), _int, _p])

BI_OK = 0
EXPORTS = ("bi_abi_version", "bi_status_str", "bi_rmsnorm", "bi_gemm", "bi_gemm_config_id",
           "bi_gemm_num_configs", "bi_gemm_with_config", "bi_gemm_launch_plan", "bi_gemm_fill", "bi_gemm_fill_config_id",
           "bi_gemm_splitk",
           "bi_gemm_splitk_workspace_bytes", "bi_gemm_splitk_for", "bi_gemm_splitk_noalloc", "bi_gemm_mswitch_control", "bi_lora_shrink_workspace_bytes",
           "bi_lora_shrink", "bi_lora_shrink_two_pass", "bi_lora_shrink_atomic", "bi_row_bitdiff",
           "bi_row_bitdiff_batch",
           "bi_decode_attention", "bi_decode_attention_workspace_bytes", "bi_lora_expand",
           "bi_lora_shrink_expand")


class BiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bi_status_str(status)}")


def library_path() -> str:
    return _LIB_PATH


def raw() -> ctypes.CDLL:
    """The loaded library, for ABI-level tests."""
    return _lib


def _check(st: int, where: str):
    if st != BI_OK:
        raise BiError(st, where)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _dims(t, name: str, ndim: int = 2) -> tuple:
    """Shape of ``t`` after checking it is a torch tensor of ``ndim`` dimensions.
    Shapes are checked before anything about the device, so a wrong shape is
    reported the same way with or without a GPU, and before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _want(t, shape: tuple, name: str):
    """Raise unless tensor ``t`` has exactly ``shape``."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _mat(t: torch.Tensor, name: str, dtypes) -> tuple[int, int]:
    """Validate a row-major device matrix; return (data_ptr, row stride)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() == 1:
        return t.data_ptr(), t.shape[0]
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.data_ptr(), t.stride(0)


def bi_abi_version() -> int:
    return int(_lib_abi_version())


def bi_status_str(status: int) -> str:
    return _lib_status_str(int(status)).decode()


def bi_rmsnorm(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
               eps: float = 1e-6, stream=None) -> torch.Tensor:
    """y = RMSNorm(x) * w, one workgroup per row (see bi.h)."""
    M, K = _dims(x, "x")
    _want(w, (K,), "w")
    if y is not None:
        _want(y, (M, K), "y")
    else:
        y = torch.empty((M, K), dtype=x.dtype, device=x.device)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, _ = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    _check(_lib_rmsnorm(px, pw, py, M, K, ldx, ldy, float(eps), _stream(stream)), "bi_rmsnorm")
    return y


def _gemm_shapes(x, w, y):
    """(M, N, K, y) for x [M, K] . w [N, K]^T, allocating y [M, N] if None."""
    M, K = _dims(x, "x")
    N, Kw = _dims(w, "w")
    if Kw != K:
        raise ValueError(f"x has K = {K} columns but w has {Kw}")
    if y is not None:
        _want(y, (M, N), "y")
    else:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    return M, N, K, y


def bi_gemm(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """y[M, N] = x[M, K] . w[N, K]^T in bf16 with fp32 accumulation (see bi.h)."""
    M, N, K, y = _gemm_shapes(x, w, y)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, ldw = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    _check(_lib_gemm(px, pw, py, M, N, K, ldx, ldw, ldy, _stream(stream)), "bi_gemm")
    return y


def bi_gemm_config_id(N: int, K: int) -> int:
    return int(_lib_gemm_config_id(N, K))


def bi_gemm_num_configs() -> int:
    return int(_lib_gemm_num_configs())


PLAN_FIELDS = ("config", "kernel", "tile_m", "tile_n", "k_stage", "threads", "workgroups")


def bi_gemm_launch_plan(M: int, N: int, K: int) -> dict:
    """What bi_gemm(M, N, K) would launch (host only; see bi.h)."""
    buf = (ctypes.c_int64 * len(PLAN_FIELDS))()
    _check(_lib_gemm_launch_plan(M, N, K, ctypes.cast(buf, _p)), "bi_gemm_launch_plan")
    return dict(zip(PLAN_FIELDS, (int(v) for v in buf)))


def bi_gemm_with_config(config: int, x: torch.Tensor, w: torch.Tensor,
                        y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M, N, K, y = _gemm_shapes(x, w, y)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, ldw = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    _check(_lib_gemm_with_config(config, px, pw, py, M, N, K, ldx, ldw, ldy, _stream(stream)),
           "bi_gemm_with_config")
    return y


def bi_gemm_fill(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """bi_gemm with the tile picked per call to fill the chip; same bits (see bi.h)."""
    M, N, K, y = _gemm_shapes(x, w, y)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, ldw = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    _check(_lib_gemm_fill(px, pw, py, M, N, K, ldx, ldw, ldy, _stream(stream)), "bi_gemm_fill")
    return y


def bi_gemm_fill_config_id(M: int, N: int, K: int) -> int:
    return int(_lib_gemm_fill_config_id(M, N, K))


def bi_gemm_splitk_workspace_bytes(M: int, N: int, split_k: int) -> int:
    return int(_lib_gemm_splitk_ws(M, N, split_k))


def bi_gemm_splitk_for(N: int, K: int) -> int:
    return int(_lib_gemm_splitk_for(N, K))


def _gemm_ws_call(fn, name, x, w, y, split_k, ws, stream):
    M, N, K, y = _gemm_shapes(x, w, y)
    if ws is not None and not isinstance(ws, torch.Tensor):
        raise TypeError("ws must be a torch.Tensor")
    if ws is None:
        need = bi_gemm_splitk_workspace_bytes(M, N, split_k if split_k else
                                              max(1, bi_gemm_splitk_for(N, K)))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, ldw = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    args = [px, pw, py, M, N, K, ldx, ldw, ldy]
    if split_k:
        args.append(split_k)
    _check(fn(*args, ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)), name)
    return y


def bi_gemm_splitk(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
                   split_k: int | None = None, ws: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Split-K GEMM with a fixed split (default bi_gemm_splitk_for(N, K)) and a
    fixed-order fp32 combine (see bi.h)."""
    if split_k is None:
        split_k = bi_gemm_splitk_for(w.shape[0], w.shape[1])
    return _gemm_ws_call(_lib_gemm_splitk, "bi_gemm_splitk", x, w, y, split_k, ws, stream)


GEMM_SPLITK_SCRATCH_BYTES = 16 << 20   # BI_GEMM_SPLITK_SCRATCH_BYTES


def bi_gemm_splitk_noalloc(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
                           split_k: int | None = None, stream=None) -> torch.Tensor:
    """bi_gemm_splitk with the partials in the library's static scratch: the
    call allocates nothing (see bi.h).  Pass ``y`` to keep the wrapper itself
    allocation-free too."""
    M, N, K, y = _gemm_shapes(x, w, y)
    if split_k is None:
        split_k = bi_gemm_splitk_for(N, K)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pw, ldw = _mat(w, "w", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    _check(_lib_gemm_splitk_noalloc(px, pw, py, M, N, K, ldx, ldw, ldy, split_k, _stream(stream)),
           "bi_gemm_splitk_noalloc")
    return y


def bi_gemm_mswitch_control(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """CONTROL ONLY: chooses split-K from M (not batch-invariant)."""
    return _gemm_ws_call(_lib_gemm_mswitch, "bi_gemm_mswitch_control", x, w, y, 0, ws, stream)


def bi_lora_shrink_workspace_bytes(M: int, R: int, split_k: int) -> int:
    return int(_lib_ws_bytes(M, R, split_k))


def bi_lora_shrink(x: torch.Tensor, a: torch.Tensor, y: torch.Tensor | None = None,
                   split_k: int = 8, ws: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Deterministic split-K LoRA shrink y[M, R] = x . a^T in fp32, one kernel
    (see bi.h); ``ws`` is optional and, when given, receives the partials."""
    return _shrink(_lib_shrink, "bi_lora_shrink", x, a, y, split_k, ws, stream, False)


def bi_lora_shrink_two_pass(x: torch.Tensor, a: torch.Tensor, y: torch.Tensor | None = None,
                            split_k: int = 8, ws: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Same bits as bi_lora_shrink, via an HBM workspace and a second kernel."""
    return _shrink(_lib_shrink_two_pass, "bi_lora_shrink_two_pass", x, a, y, split_k, ws, stream,
                   True)


def _shrink_shapes(x, a, y):
    """(M, K, R, y) for x [M, K] . a [R, K]^T, allocating y [M, R] fp32 if None."""
    M, K = _dims(x, "x")
    R, Ka = _dims(a, "a")
    if Ka != K:
        raise ValueError(f"x has K = {K} columns but a has {Ka}")
    if y is not None:
        _want(y, (M, R), "y")
    else:
        y = torch.empty((M, R), dtype=torch.float32, device=x.device)
    return M, K, R, y


def _shrink(fn, name, x, a, y, split_k, ws, stream, need_ws):
    M, K, R, y = _shrink_shapes(x, a, y)
    if ws is not None and not isinstance(ws, torch.Tensor):
        raise TypeError("ws must be a torch.Tensor")
    need = bi_lora_shrink_workspace_bytes(M, R, split_k)
    if ws is None and need > 0 and need_ws:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pa, lda = _mat(a, "a", _BF16_LIKE)
    py, ldy = _mat(y, "y", (torch.float32,))
    pws = ws.data_ptr() if ws is not None else None
    nws = ws.numel() * ws.element_size() if ws is not None else 0
    _check(fn(px, pa, py, M, K, R, ldx, lda, ldy, split_k, pws, nws, _stream(stream)), name)
    return y


def bi_lora_shrink_atomic(x: torch.Tensor, a: torch.Tensor, y: torch.Tensor | None = None,
                          split_k: int = 8, stream=None) -> torch.Tensor:
    """CONTROL ONLY: split-K shrink combined with fp32 atomics (nondeterministic)."""
    M, K, R, y = _shrink_shapes(x, a, y)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pa, lda = _mat(a, "a", _BF16_LIKE)
    py, ldy = _mat(y, "y", (torch.float32,))
    _check(_lib_shrink_atomic(px, pa, py, M, K, R, ldx, lda, ldy, split_k, _stream(stream)),
           "bi_lora_shrink_atomic")
    return y


def bi_row_bitdiff(a: torch.Tensor, b: torch.Tensor, a_rows: torch.Tensor | None = None,
                   b_rows: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                   stream=None, check_rows: bool = True) -> torch.Tensor:
    """Per row pair: [differing bits, differing elements] (int64 [nrows, 2]).

    ``check_rows`` verifies the index vectors on the host first (a device
    synchronisation); pass False only for indices already known to be valid."""
    if a.element_size() != b.element_size() or a.element_size() not in (2, 4):
        raise TypeError("a and b need the same 2- or 4-byte element size")
    ncols = a.shape[1]
    if b.shape[1] != ncols:
        raise ValueError("a and b disagree on the number of columns")
    nrows = a_rows.numel() if a_rows is not None else (
        b_rows.numel() if b_rows is not None else a.shape[0])
    for rows, name in ((a_rows, "a_rows"), (b_rows, "b_rows")):
        if rows is not None and (rows.dtype != torch.int64 or not rows.is_cuda
                                 or rows.numel() != nrows):
            raise ValueError(f"{name} must be a device int64 vector of {nrows} indices")
    if check_rows and a_rows is not None and nrows and not (0 <= int(a_rows.min()) and int(a_rows.max()) < a.shape[0]):
        raise IndexError("a_rows out of range")
    if check_rows and b_rows is not None and nrows and not (0 <= int(b_rows.min()) and int(b_rows.max()) < b.shape[0]):
        raise IndexError("b_rows out of range")
    if a_rows is None and nrows > a.shape[0] or b_rows is None and nrows > b.shape[0]:
        raise IndexError("more rows compared than present")
    if counts is None:
        counts = torch.empty((nrows, 2), dtype=torch.int64, device=a.device)
    else:
        _want(counts, (nrows, 2), "counts")
        if counts.dtype != torch.int64 or not counts.is_contiguous():
            raise ValueError("counts must be a contiguous int64 [nrows, 2] tensor")
    pa, lda = _mat(a, "a", (a.dtype,))
    pb, ldb = _mat(b, "b", (b.dtype,))
    _check(_lib_row_bitdiff(pa, lda, a_rows.data_ptr() if a_rows is not None else None,
                            pb, ldb, b_rows.data_ptr() if b_rows is not None else None,
                            nrows, ncols, a.element_size(), counts.data_ptr(), _stream(stream)),
           "bi_row_bitdiff")
    return counts


def bi_row_bitdiff_batch(items, stream=None, check_rows: bool = True) -> list:
    """Several bi_row_bitdiff comparisons in one launch.  ``items``: a sequence
    of (a, b, a_rows, b_rows, counts) with the arguments of bi_row_bitdiff
    (counts may be None).  Returns the counts tensors, one per item."""
    items = list(items)
    if not 1 <= len(items) <= BITDIFF_BATCH_MAX:
        raise ValueError(f"1 to {BITDIFF_BATCH_MAX} items")
    arr = (BitdiffItem * len(items))()
    outs = []
    for k, (a, b, a_rows, b_rows, counts) in enumerate(items):
        if a.element_size() != b.element_size() or a.element_size() not in (2, 4):
            raise TypeError("a and b need the same 2- or 4-byte element size")
        ncols = a.shape[1]
        if b.shape[1] != ncols:
            raise ValueError("a and b disagree on the number of columns")
        nrows = a_rows.numel() if a_rows is not None else (
            b_rows.numel() if b_rows is not None else a.shape[0])
        for rows, name, t in ((a_rows, "a_rows", a), (b_rows, "b_rows", b)):
            if rows is None:
                if nrows > t.shape[0]:
                    raise IndexError("more rows compared than present")
                continue
            if rows.dtype != torch.int64 or not rows.is_cuda or rows.numel() != nrows:
                raise ValueError(f"{name} must be a device int64 vector of {nrows} indices")
            if check_rows and nrows and not (0 <= int(rows.min()) and int(rows.max()) < t.shape[0]):
                raise IndexError(f"{name} out of range")
        if counts is None:
            counts = torch.empty((nrows, 2), dtype=torch.int64, device=a.device)
        else:
            _want(counts, (nrows, 2), "counts")
            if counts.dtype != torch.int64 or not counts.is_contiguous():
                raise ValueError("counts must be a contiguous int64 [nrows, 2] tensor")
        pa, lda = _mat(a, "a", (a.dtype,))
        pb, ldb = _mat(b, "b", (b.dtype,))
        arr[k] = BitdiffItem(pa, lda, a_rows.data_ptr() if a_rows is not None else None, pb, ldb,
                             b_rows.data_ptr() if b_rows is not None else None, nrows, ncols,
                             a.element_size(), counts.data_ptr())
        outs.append(counts)
    _check(_lib_row_bitdiff_batch(arr, len(items), _stream(stream)), "bi_row_bitdiff_batch")
    return outs


def bi_decode_attention_workspace_bytes(B: int, H: int, Tmax: int, D: int, split_size: int) -> int:
    return int(_lib_attn_ws(B, H, Tmax, D, split_size))


def bi_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        lens: torch.Tensor, o: torch.Tensor | None = None, split_size: int = 256,
                        ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Batch-invariant decode attention (see bi.h).  q [B, H, D]; caches
    [B, Tmax, Hkv, D]; lens int32 [B] on the device."""
    B, H, D = _dims(q, "q", 3)
    Bk, Tmax, Hkv, Dk = _dims(k_cache, "k_cache", 4)
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Bk != B or Dk != D:
        raise ValueError("cache shapes do not match q")
    _want(lens, (B,), "lens")
    if o is not None:
        _want(o, (B, H, D), "o")
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_cuda or t.dtype not in _BF16_LIKE or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    if lens.dtype != torch.int32 or not lens.is_cuda or tuple(lens.shape) != (B,):
        raise ValueError("lens must be a device int32 vector of B lengths")
    if o is None:
        o = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    if not o.is_contiguous() or tuple(o.shape) != (B, H, D):
        raise ValueError("o must be a contiguous [B, H, D] tensor")
    need = bi_decode_attention_workspace_bytes(B, H, Tmax, D, split_size)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(_lib_attn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(),
                     o.data_ptr(), B, H, Hkv, D, Tmax, split_size, ws.data_ptr(),
                     ws.numel() * ws.element_size(), _stream(stream)), "bi_decode_attention")
    return o


def bi_lora_expand(l: torch.Tensor, b: torch.Tensor, base: torch.Tensor | None = None,
                   y: torch.Tensor | None = None, scale: float = 1.0,
                   stream=None) -> torch.Tensor:
    """y = bf16(base + scale * l . b^T), l fp32 [M, R], b bf16 [N, R] (see bi.h)."""
    M, R = _dims(l, "l")
    N, Rb = _dims(b, "b")
    if Rb != R:
        raise ValueError(f"l has R = {R} columns but b has {Rb}")
    if base is not None:
        _want(base, (M, N), "base")
    if y is not None:
        _want(y, (M, N), "y")
    else:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=l.device)
    pl, ldl = _mat(l, "l", (torch.float32,))
    pb, ldb = _mat(b, "b", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    pbase, ldbase = (None, 0) if base is None else _mat(base, "base", _BF16_LIKE)
    _check(_lib_expand(pl, pb, pbase, py, M, N, R, ldl, ldb, ldbase, ldy, float(scale),
                       _stream(stream)), "bi_lora_expand")
    return y


def bi_lora_shrink_expand(x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                          base: torch.Tensor | None = None, y: torch.Tensor | None = None,
                          l: torch.Tensor | None = None, scale: float = 1.0, split_k: int = 8,
                          stream=None) -> torch.Tensor:
    """y = bf16(base + scale * shrink(x, a) . b^T) in one launch (see bi.h); l, if
    given (fp32 [M, R]), receives the shrink output."""
    M, K = _dims(x, "x")
    R, Ka = _dims(a, "a")
    N, Rb = _dims(b, "b")
    if Ka != K or Rb != R:
        raise ValueError(f"x [M, {K}], a [{R}, {Ka}] and b [N, {Rb}] disagree on K or R")
    if base is not None:
        _want(base, (M, N), "base")
    if l is not None:
        _want(l, (M, R), "l")
    if y is not None:
        _want(y, (M, N), "y")
    else:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    px, ldx = _mat(x, "x", _BF16_LIKE)
    pa, lda = _mat(a, "a", _BF16_LIKE)
    pb, ldb = _mat(b, "b", _BF16_LIKE)
    py, ldy = _mat(y, "y", _BF16_LIKE)
    pbase, ldbase = _mat(base, "base", _BF16_LIKE) if base is not None else (None, N)
    pl, ldl = _mat(l, "l", (torch.float32,)) if l is not None else (None, R)
    _check(_lib_shrink_expand(px, pa, pb, pbase, py, pl, M, K, N, R, ldx, lda, ldb, ldbase, ldy,
                              ldl, float(scale), split_k, _stream(stream)), "bi_lora_shrink_expand")
    return y
