"""CPU oracle for the batch-invariant reduction path (fp64, plain loops).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product (the
``invariant_deterministic_amd`` package and its HIP library) never imports it,
and this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (see its header for the definitions and the
passages of the pages they follow).  This module only loads the compiled
library with ctypes and marshals numpy arrays.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
exact rational arithmetic, closed forms and brute force; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -O2 without -ffast-math: no reassociation.  -ffp-contract=off: no fused
# multiply-add, so every fp64 operation rounds exactly as written.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc; return its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_bf16_decode.argtypes = [p, p, i64]
        L.oracle_bf16_round.argtypes = [p, p, i64]
        L.oracle_gemm.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64, ctypes.c_int]
        L.oracle_rmsnorm.argtypes = [p, i64, p, p, i64, i64, i64, ctypes.c_double,
                                     ctypes.c_int]
        L.oracle_combine_f32.argtypes = [p, i64, i64, p]
        L.oracle_bitdiff.argtypes = [p, p, i64, ctypes.c_int, p]
        L.oracle_decode_attention.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_int]
        L.oracle_lora_expand.argtypes = [p, p, p, p, i64, i64, i64, ctypes.c_double]
        L.oracle_max_threads.restype = ctypes.c_int
        for f in (L.oracle_bf16_decode, L.oracle_bf16_round, L.oracle_gemm,
                  L.oracle_rmsnorm, L.oracle_combine_f32, L.oracle_bitdiff,
                  L.oracle_decode_attention, L.oracle_lora_expand):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def bf16_decode(bits) -> np.ndarray:
    """Exact fp64 value of each bf16 bit pattern."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_bf16_decode(_ptr(b), _ptr(out), b.size)
    return out


def bf16_round(values) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round(_ptr(v), _ptr(out), v.size)
    return out


def gemm(x, w, threads: int = 0) -> np.ndarray:
    """fp64 ``y[i, j] = sum_k x[i, k] * w[j, k]`` for bf16 ``x [M, K]``, ``w [N, K]``."""
    x = _u16(x)
    w = _u16(w)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch {x.shape} x {w.shape}")
    M, K = x.shape
    N = w.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm(_ptr(x), K, _ptr(w), K, _ptr(y), N, M, N, K, threads)
    return y


def lora_shrink(x, a, threads: int = 0) -> np.ndarray:
    """fp64 LoRA shrink ``y[m, r] = sum_k x[m, k] * a[r, k]`` (A stored ``[R, K]``).

    Splitting K changes only the order of the sums, not the value computed, so
    every split variant is compared against this one definition."""
    return gemm(x, a, threads)


def rmsnorm(x, w, eps: float, threads: int = 0) -> np.ndarray:
    """fp64 RMSNorm of each row of bf16 ``x [M, K]`` with bf16 weight ``w [K]``."""
    x = _u16(x)
    w = _u16(w)
    if x.ndim != 2 or w.shape != (x.shape[1],):
        raise ValueError(f"shape mismatch {x.shape} / {w.shape}")
    M, K = x.shape
    y = np.empty((M, K), dtype=np.float64)
    lib().oracle_rmsnorm(_ptr(x), K, _ptr(w), _ptr(y), K, M, K, float(eps), threads)
    return y


def decode_attention(q, k, v, lens, threads: int = 0) -> np.ndarray:
    """fp64 decode attention.  q [B, H, D], k and v [B, Tmax, Hkv, D] (bf16
    bits), lens [B] valid tokens per sequence -> o [B, H, D]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, H, D = q.shape
    Bk, Tmax, Hkv, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D or H % Hkv or lens.shape != (B,):
        raise ValueError("shape mismatch")
    if np.any(lens < 1) or np.any(lens > Tmax):
        raise ValueError("lengths must be in [1, Tmax]")
    o = np.empty((B, H, D), dtype=np.float64)
    lib().oracle_decode_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(lens), _ptr(o), B, H, Hkv, D,
                                  Tmax, threads)
    return o


def lora_expand(l, b, base=None, scale: float = 1.0) -> np.ndarray:
    """fp64 ``y[m, n] = base[m, n] + scale * sum_r l[m, r] * b[n, r]`` with fp32
    ``l [M, R]``, bf16 ``b [N, R]``, optional bf16 ``base [M, N]``."""
    l = np.ascontiguousarray(l, dtype=np.float32)
    b = _u16(b)
    M, R = l.shape
    N = b.shape[0]
    if b.shape != (N, R):
        raise ValueError("shape mismatch")
    bp = 0
    if base is not None:
        base = _u16(base)
        if base.shape != (M, N):
            raise ValueError("base shape mismatch")
        bp = _ptr(base)
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_lora_expand(_ptr(l), _ptr(b), bp or None, _ptr(y), M, N, R, float(scale))
    return y


def combine_f32(partials) -> np.ndarray:
    """Left fold in fp32 over the first axis: ``((p0 + p1) + p2) + ...``."""
    p = np.ascontiguousarray(partials, dtype=np.float32)
    S = p.shape[0]
    n = p[0].size
    out = np.empty(p.shape[1:], dtype=np.float32)
    lib().oracle_combine_f32(_ptr(p), S, n, _ptr(out))
    return out


def bitdiff(a, b) -> tuple[int, int]:
    """(differing bits, differing elements) between two equal-shape arrays of
    2- or 4-byte elements, compared as raw bits."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.shape != b.shape or a.dtype.itemsize != b.dtype.itemsize:
        raise ValueError("bitdiff needs equal shapes and element sizes")
    if a.dtype.itemsize not in (2, 4):
        raise ValueError("bitdiff supports 2- and 4-byte elements")
    out = np.zeros(2, dtype=np.uint64)
    lib().oracle_bitdiff(_ptr(a), _ptr(b), a.size, a.dtype.itemsize, _ptr(out))
    return int(out[0]), int(out[1])
