"""Pins of the CPU oracle against what mathematics fixes (no GPU).

Each test checks the oracle against something other than itself: exact
rational arithmetic (``fractions.Fraction``), 50-digit decimal arithmetic,
exact integer arithmetic, closed forms, hand-derived tables in
``tests/golden/``, or brute force over every input of a tiny case.  The inputs
are chosen so that a plausible slip in the oracle (a transposed operand, a
dropped or doubled term, a wrong sign or index, eps in the wrong place, a
rounding tie sent the wrong way) fails at least one test.
"""
from __future__ import annotations

import decimal
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from invariant_deterministic_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------- exact helpers --

def bf16_fraction(h: int):
    """Exact value of a bf16 pattern as a Fraction (None for NaN, +-inf as str)."""
    s = -1 if (h >> 15) & 1 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    if e == 0xFF:
        return None if f else ("inf" if s > 0 else "-inf")
    if e == 0:
        return s * Fraction(f, 128) * Fraction(1, 2 ** 126)
    return s * (1 + Fraction(f, 128)) * (Fraction(2) ** (e - 127))


ALL_FINITE = np.array([h for h in range(1 << 16) if ((h >> 7) & 0xFF) != 0xFF],
                      dtype=np.uint16)


def random_bf16_wide(shape, seed, binades=20):
    """bf16 values with random signs and exponents spread over +-``binades``."""
    g = synth.rng(seed)
    mant = g.integers(0, 128, size=shape)
    expo = g.integers(127 - binades, 127 + binades + 1, size=shape)
    sign = g.integers(0, 2, size=shape)
    return ((sign << 15) | (expo << 7) | mant).astype(np.uint16)


# ------------------------------------------------------------------- bf16 --

def test_bf16_decode_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    dec = oracle.bf16_decode(bits)
    for h in range(1 << 16):
        ref = bf16_fraction(h)
        v = dec[h]
        if ref is None:
            assert math.isnan(v), hex(h)
        elif isinstance(ref, str):
            assert v == (math.inf if ref == "inf" else -math.inf), hex(h)
        else:
            assert Fraction(v) == ref, hex(h)
            assert math.copysign(1.0, v) == (-1.0 if h & 0x8000 else 1.0), hex(h)


def test_bf16_round_golden_table():
    n = 0
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            val, bits = line.split()
            got = int(oracle.bf16_round(np.array([float.fromhex(val)]))[0])
            assert got == int(bits, 16), f"{val}: got {got:#06x} want {bits}"
            n += 1
    assert n >= 20


def test_bf16_round_trips_every_finite_pattern():
    back = oracle.bf16_round(oracle.bf16_decode(ALL_FINITE))
    assert np.array_equal(back, ALL_FINITE)


def test_bf16_round_nan():
    assert int(oracle.bf16_round(np.array([math.nan]))[0]) & 0x7FC0 == 0x7FC0


def test_bf16_round_every_midpoint_goes_to_even():
    """Midpoints between all adjacent positive finite bf16 values, and their
    immediate double neighbours, against the exact nearest neighbour."""
    pos = np.sort(ALL_FINITE[ALL_FINITE < 0x8000])
    vals = oracle.bf16_decode(pos)
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2            # exact: both have <= 8 significant bits
    got = oracle.bf16_round(mid)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, even)
    above = oracle.bf16_round(np.nextafter(mid, np.inf))
    below = oracle.bf16_round(np.nextafter(mid, -np.inf))
    assert np.array_equal(above, pos[1:])
    assert np.array_equal(below, pos[:-1])
    # negative side is the mirror image
    assert np.array_equal(oracle.bf16_round(-mid), even | 0x8000)


def test_bf16_round_random_doubles_brute_force():
    """Random doubles: the result must be the nearest bf16 by exact distance,
    ties to even."""
    g = synth.rng(11)
    v = g.standard_normal(3000) * np.exp2(g.integers(-130, 128, size=3000))
    got = oracle.bf16_round(v)
    pos = np.sort(ALL_FINITE[ALL_FINITE < 0x8000])
    pvals = oracle.bf16_decode(pos)
    for x, h in zip(v.tolist(), got.tolist()):
        a = abs(x)
        i = int(np.searchsorted(pvals, a))
        cands = []
        for j in (i - 1, i, i + 1):
            if 0 <= j < len(pos):
                cands.append((abs(Fraction(a) - Fraction(float(pvals[j]))), int(pos[j]) % 2, int(pos[j])))
        top = Fraction(float(pvals[-1]))
        ulp = Fraction(2) ** (127 - 7)
        if Fraction(a) >= top + ulp / 2:
            want = 0x7F80
        else:
            cands.sort()
            want = cands[0][2]
        if x < 0:
            want |= 0x8000
        assert h == want, (x, hex(h), hex(want))


# ------------------------------------------------------------------- GEMM --

def test_gemm_integer_inputs_exact():
    """Integer inputs: every partial sum is an integer far below 2^53, so the
    fp64 result must equal the exact integer product.  Non-square shapes catch
    a transposed operand; signed values catch sign slips."""
    for (M, N, K), seed in (((5, 7, 1024), 1), ((3, 11, 4096), 2), ((2, 3, 14336), 3)):
        x = synth.int_bf16((M, K), seed, -4, 4)
        w = synth.int_bf16((N, K), seed + 100, -4, 4)
        xi = oracle.bf16_decode(x).astype(np.int64)
        wi = oracle.bf16_decode(w).astype(np.int64)
        exact = xi @ wi.T
        y = oracle.gemm(x, w)
        assert np.array_equal(y, exact.astype(np.float64))
        # and the bf16 rounding of the exact integers (ties exercised by values
        # in (256, 512) and beyond)
        yb = oracle.bf16_round(y)
        for v, b in zip(exact.ravel().tolist(), yb.ravel().tolist()):
            assert Fraction(float(oracle.bf16_decode(np.array([b], np.uint16))[0])) == \
                _nearest_even_int_in_bf16(v)


def _nearest_even_int_in_bf16(v: int) -> Fraction:
    """Nearest bf16 value to integer v by exact search (ties to even fraction)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.bit_length() - 1           # 2^e <= a < 2^(e+1)
    q = Fraction(2) ** (e - 7)       # quantum of that binade
    lo = (Fraction(a) // q) * q
    hi = lo + q
    dl, dh = Fraction(a) - lo, hi - Fraction(a)
    if dl < dh:
        r = lo
    elif dh < dl:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return r if v > 0 else -r


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
def test_gemm_brute_force_small_k(K):
    """K <= 8, values across +-20 binades: compare with exact rational sums;
    the fp64 sum may err by at most (K-1) * 2^-53 * sum|terms|."""
    x = random_bf16_wide((6, K), 20 + K)
    w = random_bf16_wide((5, K), 40 + K)
    y = oracle.gemm(x, w)
    for i in range(6):
        for j in range(5):
            terms = [bf16_fraction(int(x[i, k])) * bf16_fraction(int(w[j, k])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            bound = (K - 1) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[i, j])) - exact) <= bound


def test_gemm_brute_force_all_orders_k8():
    """Every one of the 8! sequential fp32 summation orders of one K=8 dot
    product stays within (K-1)*2^-24*sum|t| of the exact value, and more than
    one distinct fp32 result appears: the spread that reduction order alone
    causes, which the batch-invariant kernels must pin down."""
    x = random_bf16_wide((1, 8), 78, binades=6)
    w = random_bf16_wide((1, 8), 79, binades=6)
    terms32 = (oracle.bf16_decode(x[0]) * oracle.bf16_decode(w[0])).astype(np.float32)
    exact = sum((bf16_fraction(int(x[0, k])) * bf16_fraction(int(w[0, k])) for k in range(8)),
                Fraction(0))
    bound = 7 * Fraction(1, 2 ** 24) * sum(abs(Fraction(float(t))) for t in terms32)
    seen = set()
    for perm in itertools.permutations(range(8)):
        acc = np.float32(0.0)
        for k in perm:
            acc = np.float32(acc + terms32[k])
        seen.add(float(acc))
        assert abs(Fraction(float(acc)) - exact) <= bound
    assert len(seen) > 1
    y = oracle.gemm(x, w)[0, 0]
    assert abs(Fraction(float(y)) - exact) <= 7 * Fraction(1, 2 ** 53) * \
        sum(abs(Fraction(float(t))) for t in terms32)


def test_gemm_identity_and_one_hot():
    K = 64
    x = synth.normal_bf16((9, K), 5)
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    y = oracle.gemm(x, eye)
    assert np.array_equal(oracle.bf16_round(y), x)
    # one-hot rows of X pick out a column of W^T: y[r, j] = w[j, k_r]
    w = synth.normal_bf16((13, K), 6)
    ks = np.array([0, 1, 17, 63])
    oh = np.zeros((len(ks), K), dtype=np.uint16)
    oh[np.arange(len(ks)), ks] = 0x3F80
    y = oracle.gemm(oh, w)
    assert np.array_equal(oracle.bf16_round(y), w[:, ks].T)


def test_nonassociativity_case():
    """(a+b)+c != a+(b+c) in fp32 for a=1, b=c=2^-24 -- the pages' example of
    order-dependent rounding -- and the fp64 oracle gets the exact sum."""
    a, b = np.float32(1.0), np.float32(2.0 ** -24)
    left = np.float32(np.float32(a + b) + b)
    right = np.float32(a + np.float32(b + b))
    assert left == np.float32(1.0)
    assert right == np.float32(1.0 + 2.0 ** -23)
    assert left != right
    x = np.zeros((1, 3), np.uint16)
    x[0] = 0x3F80
    w = synth.f32_to_bf16_bits(np.array([[1.0, 2.0 ** -24, 2.0 ** -24]], np.float32))
    assert oracle.gemm(x, w)[0, 0] == 1.0 + 2.0 ** -23
    assert oracle.gemm(x[:, ::-1].copy(), w[:, ::-1].copy())[0, 0] == 1.0 + 2.0 ** -23


def test_gemm_thread_count_does_not_change_bits():
    x = synth.normal_bf16((33, 256), 8)
    w = synth.normal_bf16((17, 256), 9)
    a = oracle.gemm(x, w, threads=1)
    b = oracle.gemm(x, w, threads=0)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


# ---------------------------------------------------------------- RMSNorm --

def _exact_rmsnorm_row(xrow, wvec, eps_f64, digits=50):
    ctx = decimal.Context(prec=digits)
    xs = [bf16_fraction(int(h)) for h in xrow]
    ws = [bf16_fraction(int(h)) for h in wvec]
    K = len(xs)
    ms = sum((v * v for v in xs), Fraction(0)) / K + Fraction(eps_f64)
    d = ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator))
    r = ctx.divide(decimal.Decimal(1), ctx.sqrt(d))
    return [ctx.multiply(ctx.multiply(decimal.Decimal(v.numerator) / decimal.Decimal(v.denominator), r),
                         decimal.Decimal(wv.numerator) / decimal.Decimal(wv.denominator))
            for v, wv in zip(xs, ws)]


@pytest.mark.parametrize("K", [1, 2, 4, 7, 8])
def test_rmsnorm_brute_force_small_k(K):
    x = random_bf16_wide((4, K), 90 + K, binades=10)
    w = random_bf16_wide((K,), 99 + K, binades=2)
    eps = float(np.float32(1e-6))
    y = oracle.rmsnorm(x, w, eps)
    for i in range(4):
        ex = _exact_rmsnorm_row(x[i], w, eps)
        for k in range(K):
            e = float(ex[k])
            assert abs(y[i, k] - e) <= 2.0 ** -49 * abs(e) + 1e-300


def test_rmsnorm_unit_weight_closed_form():
    """w = 1: mean_k y^2 = ms / (ms + eps) exactly in real arithmetic (= 1 when
    eps = 0); eps inside the root is what makes this hold."""
    K = 1024
    x = synth.normal_bf16((16, K), 31, std=1.0 / 32)
    ones = np.full(K, 0x3F80, np.uint16)
    for eps in (float(np.float32(1e-6)), 0.0, 1.0):
        y = oracle.rmsnorm(x, ones, eps)
        xd = oracle.bf16_decode(x)
        ms = (xd * xd).mean(axis=1)
        lhs = (y * y).mean(axis=1)
        rhs = ms / (ms + eps)
        assert np.allclose(lhs, rhs, rtol=1e-12, atol=0)


def test_rmsnorm_constant_rows_exact():
    """x = c * 1 with c = 2^j and eps = 0 gives y = sign(c) * w exactly."""
    K = 256
    w = synth.normal_bf16((K,), 32, mean=1.0, std=0.1)
    for j in (-20, -3, 0, 5, 40):
        for s in (1.0, -1.0):
            x = synth.f32_to_bf16_bits(np.full((1, K), s * 2.0 ** j, np.float32))
            y = oracle.rmsnorm(x, w, 0.0)
            want = oracle.bf16_decode(w) * s
            assert np.array_equal(y[0], want)


def test_rmsnorm_power_of_two_scale_invariance():
    K = 512
    x = synth.normal_bf16((8, K), 33)
    w = synth.normal_bf16((K,), 34, mean=1.0, std=0.1)
    y = oracle.rmsnorm(x, w, 0.0)
    for j in (-6, 3, 9):
        xs = oracle.bf16_round(oracle.bf16_decode(x) * 2.0 ** j)   # exact rescale
        ys = oracle.rmsnorm(xs, w, 0.0)
        assert np.array_equal(y.view(np.uint64), ys.view(np.uint64))


def test_rmsnorm_zero_row_and_row_independence():
    K = 128
    x = synth.normal_bf16((5, K), 35)
    x[2] = 0
    w = synth.normal_bf16((K,), 36, mean=1.0, std=0.1)
    y = oracle.rmsnorm(x, w, 1e-6)
    assert np.all(y[2] == 0.0)
    for i in range(5):      # each row alone gives the same bits
        yi = oracle.rmsnorm(x[i:i + 1], w, 1e-6)
        assert np.array_equal(yi[0].view(np.uint64), y[i].view(np.uint64))


def test_rmsnorm_uses_weight_per_column():
    K = 8
    x = synth.f32_to_bf16_bits(np.ones((1, K), np.float32))
    w = synth.f32_to_bf16_bits(np.arange(1, K + 1, dtype=np.float32))
    y = oracle.rmsnorm(x, w, 0.0)
    assert np.array_equal(y[0], np.arange(1, K + 1, dtype=np.float64))


# ----------------------------------------------------- fixed-order combine --

def _round_f32_exact(q: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 value, ties to even (normal range)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (e - 23)
    lo = (a // quantum) * quantum
    hi = lo + quantum
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / quantum) % 2 == 0 else hi
    return r if q > 0 else -r


def test_combine_each_step_is_one_correct_fp32_rounding():
    """Random partials: each step of the left fold must be the correctly
    rounded fp32 of (previous + next), checked with exact rationals."""
    g = synth.rng(41)
    p = (g.standard_normal((8, 64)) * np.exp2(g.integers(-8, 8, size=(8, 64)))).astype(np.float32)
    got = oracle.combine_f32(p)
    for e in range(64):
        acc = Fraction(float(p[0, e]))
        for s in range(1, 8):
            acc = _round_f32_exact(acc + Fraction(float(p[s, e])))
        assert Fraction(float(got[e])) == acc


def test_combine_order_pin():
    """p = [1, 2^-24, 2^-24, 0...]: the left fold gives exactly 1.0, whereas
    summing the two small terms first would give 1 + 2^-23."""
    p = np.zeros((8, 1), np.float32)
    p[0], p[1], p[2] = 1.0, 2.0 ** -24, 2.0 ** -24
    assert oracle.combine_f32(p)[0] == np.float32(1.0)
    assert oracle.combine_f32(p[[1, 2, 0, 3, 4, 5, 6, 7]])[0] == np.float32(1.0 + 2.0 ** -23)


def test_combine_integer_partials_exact():
    g = synth.rng(42)
    p = g.integers(-1000, 1000, size=(8, 100)).astype(np.float32)
    assert np.array_equal(oracle.combine_f32(p), p.astype(np.int64).sum(axis=0).astype(np.float32))


def test_fixed_order_golden_file_matches_oracle():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "mk", os.path.join(GOLDEN, "make_fixed_order_pins.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(GOLDEN, "fixed_order_pins.txt")) as f:
        stored = [tuple(c.strip() for c in ln.split("|")) for ln in f
                  if ln.strip() and not ln.startswith("#")]
    fresh = [tuple(str(c) for c in r) for r in mk.pins()]
    assert stored == fresh
    table = {r[0]: r for r in stored}
    # the hand derivation: ascending K order gives 1 + 2^-8 in fp32, a bf16 tie
    # that goes to the even neighbour 1.0 = 0x3F80; reversed order keeps both
    # 2^-24 terms and lands above the tie.
    assert table["gemm_korder_ascending"][3:] == ("0x3F808000", "0x3F80")
    assert table["gemm_korder_descending_is_wrong"][4] == "0x3F81"
    assert table["shrink_split8_fixed_order"][4] == "0x3F800000"
    assert table["shrink_atomic_any_of"][4] == "0x3F800000,0x3F800001"


# ------------------------------------------------------- bit differences --

def test_bitdiff_hand_pins():
    u16 = lambda *v: np.array(v, dtype=np.uint16)
    u32 = lambda *v: np.array(v, dtype=np.uint32)
    assert oracle.bitdiff(u16(0x0000), u16(0x8000)) == (1, 1)     # +0 vs -0
    assert oracle.bitdiff(u16(0x3F80), u16(0x3F81)) == (1, 1)
    assert oracle.bitdiff(u16(0xFFFF), u16(0x0000)) == (16, 1)
    assert oracle.bitdiff(u16(1, 2, 3), u16(1, 2, 3)) == (0, 0)
    assert oracle.bitdiff(u32(0x3F800000, 7), u32(0x3F800001, 0)) == (4, 2)
    assert oracle.bitdiff(u32(0x7FC00000), u32(0x7FC00001)) == (1, 1)   # NaN payload


def test_bitdiff_random_against_python_popcount():
    g = synth.rng(43)
    a = g.integers(0, 1 << 32, size=1000, dtype=np.uint64).astype(np.uint32)
    b = a.copy()
    flip = g.integers(0, 1000, size=37)
    for i in flip:
        b[i] ^= np.uint32(1 << int(g.integers(0, 32)))
    bits = sum(bin(int(x) ^ int(y)).count("1") for x, y in zip(a, b))
    elems = sum(1 for x, y in zip(a, b) if x != y)
    assert oracle.bitdiff(a, b) == (bits, elems)


# ------------------------------------------------------- decode attention --

def _attn_exact(q, k, v, lens, digits=50):
    """Brute-force decode attention with 50-digit decimals (exact dot products,
    decimal exp), for tiny sizes."""
    ctx = decimal.Context(prec=digits)
    B, H, D = q.shape
    _, Tmax, Hkv, _ = k.shape
    G = H // Hkv
    dec = lambda h: (lambda f: ctx.divide(decimal.Decimal(f.numerator), decimal.Decimal(f.denominator)))(bf16_fraction(int(h)))
    out = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            kh = h // G
            scale = ctx.divide(decimal.Decimal(1), ctx.sqrt(decimal.Decimal(D)))
            s = []
            for t in range(int(lens[b])):
                acc = decimal.Decimal(0)
                for d in range(D):
                    acc = ctx.add(acc, ctx.multiply(dec(q[b, h, d]), dec(k[b, t, kh, d])))
                s.append(ctx.multiply(acc, scale))
            mx = max(s)
            p = [ctx.exp(ctx.subtract(x, mx)) for x in s]
            l = sum(p, decimal.Decimal(0))
            for d in range(D):
                num = sum((ctx.multiply(p[t], dec(v[b, t, kh, d])) for t in range(len(p))), decimal.Decimal(0))
                out[b, h, d] = float(ctx.divide(num, l))
    return out


def test_attention_brute_force_small():
    """B=2, H=4 query heads over Hkv=2 key/value heads (groups of 2), D=4,
    ragged lengths 3 and 5: against 50-digit decimal arithmetic."""
    q = random_bf16_wide((2, 4, 4), 501, binades=2)
    k = random_bf16_wide((2, 6, 2, 4), 502, binades=2)
    v = random_bf16_wide((2, 6, 2, 4), 503, binades=3)
    lens = np.array([3, 5], np.int32)
    o = oracle.decode_attention(q, k, v, lens)
    ex = _attn_exact(q, k, v, lens)
    assert np.allclose(o, ex, rtol=1e-13, atol=1e-13 * np.abs(ex).max())


def test_attention_single_token_is_value():
    q = synth.normal_bf16((3, 8, 64), 504)
    k = synth.normal_bf16((3, 4, 2, 64), 505)
    v = synth.normal_bf16((3, 4, 2, 64), 506)
    o = oracle.decode_attention(q, k, v, np.ones(3, np.int32))
    vd = oracle.bf16_decode(v)
    for h in range(8):
        assert np.array_equal(o[:, h], vd[:, 0, h // 4])


def test_attention_uniform_keys_average_values():
    """Equal keys give equal weights: the output is the plain mean of V."""
    B, H, Hkv, D, T = 2, 4, 4, 32, 37
    q = synth.normal_bf16((B, H, D), 507)
    k = np.broadcast_to(synth.normal_bf16((1, 1, Hkv, D), 508), (B, T, Hkv, D)).copy()
    v = synth.normal_bf16((B, T, Hkv, D), 509)
    o = oracle.decode_attention(q, k, v, np.full(B, T, np.int32))
    mean = oracle.bf16_decode(v).mean(axis=1)          # [B, Hkv, D]
    assert np.allclose(o, mean, rtol=1e-13, atol=1e-15)


def test_attention_dominant_key_and_masked_tail():
    """One key far above the rest selects its value; positions past a
    sequence's length (filled with NaN) are never read."""
    B, H, D, Tmax = 2, 2, 16, 9
    q = synth.f32_to_bf16_bits(np.ones((B, H, D), np.float32))
    k = synth.normal_bf16((B, Tmax, H, D), 510, std=0.01)
    k[:, 2] = synth.f32_to_bf16_bits(np.full((B, H, D), 8.0, np.float32))   # score 8*16/4 = 32
    v = synth.normal_bf16((B, Tmax, H, D), 511)
    lens = np.array([5, 3], np.int32)
    k[0, 5:] = 0x7FC0
    v[0, 5:] = 0x7FC0
    k[1, 3:] = 0x7FC0
    v[1, 3:] = 0x7FC0
    o = oracle.decode_attention(q, k, v, lens)
    assert np.all(np.isfinite(o))
    vd = oracle.bf16_decode(v)
    assert np.allclose(o[:, :, :], vd[:, 2, :, :], rtol=0, atol=1e-12 * 8)


# ------------------------------------------------------------ LoRA expand --

def test_lora_expand_integer_inputs_exact():
    g = synth.rng(801)
    l = g.integers(-50, 50, size=(7, 16)).astype(np.float32)
    b = synth.int_bf16((13, 16), 802, -8, 8)
    base = synth.int_bf16((7, 13), 803, -100, 100)
    bi = oracle.bf16_decode(b).astype(np.int64)
    exact = oracle.bf16_decode(base).astype(np.int64) + 3 * (l.astype(np.int64) @ bi.T)
    assert np.array_equal(oracle.lora_expand(l, b, base, scale=3.0), exact.astype(np.float64))
    assert np.array_equal(oracle.lora_expand(l, b, None, scale=1.0), (l.astype(np.int64) @ bi.T).astype(np.float64))


def test_lora_expand_brute_force_rational():
    g = synth.rng(804)
    l = (g.standard_normal((3, 16)) * 3).astype(np.float32)
    b = random_bf16_wide((5, 16), 805, binades=6)
    base = random_bf16_wide((3, 5), 806, binades=4)
    y = oracle.lora_expand(l, b, base, scale=0.5)
    for m in range(3):
        for n in range(5):
            terms = [Fraction(float(l[m, r])) * bf16_fraction(int(b[n, r])) for r in range(16)]
            exact = bf16_fraction(int(base[m, n])) + Fraction(1, 2) * sum(terms, Fraction(0))
            bound = 16 * Fraction(1, 2 ** 52) * (abs(bf16_fraction(int(base[m, n]))) + sum(abs(t) for t in terms))
            assert abs(Fraction(float(y[m, n])) - exact) <= bound


def test_lora_expand_zero_scale_returns_base():
    base = synth.normal_bf16((4, 9), 807)
    l = np.ones((4, 16), np.float32)
    b = synth.normal_bf16((9, 16), 808)
    assert np.array_equal(oracle.lora_expand(l, b, base, scale=0.0), oracle.bf16_decode(base))
