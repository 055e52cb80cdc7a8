"""Host checks of the arithmetic the tiled GEMM relies on to skip the
int -> float conversion of each group sum (no GPU; numpy emulation).

The integer MFMA adds 256 P (the int8 operands carry 16 q each, so
|256 P| <= 2^20) to its C operand.  Started from the bits of 3.0f, the
result read as fp32 must be exactly 3 + P 2^-14 for every reachable P; the
accumulator then takes, per k-pair, acc' - 3 (S_0 + S_1) followed by one fma
per group, S_h (3 + P_h 2^-14), and the epilogue multiplies by 2^14.
"""
import numpy as np

OFFSET_BITS = 0x40400000   # 3.0f


def _as_f32(bits):
    return np.asarray(bits, dtype=np.int64).astype(np.uint32).view(np.float32)


def _fma32(a, b, c):
    """fp32 fma: the product of two fp32 values is exact in fp64 (48 bits);
    the sum is rounded once to fp64 and then to fp32 -- a double rounding
    that differs from a true fma only in rare ties, far below what these
    checks resolve."""
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


def test_offset_bits_read_as_three_plus_scaled_sum():
    """Every P with |P| <= 4096 (64 products of int4 codes, at most 64 * 64):
    bits(3.0f) + 256 P reads as 3 + P / 16384 exactly, exponent unchanged."""
    assert _as_f32(OFFSET_BITS) == np.float32(3.0)
    p = np.arange(-4096, 4097, dtype=np.int64)
    got = _as_f32(OFFSET_BITS + 256 * p).astype(np.float64)
    assert np.array_equal(got, 3.0 + p / 16384.0)
    # the widest swing stays inside [2, 4): one exponent, so linear in P
    assert got.min() >= 2.0 and got.max() < 4.0


def test_offset_correction_products_are_exact():
    """The correction MFMA's operands: s_x doubled in fp16 (s_x <= 65504 / 7
    from an fp16 X, so 2 s_x cannot overflow) and every product of two fp16
    values exact in fp32, so 3 (S_0 + S_1) enters with only the MFMA's own
    sum rounding."""
    rng = np.random.default_rng(7)
    sx = rng.uniform(2.0 ** -24, 65504 / 7, 10000).astype(np.float16)
    assert np.all(np.isfinite((sx.astype(np.float32) * 2).astype(np.float16)))
    assert np.array_equal((sx.astype(np.float32) * 2).astype(np.float16).astype(np.float64),
                          2 * sx.astype(np.float64))
    sw = rng.uniform(1e-4, 10.0, 10000).astype(np.float16)
    prod = sx.astype(np.float32) * sw.astype(np.float32)
    assert np.array_equal(prod.astype(np.float64), sx.astype(np.float64) * sw.astype(np.float64))


def test_offset_accumulation_matches_exact_sum():
    """Emulated in fp32 over a long K (224 groups, as K = 14336), with
    scale magnitudes spanning 10^4 and sums near the int4 extremes: the
    offset-carrying accumulator, times 2^14, stays within 1e-5 of the exact
    sum relative to the sum of |S P| (the bound the fp32 accumulation of the
    plain convert + fma path meets with a wide margin too)."""
    rng = np.random.default_rng(11)
    for trial in range(20):
        G = 224
        sx = rng.uniform(1e-3, 10.0, G).astype(np.float16).astype(np.float64)
        sw = (rng.uniform(1e-3, 1.0, G) * 10.0 ** rng.uniform(-2, 0, G)).astype(np.float16).astype(np.float64)
        S = (sx * sw).astype(np.float32)           # exact (fp16 x fp16)
        P = rng.integers(-4096 if trial % 2 else -300, 4097 if trial % 2 else 301, G)
        D = _as_f32(OFFSET_BITS + 256 * P)
        acc = np.float32(0.0)
        for kp in range(G // 2):
            s0, s1 = S[2 * kp], S[2 * kp + 1]
            acc = np.float32(np.float64(acc) - 3.0 * (np.float64(s0) + np.float64(s1)))
            acc = _fma32(s0, D[2 * kp], acc)
            acc = _fma32(s1, D[2 * kp + 1], acc)
        got = np.float64(acc) * 16384.0
        exact = float(np.sum(S.astype(np.float64) * P))
        scale = float(np.sum(np.abs(S.astype(np.float64) * P)))
        assert abs(got - exact) <= 1e-5 * scale, (trial, got, exact, scale)


def test_offset_emulation_catches_a_dropped_correction():
    """The same emulation without the per-k-pair correction is far off: the
    check above would notice a kernel that forgot to remove the offsets."""
    rng = np.random.default_rng(3)
    S = rng.uniform(1e-3, 1.0, 64).astype(np.float32)
    P = rng.integers(-300, 301, 64)
    D = _as_f32(OFFSET_BITS + 256 * P)
    acc = np.float32(0.0)
    for h in range(64):
        acc = _fma32(S[h], D[h], acc)
    exact = float(np.sum(S.astype(np.float64) * P))
    scale = float(np.sum(np.abs(S.astype(np.float64) * P)))
    assert abs(np.float64(acc) * 16384.0 - exact) > 1e-2 * scale


# ---------------------------------------------------------------------------
# The quantizer's division-free quotient.  The kernels round x / s (x an fp16
# value, s the group's fp16 scale) as t0 = fl(x rs), e = fma(-t0, s, x),
# t = fma(e, rs, t0), n = rint(t), with rs the hardware reciprocal of s
# (within 1 ulp of 1/s).  The rule is n = rint(fl32(x / s)), ties to even.

def _f16_values(lo, hi):
    """Every positive finite fp16 value in [lo, hi], as fp64."""
    v = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    return v[(v >= lo) & (v <= hi)]


def _fl32_sum(a, b):
    """fl32(a + b) of fp64 values, rounded once: the fp64 sum plus its exact
    error (TwoSum) decide the one case where rounding the fp64 sum to fp32
    differs from rounding the exact sum -- an fp64 sum exactly halfway
    between two fp32 values."""
    hi = a + b
    bv = hi - a
    lo = (a - (hi - bv)) + (b - bv)
    r = hi.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    r64, up64, dn64 = r.astype(np.float64), up.astype(np.float64), dn.astype(np.float64)
    r = np.where((r64 < hi) & (hi - r64 == up64 - hi) & (lo > 0), up, r)
    r = np.where((r64 > hi) & (r64 - hi == hi - dn64) & (lo < 0), dn, r)
    return r


def _kernel_quotient(x, s, rs):
    """The kernels' t for fp64 arrays x, s (fp16 values) and fp32 rs; also
    checks that the residual e is exact in fp32."""
    x32, s32 = x.astype(np.float32), s.astype(np.float32)
    t0 = x32 * rs                                            # fl32 product
    e64 = x - t0.astype(np.float64) * s                      # exact in fp64 (<= 36 bits)
    e = e64.astype(np.float32)
    assert np.array_equal(e.astype(np.float64), e64), "the residual is not exact in fp32"
    return _fl32_sum(t0.astype(np.float64), e.astype(np.float64) * rs.astype(np.float64))


def _rne_exact(x, s):
    """Nearest integer to x / s, ties to even, in integer arithmetic
    (positive fp16 values are integer multiples of 2^-24)."""
    X = np.rint(x * 2.0 ** 24).astype(np.int64)
    S = np.rint(s * 2.0 ** 24).astype(np.int64)
    q, r = np.divmod(X, S)
    return q + (2 * r > S) + ((2 * r == S) & (q % 2 == 1))


def _check_scales(scales, x_hi_ratio=11.0):
    """Every positive fp16 x with s/4 <= x <= x_hi_ratio s (smaller x give 0
    on both sides), for each scale s and rs at 1/s rounded and at its two
    neighbours: the kernels' rint(t) equals the exact rounding and numpy's
    rint(fl32(x / s)).  Returns how many exact ties were met."""
    ties = 0
    for s in scales:
        x = _f16_values(s / 4, min(x_hi_ratio * s, 65504.0))
        sv = np.full_like(x, s)
        want = _rne_exact(x, sv)
        assert np.array_equal(np.rint(x.astype(np.float32) / np.float32(s)).astype(np.int64), want)
        rn = np.float32(1.0) / np.float32(s)
        for rs in (rn, np.nextafter(rn, np.float32(0)), np.nextafter(rn, np.float32(np.inf))):
            t = _kernel_quotient(x, sv, np.full(x.shape, rs, np.float32))
            got = np.rint(t).astype(np.int64)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"s={s!r} rs={rs!r} x={x[bad[:4]]} got {got[bad[:4]]} want {want[bad[:4]]}"
        ties += int(np.sum(np.rint(x / s * 2) == x / s * 2) - np.sum(np.rint(x / s) == x / s))
    return ties


def test_division_free_quotient_every_significand():
    """s over all 1024 fp16 significands in [1, 2) (a power-of-two scaling of
    s and x scales every step exactly, so this covers every normal s whose x
    range stays normal), x over every fp16 value up to 11 s."""
    s = np.arange(0x3C00, 0x4000, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert _check_scales(s) > 2000       # exact half-integer quotients are met (2233)


def test_division_free_quotient_subnormal_and_edge_scales():
    """Every subnormal scale (the group's absmax below 7 * 2^-14, including
    the 2^-24 floor of an all-zero group), the smallest normal ones, and
    the largest an fp16 X can give (65504 / 7 -> 9360)."""
    sub = np.arange(1, 0x0400, dtype=np.uint16).view(np.float16).astype(np.float64)
    edge = np.arange(0x0400, 0x0440, dtype=np.uint16).view(np.float16).astype(np.float64)
    top = np.arange(0x7000, 0x7092, 8, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert _check_scales(np.concatenate([sub, edge, top])) > 0


def test_plain_reciprocal_product_misrounds_ties():
    """Without the Newton step, rint(fl(x rs)) rounds some exact
    half-integer quotients the wrong way (fl(x rs) lands a hair off the
    tie), so the step and the checks above are not vacuous."""
    s = np.arange(0x3C00, 0x4000, dtype=np.uint16).view(np.float16).astype(np.float64)
    wrong = 0
    for sv in s:
        x = _f16_values(sv / 4, 11 * sv)
        rs = np.float32(1.0) / np.float32(sv)
        naive = np.rint(x.astype(np.float32) * rs).astype(np.int64)
        wrong += int(np.sum(naive != _rne_exact(x, np.full_like(x, sv))))
    assert wrong > 0
