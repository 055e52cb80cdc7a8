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
