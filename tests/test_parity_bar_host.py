"""Host checks of the parity bar's near-tie rule (tests/parity_bar.py): only
an fp16 neighbour across a midpoint that the exact value sits on, within the
kernel's error bound, passes beyond the max bar; everything else fails.  The
bound itself is checked against an fp32 emulation of the kernel's
offset-carrying accumulation on the worst rows the workloads produce."""
import numpy as np
import pytest

from oracle import w4a4_oracle as O
from tests.parity_bar import check_y, kernel_error_bound, near_tie_flips


def _mid(v16):
    """Midpoint between the fp16 value v16 and its upper neighbour (fp64)."""
    up = np.nextafter(np.float16(v16), np.float16(np.inf))
    return 0.5 * (float(v16) + float(up)), up


def test_near_tie_rule():
    v = np.float16(300.0)                     # fp16 spacing 0.25 there
    mid, up = _mid(v)
    ref = np.array([v, v, v, v], np.float16)  # the oracle's rounding of y64
    gpu = np.array([up, up, up, np.float16(300.5)], np.float16)
    E = np.full(4, 1e-3)
    y64 = np.array([mid - 1e-4,               # within the bound of the tie: passes
                    mid - 0.05,               # a fifth of the spacing from it: not a tie
                    mid - 2e-3,               # just outside the bound
                    mid - 1e-4])              # two spacings away: not neighbours
    assert near_tie_flips(gpu, ref, y64, E).tolist() == [True, False, False, False]


def test_check_y_passes_only_near_tie_flips():
    rng = np.random.default_rng(0)
    y64 = (rng.standard_normal(4096) * 5.0).reshape(64, 64)
    y64[0, 7] = _mid(np.float16(300.0))[0] + 1e-6   # a large output right at a tie
    ref = y64.astype(np.float16)
    gpu = ref.copy()
    gpu[0, 7] = np.float16(300.0) if ref[0, 7] != np.float16(300.0) else _mid(np.float16(300.0))[1]
    bound = lambda r, c: np.full(len(r), 1e-4)
    assert check_y(gpu, ref, "tie", y64=y64, err_bound=bound, say=lambda *a: None) == 1
    with pytest.raises(AssertionError):          # without the exact values: a plain violation
        check_y(gpu, ref, "tie", say=lambda *a: None)
    with pytest.raises(AssertionError):          # a bound smaller than the distance to the tie
        check_y(gpu, ref, "tie", y64=y64, err_bound=lambda r, c: np.full(len(r), 1e-7), say=lambda *a: None)
    bad = ref.copy()
    bad[1, 9] = np.float16(float(ref[1, 9]) + 1.0)   # a real error of 1.0 on rms ~5: beyond the bar
    with pytest.raises(AssertionError):
        check_y(bad, ref, "error", y64=y64, err_bound=bound, say=lambda *a: None)


def _emulate_kernel(qx, sx, qw, sw):
    """fp32 emulation of the tiled kernel's group-sum accumulation for one
    output element: acc' = acc 2^-14, per k-pair acc' -= 3 (S0 + S1) (one
    rounding), then acc' += S_h * (3 + P_h 2^-14) for h = 0, 1 (fma: one
    rounding each); returns acc' * 2^14."""
    f = np.float32
    acc = f(0.0)
    G = qx.shape[0] // 64
    P = [int(np.dot(qx[64 * g: 64 * g + 64].astype(np.int64), qw[64 * g: 64 * g + 64].astype(np.int64)))
         for g in range(G)]
    S = [f(f(sx[g]) * f(sw[g])) for g in range(G)]
    for p in range(G // 2):
        acc = f(acc - f(3.0) * (S[2 * p] + S[2 * p + 1]))
        for h in range(2):
            t = f(3.0) + f(P[2 * p + h]) * f(2.0 ** -14)          # exact
            acc = f(np.float64(S[2 * p + h]) * np.float64(t) + np.float64(acc))   # fma
    return np.float64(acc) * 2.0 ** 14


def test_kernel_error_bound_covers_the_emulated_accumulation():
    """Heavy-tailed rows (Student-t x 30 outliers, like the prefill workload)
    against normal weights: the fp32 emulation stays within the bound."""
    rng = np.random.default_rng(1)
    K, n = 4096, 24
    x = rng.standard_t(3.0, size=(n, K))
    x[:, rng.choice(K, 41, replace=False)] *= 30.0
    w = rng.standard_normal((n, K)) * 0.02
    qx, sx = O.quantize_groups(x.astype(np.float16))
    qw, sw = O.quantize_groups(w.astype(np.float16))
    bound = kernel_error_bound(qx, sx, qw, sw, None, None, None, None)
    rows = np.arange(n)
    E = bound(rows, rows)
    for i in range(n):
        exact = O.main_term(qx[i:i + 1], sx[i:i + 1], qw[i:i + 1], sw[i:i + 1])[0, 0]
        got = _emulate_kernel(qx[i], sx[i], qw[i], sw[i])
        assert abs(got - exact) <= E[i], (i, got, exact, E[i])
    # and it is not vacuous: far below one fp16 spacing of these outputs
    assert np.all(E < 0.05)
