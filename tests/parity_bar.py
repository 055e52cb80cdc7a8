"""The layer's parity bar (no GPU needed): max|dY| <= 2e-2 rms(Y_oracle) and
mean|dY| <= 2e-3 rms(Y_oracle), rms over every compared output, with the
oracle's exact values deciding the rounding of near ties."""
import numpy as np

MAX_TOL = 2e-2
MEAN_TOL = 2e-3


# Rounding near a tie: where the oracle's exact (fp64) output lies within the
# kernel's own fp32 error of the midpoint between two neighbouring fp16
# values, the GPU's value may land on the other side, and either neighbour is
# a correct fp16 rounding of a value that close to exact.


def kernel_error_bound(qx, sx, qw, sw, la, lu, a, b):
    """Per-element bound on |fp32 result - exact| of the GPU epilogue before
    its fp16 rounding, for elements (rows[i], cols[i]) (a callable).

    The tiled kernel keeps acc' = acc 2^-14 in fp32; each group sum arrives
    as 3 + P 2^-14 and per k-pair the offsets leave through one MFMA.  Per
    k-pair that is at most 6 roundings (4 inside the offset MFMA's sum, one
    per fma), each within 2^-24 of a value no larger, in acc units, than the
    running sum plus the carried offset 3 2^14 (S0 + S1).  With G groups,
    A = sum_g S_g |P_g|, Sigma = sum_g S_g, L = sum_r |lora_act_r L_up_r|:
    LoRA adds the fp16 hi + lo split of lora_act (2^-22 relative) and 2R
    MFMA terms, the affine one fma:
        |err| <= 2^-24 (|a| ((3G + 2R + 2) A + 18 2^14 Sigma + (2R + 5) L) + |b|).
    Every rounding at its worst and of one sign: loose by about the square
    root of the rounding count in practice."""
    G = qx.shape[1] // 64
    R = 0 if la is None else la.shape[1]

    def bound(rows, cols):
        xq = qx[rows].reshape(len(rows), G, 64).astype(np.int64)
        wq = qw[cols].reshape(len(cols), G, 64).astype(np.int64)
        P = (xq * wq).sum(axis=2)
        S = sx[rows].astype(np.float64) * sw[cols].astype(np.float64)
        A = (S * np.abs(P)).sum(axis=1)
        Sigma = S.sum(axis=1)
        L = np.zeros(len(rows)) if R == 0 else np.abs(la[rows] * lu[cols].astype(np.float64)).sum(axis=1)
        aa = np.abs(np.asarray(a, np.float64)[cols]) if a is not None else np.ones(len(cols))
        bb = np.abs(np.asarray(b, np.float64)[cols]) if b is not None else np.zeros(len(cols))
        return 2.0 ** -24 * (aa * ((3 * G + 2 * R + 2) * A + 18 * 2.0 ** 14 * Sigma + (2 * R + 5) * L) + bb)

    return bound


def near_tie_flips(yg16, yr16, y64, E):
    """Mask of elements whose fp16 values are the two neighbours around the
    exact value y64, with y64 within E of their midpoint."""
    yg = yg16.astype(np.float64)
    yr = yr16.astype(np.float64)
    lo, hi = np.minimum(yg, yr), np.maximum(yg, yr)
    adjacent = np.nextafter(lo.astype(np.float16), np.float16(np.inf)).astype(np.float64) == hi
    between = (lo <= y64) & (y64 <= hi)
    near = np.abs(y64 - 0.5 * (lo + hi)) <= E
    return adjacent & between & near & (yg != yr)


def check_y(y_gpu, y_ref, what, y64=None, err_bound=None, say=print):
    """The layer bar: max|dY| <= 2e-2 rms(Y_oracle), mean|dY| <= 2e-3 rms,
    rms over every compared output.  Given the oracle's exact values y64 and
    the kernel's error bound (kernel_error_bound, called with the row and
    column indices of the elements concerned), an element beyond the max bar
    still passes if it is the other correct rounding of a near tie
    (near_tie_flips): at heavy-tailed outputs the fp16 spacing alone exceeds
    2e-2 rms (|Y| > 2^11 * 2e-2 rms), and the pages' own per-layer check
    (2e-2 of max|y_ref|) accepts such a flip.  Returns the number of
    elements passed that way."""
    yg = y_gpu.astype(np.float64)
    yr = y_ref.astype(np.float64)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(yr ** 2))
    err = np.abs(yg - yr)
    over = err > MAX_TOL * rms
    flips = np.zeros_like(over)
    if y64 is not None and err_bound is not None and over.any():
        idx = np.argwhere(over)
        E = err_bound(idx[:, 0], idx[:, 1])
        flips[over] = near_tie_flips(y_gpu[over], y_ref[over], y64[over], E)
        over &= ~flips
    rest = err[~flips]
    say(f"{what}: rms={rms:.4g} max|dY|/rms={err.max() / rms:.3g} mean|dY|/rms={err.mean() / rms:.3g}"
        f" (near-tie flips beyond the max bar: {int(flips.sum())}; max over the rest "
        f"{(rest.max() if rest.size else 0.0) / rms:.3g})")
    assert not over.any(), (f"{what}: {int(over.sum())} outputs beyond {MAX_TOL}*rms (rms {rms}), first at "
                            f"{np.argwhere(over)[0]}: {err[over][0]}")
    assert err.mean() <= MEAN_TOL * rms, f"{what}: mean err {err.mean()} > {MEAN_TOL}*{rms}"
    return int(flips.sum())
