"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived values (tests/golden), closed forms, invariants, special cases
that reduce to a library routine, and brute force on tiny inputs.

Each test names the mistake it is meant to catch.
"""
import itertools
import json
import os
import struct

import numpy as np
import pytest

from oracle import w4a4_oracle as O
from w4a4_gemm_lora_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits16(a):
    return np.asarray(a, np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# fp16 rounding used by the oracle (numpy's cast) -- ties and range
# ----------------------------------------------------------------------------
def test_fp16_rounding_ties_and_overflow():
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10 -> even (1.0)
    assert O.to_fp16(np.float64(1 + 2 ** -11)) == np.float16(1.0)
    # 1 + 3*2^-11 is halfway between 1+2^-10 and 1+2^-9 -> even (1+2^-9)
    assert float(O.to_fp16(np.float64(1 + 3 * 2 ** -11))) == 1 + 2 ** -9
    # subnormal ties: 2^-25 -> 0, 3*2^-25 -> 2^-23
    assert float(O.to_fp16(np.float64(2 ** -25))) == 0.0
    assert float(O.to_fp16(np.float64(3 * 2 ** -25))) == 2 ** -23
    # largest finite 65504; 65519.99 rounds to it, 65520 overflows to inf
    assert float(O.to_fp16(np.float64(65519.99))) == 65504.0
    assert np.isinf(O.to_fp16(np.float64(65520.0)))
    # agrees with Python's own binary16 packing on random doubles
    rng = np.random.default_rng(1)
    v = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 10, 2000))
    ours = O.to_fp16(v).astype(np.float64)
    py = np.array([struct.unpack("e", struct.pack("e", float(t)))[0] if abs(t) < 65504 else np.nan
                   for t in v])
    ok = ~np.isnan(py)
    assert np.array_equal(ours[ok], py[ok])


# ----------------------------------------------------------------------------
# Quantizer
# ----------------------------------------------------------------------------
def test_quantizer_golden_groups():
    """Hand-derived cases: ties to even, the /7 rule, dividing by the stored
    fp16 scale, the zero-group floor and the subnormal clamp."""
    cases = _load("quantize_cases.json")["groups"]
    for c in cases:
        x = np.zeros((1, 64), np.float16)
        x[0, : len(c["x"])] = np.array(c["x"], np.float64).astype(np.float16)
        assert np.array_equal(x[0, : len(c["x"])].astype(np.float64), np.array(c["x"])), c["name"]
        q, s = O.quantize_groups(x)
        want = np.zeros(64, np.int8)
        want[: len(c["q"])] = c["q"]
        assert np.array_equal(q[0], want), (c["name"], q[0][:16])
        assert int(_bits16(s)[0, 0]) == c["s_bits"], c["name"]


def test_quantizer_group_boundaries():
    """Two golden groups side by side in one 128-wide row keep their own
    scales (catches a wrong group width or offset)."""
    cases = {c["name"]: c for c in _load("quantize_cases.json")["groups"]}
    a, b = cases["unit_scale_ties"], cases["divide_by_stored_fp16_scale"]
    x = np.zeros((2, 128), np.float16)
    x[0, : len(a["x"])] = a["x"]
    x[0, 64: 64 + len(b["x"])] = b["x"]
    x[1, : len(b["x"])] = b["x"]
    x[1, 64: 64 + len(a["x"])] = a["x"]
    q, s = O.quantize_groups(x)
    assert _bits16(s).tolist() == [[a["s_bits"], b["s_bits"]], [b["s_bits"], a["s_bits"]]]
    assert q[0, : len(a["q"])].tolist() == a["q"]
    assert q[0, 64: 64 + len(b["q"])].tolist() == b["q"]
    assert q[1, 64: 64 + len(a["q"])].tolist() == a["q"]


def _random_rows(seed, rows=64, K=512):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(-8, 8, size=(rows, 1)))
    return (rng.standard_normal((rows, K)) * scale).astype(np.float16)


def test_quantizer_round_trip_bound_and_absmax_code():
    """|x - q*s| <= s/2 (+ fp32 division rounding) for normal scales, and the
    group's absmax element always maps to |q| = 7 (pins 'absmax / 7')."""
    x = _random_rows(2)
    q, s = O.quantize_groups(x)
    xs = x.astype(np.float64).reshape(64, -1, 64)
    qs = q.astype(np.float64).reshape(64, -1, 64)
    ss = s.astype(np.float64)[:, :, None]
    normal = (ss >= 2.0 ** -14)
    err = np.abs(xs - qs * ss)
    bound = ss / 2 + np.abs(xs) * 2.0 ** -23
    assert np.all(err[np.broadcast_to(normal, err.shape)] <= bound[np.broadcast_to(normal, err.shape)])
    amax_q = np.max(np.abs(qs), axis=2)
    assert np.all(amax_q[normal[:, :, 0]] == 7)
    assert q.min() >= -7  # -8 is unreachable with a normal scale


def test_quantizer_odd_symmetry_and_power_of_two_equivariance():
    x = _random_rows(3)
    q, s = O.quantize_groups(x)
    qn, sn = O.quantize_groups(-x)
    assert np.array_equal(qn, -q) and np.array_equal(_bits16(sn), _bits16(s))
    # scaling by 2^j keeps q and scales s by 2^j while everything stays normal
    y = (x.astype(np.float64) * 8.0)
    keep = np.all(np.abs(y) < 6e4, axis=1) & np.all(s.astype(np.float64) >= 2.0 ** -11, axis=1)
    q8, s8 = O.quantize_groups(y[keep].astype(np.float16))
    assert np.array_equal(q8, q[keep])
    assert np.array_equal(s8.astype(np.float64), s[keep].astype(np.float64) * 8.0)


def test_quantizer_brute_force_all_fp16_values_unit_scale():
    """Every finite fp16 v with |v| <= 7 in a group whose absmax is 7 (so the
    scale is exactly 1) must quantize to Python's round-half-even of v."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    v = v[np.isfinite(v) & (np.abs(v.astype(np.float64)) <= 7.0)]
    x = np.zeros((len(v), 64), np.float16)
    x[:, 0] = 7.0
    x[:, 1] = v
    q, s = O.quantize_groups(x)
    assert np.all(s.astype(np.float64) == 1.0)
    want = np.array([round(float(t)) for t in v.astype(np.float64)], np.int64)  # banker's rounding
    assert np.array_equal(q[:, 1].astype(np.int64), want)


def test_unpack_qweight_golden():
    g = _load("qweight_nibbles.json")
    q = O.unpack_qweight(np.array([g["bytes"]], np.uint8), 2 * len(g["bytes"]))
    assert q[0].tolist() == g["q"]


# ----------------------------------------------------------------------------
# Integer group sums
# ----------------------------------------------------------------------------
def test_group_psums_brute_force_python_ints():
    rng = np.random.default_rng(4)
    M, N, K = 3, 4, 192
    qx = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    P = O.group_psums(qx, qw)
    for m, n, g in itertools.product(range(M), range(N), range(K // 64)):
        s = 0
        for k in range(64 * g, 64 * g + 64):
            s += int(qx[m, k]) * int(qw[n, k])
        assert P[m, n, g] == s


def test_group_psums_extremes_basis_and_permutation():
    K = 256
    # extreme magnitude: all -8 gives 64*64 = 4096 per group
    P = O.group_psums(np.full((1, K), -8, np.int8), np.full((2, K), -8, np.int8))
    assert np.all(P == 4096)
    # basis probe: q_x = e_k selects q_w[:, k] in group k // 64
    rng = np.random.default_rng(5)
    qw = rng.integers(-8, 8, size=(5, K)).astype(np.int8)
    for k in (0, 63, 64, 200):
        e = np.zeros((1, K), np.int8)
        e[0, k] = 1
        P = O.group_psums(e, qw)
        want = np.zeros((1, 5, K // 64), np.int64)
        want[0, :, k // 64] = qw[:, k]
        assert np.array_equal(P, want)
    # permuting the 64-blocks of K in both operands permutes P along g
    qx = rng.integers(-8, 8, size=(3, K)).astype(np.int8)
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(64 * p, 64 * p + 64) for p in perm])
    assert np.array_equal(O.group_psums(qx[:, idx], qw[:, idx]), O.group_psums(qx, qw)[:, :, perm])


# ----------------------------------------------------------------------------
# Main term, LoRA, affine
# ----------------------------------------------------------------------------
def test_main_term_equals_dequantized_matmul():
    """sum_g s_x s_w P == (q_x s_x) @ (q_w s_w)^T (dequantized reference,
    'INT4 Kernel Architecture, in depth', per-layer validation)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((20, 320)).astype(np.float16)
    w = (rng.standard_normal((24, 320)) * 0.02).astype(np.float16)
    qx, sx = O.quantize_groups(x)
    qw, sw = O.quantize_groups(w)
    xh = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 64, axis=1)
    wh = qw.astype(np.float64) * np.repeat(sw.astype(np.float64), 64, axis=1)
    ref = xh @ wh.T
    got = O.main_term(qx, sx, qw, sw)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_integer_inputs_give_exact_plain_matmul():
    """With every group's absmax 7 the scales are 1 and the layer without
    LoRA is the plain integer product X W^T (computed with Python ints)."""
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 128
    x = rng.integers(-7, 8, size=(M, K)).astype(np.float64)
    w = rng.integers(-7, 8, size=(N, K)).astype(np.float64)
    x[:, 0] = 7.0
    x[:, 64] = -7.0
    w[:, 5] = 7.0
    w[:, 100] = 7.0
    out = O.linear(x.astype(np.float16), None, None, w16=w.astype(np.float16))
    for m in range(M):
        for n in range(N):
            assert out["main"][m, n] == sum(int(x[m, k]) * int(w[n, k]) for k in range(K))


def test_golden_layer():
    c = _load("layer_case.json")
    M, K, N, R = c["M"], c["K"], c["N"], c["R"]
    x = np.zeros((M, K), np.float16)
    for k, v in c["x_row0"]:
        x[0, k] = v
    w = np.zeros((N, K), np.float16)
    for n, ent in c["w"].items():
        for k, v in ent:
            w[int(n), k] = v
    ld = np.zeros((K, R), np.float16)
    for k, r, v in c["lora_down"]:
        ld[k, r] = v
    lu = np.zeros((N, R), np.float16)
    for n, r, v in c["lora_up"]:
        lu[n, r] = v
    out = O.linear(x, ld, lu, np.array(c["col_scale"], np.float32), np.array(c["bias"], np.float32), w16=w)
    e = c["expect"]
    assert out["sx"].astype(np.float64).tolist() == [e["sx"]]
    assert out["sw"].astype(np.float64).tolist() == e["sw"]
    nz = [[int(k), int(out["qx"][0, k])] for k in np.nonzero(out["qx"][0])[0]]
    assert nz == e["qx_nonzero"]
    assert O.group_psums(out["qx"], out["qw"]).tolist() == e["P"]
    assert out["main"].tolist() == e["main"]
    assert out["lora_act"].tolist() == e["lora_act"]
    assert out["lora"].tolist() == e["lora"]
    assert out["y"].astype(np.float64).tolist() == e["y"]


def _case(seed, M=6, K=256, N=10, R=16):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((M, K)).astype(np.float16),
        w=(rng.standard_normal((N, K)) * 0.02).astype(np.float16),
        ld=(rng.standard_normal((K, R)) * 0.02).astype(np.float16),
        lu=(rng.standard_normal((N, R)) * 0.02).astype(np.float16),
        a=rng.uniform(0.9, 1.1, N).astype(np.float32),
        b=(rng.standard_normal(N) * 0.01).astype(np.float32),
    )


def test_rank_zero_reduces_to_plain_w4a4():
    c = _case(8)
    full = O.linear(c["x"], c["ld"], np.zeros_like(c["lu"]), c["a"], c["b"], w16=c["w"])
    none = O.linear(c["x"], None, None, c["a"], c["b"], w16=c["w"])
    plain = O.to_fp16(c["a"].astype(np.float64) * none["main"] + c["b"].astype(np.float64))
    assert np.array_equal(_bits16(full["y"]), _bits16(plain))
    assert np.array_equal(_bits16(none["y"]), _bits16(plain))


def test_lora_associativity_and_one_hot():
    c = _case(9)
    out = O.linear(c["x"], c["ld"], c["lu"], w16=c["w"])
    assoc = c["x"].astype(np.float64) @ (c["ld"].astype(np.float64) @ c["lu"].astype(np.float64).T)
    assert np.allclose(out["lora"], assoc, rtol=0, atol=1e-12)
    # one-hot factors pick single entries: lora[m,n] = X[m,k] * L_up[n,r]
    K, R = c["ld"].shape
    ld = np.zeros((K, R), np.float16)
    ld[37, 3] = 1.0
    out = O.linear(c["x"], ld, c["lu"], w16=c["w"])
    want = c["x"][:, 37].astype(np.float64)[:, None] * c["lu"][:, 3].astype(np.float64)[None, :]
    assert np.array_equal(out["lora"], want)


def test_affine_identity_and_power_of_two_scale():
    c = _case(10)
    N = c["w"].shape[0]
    ident = O.linear(c["x"], c["ld"], c["lu"], np.ones(N, np.float32), np.zeros(N, np.float32), w16=c["w"])
    bare = O.linear(c["x"], c["ld"], c["lu"], w16=c["w"])
    assert np.array_equal(_bits16(ident["y"]), _bits16(O.to_fp16(bare["main"] + bare["lora"])))
    two = O.linear(c["x"], c["ld"], c["lu"], np.full(N, 2.0, np.float32), np.zeros(N, np.float32), w16=c["w"])
    assert np.array_equal(two["y"].astype(np.float64), 2.0 * ident["y"].astype(np.float64))
    # the bias is added once, after the scale
    bias = O.linear(c["x"], c["ld"], c["lu"], np.full(N, 2.0, np.float32), np.full(N, 0.5, np.float32), w16=c["w"])
    assert np.allclose(bias["y64"], two["y64"] + 0.5, rtol=0, atol=1e-12)


def test_whole_layer_brute_force_python():
    """Tiny layer evaluated entirely with Python ints/floats in loops."""
    c = _case(11, M=2, K=128, N=3, R=16)
    out = O.linear(c["x"], c["ld"], c["lu"], c["a"], c["b"], w16=c["w"])
    qx, sx, qw, sw = out["qx"], out["sx"], out["qw"], out["sw"]
    M, K = c["x"].shape
    N, R = c["lu"].shape
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for g in range(K // 64):
                p = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(64 * g, 64 * g + 64))
                acc += float(sx[m, g]) * float(sw[n, g]) * p
            lo = 0.0
            for r in range(R):
                la = sum(float(c["x"][m, k]) * float(c["ld"][k, r]) for k in range(K))
                lo += la * float(c["lu"][n, r])
            y = float(c["a"][n]) * (acc + lo) + float(c["b"][n])
            assert abs(out["y64"][m, n] - y) <= 1e-12 * max(1.0, abs(y))
            yh = struct.unpack("e", struct.pack("e", y))[0]
            assert abs(float(out["y"][m, n]) - yh) <= abs(yh) * 2 ** -10  # same fp16 or 1-ulp tie


# ----------------------------------------------------------------------------
# RMSNorm of the fused norm + quantize pass
# ----------------------------------------------------------------------------
def test_rmsnorm_constant_rows_closed_form():
    """A constant row c has mean square c^2, so with eps = 0 every output is
    sign(c) exactly (catches a sum in place of a mean, a missing square root,
    a sign slip); with eps > 0 it is c / sqrt(c^2 + eps)."""
    K = 256
    cs = np.array([1.0, -3.5, 0.015625, -1000.0, 2.0 ** -10], np.float16)
    x = np.repeat(cs[:, None], K, axis=1)
    ones = np.ones(K, np.float16)
    y = O.rms_norm(x, ones, 0.0)
    assert np.array_equal(y.astype(np.float64), np.sign(cs.astype(np.float64))[:, None] * np.ones((1, K)))
    eps = 0.25
    y = O.rms_norm(x, ones, eps).astype(np.float64)
    c64 = cs.astype(np.float64)
    expect = c64 / np.sqrt(c64 * c64 + eps)
    assert np.all(np.abs(y - expect[:, None]) <= 2.0 ** -10 * np.abs(expect[:, None]))


def test_rmsnorm_unit_mean_square():
    """With gamma = 1 and eps = 0 each output row has mean square 1 (up to
    the fp16 rounding of its elements): pins the normalizing axis and the
    1/sqrt."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 512)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float16)
    y = O.rms_norm(x, np.ones(512, np.float16), 0.0).astype(np.float64)
    ms = (y * y).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 2e-3), ms


def test_rmsnorm_gamma_scale_and_permutation():
    """gamma multiplies column k: a power-of-two gamma scales the output
    exactly, and permuting the columns of X together with gamma permutes the
    output (catches gamma indexed by row or left out).  With eps = 0,
    scaling X by 2^j leaves the output unchanged."""
    rng = np.random.default_rng(6)
    K = 384
    x = rng.standard_normal((5, K)).astype(np.float16)
    g = rng.uniform(0.5, 2.0, K).astype(np.float16)
    base = O.rms_norm(x, g, 1e-5)
    assert np.array_equal(_bits16(O.rms_norm(x, (g.astype(np.float64) * 4).astype(np.float16), 1e-5)),
                          _bits16((base.astype(np.float64) * 4).astype(np.float16)))
    perm = rng.permutation(K)
    assert np.array_equal(_bits16(O.rms_norm(x[:, perm], g[perm], 1e-5)), _bits16(base[:, perm]))
    assert np.array_equal(_bits16(O.rms_norm((x.astype(np.float64) * 8).astype(np.float16), g, 0.0)),
                          _bits16(O.rms_norm(x, g, 0.0)))
    # rows are independent
    assert np.array_equal(_bits16(O.rms_norm(x[2:3], g, 1e-5)), _bits16(base[2:3]))


def test_rmsnorm_matches_library_routine():
    """torch's own rms_norm in fp64 (x * rsqrt(mean(x^2) + eps) * weight),
    rounded the same way (fp32, then fp16), agrees to within one fp16 ulp
    everywhere and exactly almost everywhere (the two differ only in the last
    fp64 bit of the reciprocal square root)."""
    import torch
    rng = np.random.default_rng(7)
    M, K, eps = 12, 1024, 1e-6
    x = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    g = rng.uniform(0.2, 3.0, K).astype(np.float16)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (K,),
                                       weight=torch.from_numpy(g.astype(np.float64)), eps=eps)
    ref16 = ref.numpy().astype(np.float32).astype(np.float16)
    got = O.rms_norm(x, g, eps)
    d = np.abs(_bits16(got).astype(np.int32) - _bits16(ref16).astype(np.int32))
    assert d.max() <= 1
    assert (d == 0).mean() > 0.999


def test_quantize_act_rmsnorm_is_norm_then_quantize():
    """The fused pass is exactly the quantizer and LoRA-down applied to the
    normalized fp16 rows."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((7, 256)).astype(np.float16)
    g = rng.uniform(0.5, 1.5, 256).astype(np.float16)
    ld = (rng.standard_normal((256, 16)) * 0.02).astype(np.float16)
    xn, qx, sx, la = O.quantize_act_rmsnorm(x, g, 1e-6, ld)
    qx2, sx2, la2 = O.quantize_act(O.rms_norm(x, g, 1e-6), ld)
    assert np.array_equal(qx, qx2) and np.array_equal(_bits16(sx), _bits16(sx2)) and np.array_equal(la, la2)
    # and the quantizer saw the normalized values: |xn - q*s| <= s/2 per group
    deq = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(xn.astype(np.float64) - deq) <= np.repeat(sx.astype(np.float64), 64, axis=1) / 2)


# ----------------------------------------------------------------------------
# MLP gated activation
# ----------------------------------------------------------------------------
def test_silu_closed_forms_and_identity():
    """SiLU(0) = 0; SiLU(v) - SiLU(-v) = v (odd part is v/2, catches a sign
    slip in the exponent); SiLU(v) -> v for large v and -> 0 for very negative
    v; SiLU(ln 3) = ln 3 * 3/4 exactly in the reals."""
    assert O.silu(0.0) == 0.0
    v = np.linspace(-12, 12, 97)
    assert np.allclose(O.silu(v) - O.silu(-v), v, rtol=0, atol=1e-12)
    assert abs(O.silu(40.0) - 40.0) < 1e-12 and abs(O.silu(-40.0)) < 1e-15
    assert abs(O.silu(np.log(3.0)) - np.log(3.0) * 0.75) < 1e-15


def test_glu_rounding_and_zeros():
    """h = fp16(SiLU(g) * u): u = 0 or g = 0 gives 0, u = 1 gives fp16(SiLU(g)),
    and the product is taken in fp64 and rounded once."""
    g = np.array([0.0, 1.5, -2.25, 7.0, 0.3330078125], np.float16)
    assert not np.any(O.glu(g, np.zeros(5, np.float16)).astype(np.float64))
    assert O.glu(np.zeros(5, np.float16), np.full(5, 3.0, np.float16)).astype(np.float64).sum() == 0
    s64 = g.astype(np.float64) / (1 + np.exp(-g.astype(np.float64)))
    assert np.array_equal(O.glu(g, np.ones(5, np.float16)), s64.astype(np.float16))
    u = np.full(5, 1.0009765625, np.float16)   # 1 + 2^-10
    assert np.array_equal(O.glu(g, u), (s64 * float(u[0])).astype(np.float16))


def test_mlp_gate_up_wiring():
    """The gate/up pair feeds the gate output to SiLU and multiplies by the
    up output, not the other way round: with an up projection that is
    exactly 1 (zero weights, no LoRA, bias 1) h equals fp16(SiLU(g)), and
    with a gate projection that is exactly 0 (bias 0) h is 0 whatever u is."""
    rng = np.random.default_rng(77)
    M, K, N = 5, 128, 16
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.1).astype(np.float16)
    zero_w = np.zeros((N, K), np.float16)
    gate = dict(lora_down16=None, lora_up16=None, w16=w)
    one = dict(lora_down16=None, lora_up16=None, w16=zero_w, bias=np.ones(N, np.float32))
    g, u, h = O.mlp_gate_up(x, gate, one)
    assert np.all(u.astype(np.float64) == 1.0)
    gd = g.astype(np.float64)
    assert np.array_equal(_bits16(h), _bits16((gd / (1.0 + np.exp(-gd))).astype(np.float16)))
    # swapped roles would give SiLU(1) * g, which differs here
    assert not np.array_equal(_bits16(h), _bits16((gd * (1.0 / (1.0 + np.exp(-1.0)))).astype(np.float16)))
    zero = dict(lora_down16=None, lora_up16=None, w16=zero_w, bias=np.zeros(N, np.float32))
    _, _, h0 = O.mlp_gate_up(x, zero, gate)
    assert not np.any(h0.astype(np.float64))


def test_linear_on_index_subsets_equals_full_evaluation_restricted():
    """linear(rows=, cols=) (each row of X and of W is quantized on its own, so
    a subset evaluates the same definition) against the full evaluation taken
    at the same indices, for fp16 W and for checkpoint codes: codes, scales,
    group sums' main term and Y identical; lora_act / LoRA / the fp64 output
    equal up to the summation order of the library matrix product (a shape-
    dependent blocking), i.e. within a few fp64 ulps."""
    rng = np.random.default_rng(5)
    for use_q in (False, True):
        c = workloads.random_case(40, 512, 96, 32, seed=77 + use_q)
        kw = dict(w16=c["w"])
        if use_q:
            q = rng.integers(-8, 8, size=(96, 512))
            nib = (q & 0xF).astype(np.uint8)
            kw = dict(qweight=(nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8),
                      w_scales=rng.uniform(1e-3, 1e-2, (96, 8)).astype(np.float16))
        full = O.linear(c["x"], c["lora_down"], c["lora_up"], c["col_scale"], c["bias"], **kw)
        rows = np.sort(rng.choice(40, 9, replace=False))
        cols = np.sort(rng.choice(96, 13, replace=False))
        sub = O.linear(c["x"], c["lora_down"], c["lora_up"], c["col_scale"], c["bias"], rows=rows, cols=cols, **kw)
        for k in ("qx", "sx"):
            assert np.array_equal(sub[k], full[k][rows]), k
        for k in ("qw", "sw"):
            assert np.array_equal(sub[k], full[k][cols]), k
        for k in ("main", "y"):
            assert np.array_equal(sub[k], full[k][np.ix_(rows, cols)]), k
        np.testing.assert_allclose(sub["lora_act"], full["lora_act"][rows], rtol=1e-13, atol=1e-15)
        for k in ("lora", "y64"):
            ref = full[k][np.ix_(rows, cols)]
            assert np.max(np.abs(sub[k] - ref)) <= 1e-13 * np.max(np.abs(ref)), k
