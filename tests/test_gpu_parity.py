"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed codes, scales and per-group integer sums bit-exact; lora_act
within 1e-4 * rms; Y within max|dY| <= 2e-2 * rms(Y_oracle) and
mean|dY| <= 2e-3 * rms(Y_oracle), rms over every compared output; an output
beyond the max bar passes only as the other correct fp16 rounding of a near
tie (tests/parity_bar.py).  Every workload is compared output by output,
the largest (M=8192, K=N=4096) too.
"""
import json
import os
import sys

import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from oracle import w4a4_oracle as O
from tests.layout_unpack import split_act_blob, split_weight_blob
from tests.parity_bar import MAX_TOL, MEAN_TOL, check_y, kernel_error_bound

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_y(y_gpu, y_ref, what, y64=None, ref=None, case=None, rows=None):
    """The layer bar (tests/parity_bar.py); with the oracle's dict `ref` (and
    the case's affine and L_up) near-tie roundings are judged against the
    kernel's error bound.  rows: the rows of ref that y_gpu's rows are."""
    bound = None
    if ref is not None:
        inner = kernel_error_bound(ref["qx"], ref["sx"], ref["qw"], ref["sw"], ref["lora_act"],
                                   case.get("lora_up"), case.get("col_scale"), case.get("bias"))
        rmap = np.arange(ref["qx"].shape[0]) if rows is None else np.asarray(rows)
        bound = lambda r, c: inner(rmap[r], c)
    check_y(y_gpu, y_ref, what, y64=y64, err_bound=bound, say=_say)


def _to_dev(a):
    torch = _torch()
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class GpuLayerRun:
    """Pack, quantize and run one layer on the GPU; keep host copies."""

    def __init__(self, case, use_qweight=False, ldx=None, ldy=None, R=None, norm=None):
        torch = _torch()
        self.M, self.K, self.N = case["M"], case["K"], case["N"]
        self.R = case["R"] if R is None else R
        M, K, N, R = self.M, self.K, self.N, self.R
        self.ldx = K if ldx is None else ldx
        self.ldy = N if ldy is None else ldy
        self.wblob = W.alloc_weight_blob(N, K, R)
        self.wblob.fill_(0xA5)   # garbage: every byte the packer owns must be written
        kw = dict(lora_down=_to_dev(case["lora_down"]) if R else None,
                  lora_up=_to_dev(case["lora_up"]) if R else None,
                  col_scale=_to_dev(case.get("col_scale")), bias=_to_dev(case.get("bias")))
        if use_qweight:
            W.w4a4_pack_weights(N, K, R, self.wblob, qweight=_to_dev(case["qweight"]),
                                w_scales=_to_dev(case["w_scales"]), **kw)
        else:
            W.w4a4_pack_weights(N, K, R, self.wblob, w_fp16=_to_dev(case["w"]), **kw)
        xs = np.zeros((max(M, 1), self.ldx), np.float16)
        xs[:M, :K] = case["x"]
        self.x = _to_dev(xs)
        self.act = W.alloc_act_blob(M, K, R)
        self.act.fill_(0x5A)
        if norm is None:
            W.w4a4_quantize_act(M, K, R, self.x, self.wblob, self.act, ldx=self.ldx)
        else:   # (gamma fp16 [K], eps): the fused RMSNorm + quantize pass
            self.gamma = _to_dev(norm[0])
            W.w4a4_quantize_act_rmsnorm(M, K, R, self.x, self.gamma, norm[1], self.wblob, self.act,
                                        ldx=self.ldx)
        self.y = torch.full((max(M, 1), self.ldy), float("nan"), dtype=torch.float16, device="cuda")
        W.w4a4_linear(M, N, K, R, self.act, self.wblob, self.y, ldy=self.ldy)
        torch.cuda.synchronize()

    def host_act(self):
        _, offs, ks = W.w4a4_act_layout(self.M, self.K, self.R, with_splits=True)
        return split_act_blob(self.act.cpu().numpy(), self.M, self.K, self.R, offs, ks)

    def host_weights(self):
        _, offs = W.w4a4_weight_layout(self.N, self.K, self.R)
        return split_weight_blob(self.wblob.cpu().numpy(), self.N, self.K, self.R, offs)

    def host_y(self):
        return self.y.cpu().numpy()

    def psums(self, m0, mc, n0, nc):
        torch = _torch()
        out = torch.zeros((mc, nc, self.K // 64), dtype=torch.int32, device="cuda")
        W.w4a4_debug_group_psums(self.M, self.N, self.K, self.R, self.act, self.wblob, m0, mc, n0, nc, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def _check_quant(run, case, ref_qx, ref_sx):
    a = run.host_act()
    M = run.M
    assert np.array_equal(a["qx"][:M], ref_qx), "X codes differ"
    assert np.array_equal(a["sx"][:M].view(np.uint16), ref_sx.view(np.uint16)), "X scales differ"
    assert not np.any(a["qx"][M:]) and not np.any(a["sx"][M:].view(np.uint16)), "padding rows not zero"
    return a


def _check_weights(run, case, ref_qw, ref_sw):
    w = run.host_weights()
    assert np.array_equal(w["qw"], ref_qw), "W codes differ"
    assert np.array_equal(w["sw"].view(np.uint16), ref_sw.view(np.uint16)), "W scales differ"
    if run.R:
        assert np.array_equal(w["lora_down"].view(np.uint16), case["lora_down"].view(np.uint16))
        assert np.array_equal(w["lora_up"].view(np.uint16), case["lora_up"].view(np.uint16))
    a_ref = case["col_scale"] if case.get("col_scale") is not None else np.ones(run.N, np.float32)
    b_ref = case["bias"] if case.get("bias") is not None else np.zeros(run.N, np.float32)
    assert np.array_equal(w["a"], a_ref) and np.array_equal(w["b"], b_ref)
    return w


def _check_lora_act(a, ref_la, M):
    """lora_act (the in-order sum of the partials) within 1e-4 * rms of the
    oracle; every partial's padding rows are zero."""
    if ref_la is None or ref_la.shape[1] == 0:
        return
    got = a["lora_act"][:M].astype(np.float64)
    rms = np.sqrt(np.mean(ref_la ** 2)) + 1e-30
    d = np.abs(got - ref_la).max()
    _say(f"lora_act max|d|/rms = {d / rms:.3g} (partials: {a['lora_parts'].shape[0]})")
    assert d <= 1e-4 * rms
    assert not np.any(a["lora_parts"][:, M:]), "padding lora_act rows not zero"


# ---------------------------------------------------------------------------
def test_quantizer_golden_groups_on_gpu():
    cases = json.load(open(os.path.join(GOLDEN, "quantize_cases.json")))["groups"]
    K = 128
    x = np.zeros((len(cases), K), np.float16)
    want_q = np.zeros((len(cases), K), np.int8)
    for i, c in enumerate(cases):
        x[i, : len(c["x"])] = c["x"]
        want_q[i, : len(c["q"])] = c["q"]
        # second group: the same values negated
        x[i, 64: 64 + len(c["x"])] = -np.array(c["x"], np.float16)
    torch = _torch()
    M = len(cases)
    act = W.alloc_act_blob(M, K, 0)
    W.w4a4_quantize_act(M, K, 0, _to_dev(x), None, act)
    torch.cuda.synchronize()
    _, offs = W.w4a4_act_layout(M, K, 0)
    a = split_act_blob(act.cpu().numpy(), M, K, 0, offs)
    for i, c in enumerate(cases):
        assert a["qx"][i, :64].tolist() == want_q[i, :64].tolist(), c["name"]
        assert int(a["sx"][i, 0].view(np.uint16)) == c["s_bits"], c["name"]
        assert int(a["sx"][i, 1].view(np.uint16)) == c["s_bits"], c["name"]
    # the negated group matches the oracle (the clamp makes -x asymmetric at +-8.5)
    qx, sx = O.quantize_groups(x)
    assert np.array_equal(a["qx"][:M], qx)


def _every_quotient_groups():
    """fp16 rows whose 64-groups put every fp16 x against many scales: each
    group holds its absmax A first (so s = fp16(A / 7)) and then 63 values
    taken in order, with alternating signs, from every fp16 value in
    [A / 28, A] (smaller values quantize to 0).  A runs over every fp16 value
    in [7, 14) (s over [1, 2)) and every 16th one below 7 * 2^-14 (subnormal
    scales, from the 2^-24 floor up)."""
    allv = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    a_norm = allv[(allv >= 7) & (allv < 14)]
    a_sub = allv[allv < np.float16(7 * 2.0 ** -14)][::16]
    groups = []
    for A in np.concatenate([a_norm, a_sub]):
        x = allv[(allv >= np.float16(A / 28)) & (allv <= A)]
        x = np.where(np.arange(x.size) % 2 == 1, -x, x).astype(np.float16)
        n = -(-x.size // 63)
        body = np.zeros(n * 63, np.float16)
        body[: x.size] = x
        g = np.empty((n, 64), np.float16)
        g[:, 0] = A
        g[:, 1:] = body.reshape(n, 63)
        groups.append(g)
    return np.concatenate(groups)


def test_quantizer_every_quotient_on_gpu():
    """Codes and scales bit-exact against the oracle's IEEE-division
    quantizer over every fp16 value against ~1500 scales: the activation
    pass divides by no scale (one Newton step from the hardware reciprocal
    gives the quotient), and ties, the clamp at -8 (A's negated neighbours
    never reach it, the subnormal scales do) and the 2^-24 floor must come
    out as the rule has them."""
    g = _every_quotient_groups()
    K = 4096
    M = -(-g.shape[0] // (K // 64))
    x = np.zeros((M * (K // 64), 64), np.float16)
    x[: g.shape[0]] = g
    x = x.reshape(M, K)
    _say(f"[quant] every quotient: {g.shape[0]} groups, M={M} K={K}")
    torch = _torch()
    act = W.alloc_act_blob(M, K, 0)
    W.w4a4_quantize_act(M, K, 0, _to_dev(x), None, act)
    torch.cuda.synchronize()
    _, offs = W.w4a4_act_layout(M, K, 0)
    a = split_act_blob(act.cpu().numpy(), M, K, 0, offs)
    qx, sx = O.quantize_groups(x)
    assert np.array_equal(a["sx"][:M].view(np.uint16), sx.view(np.uint16))
    bad = np.argwhere(a["qx"][:M] != qx)
    assert bad.size == 0, (f"{len(bad)} codes differ, first at {bad[:3].tolist()}: x="
                           f"{[float(x[r, c]) for r, c in bad[:3]]}")


WORKLOAD_CASES = ["small", "mlp_up", "mlp_down", "decode-1", "decode-2", "decode-3", "decode-4", "decode-8", "decode-13",
                  "decode-16"]


def _workload(name):
    if name.startswith("decode-"):
        return workloads.generate("decode", M=int(name.split("-")[1]))
    return workloads.generate(name)


@pytest.mark.parametrize("name", WORKLOAD_CASES)
def test_workload_parity_full_output(name):
    case = _workload(name)
    _say(f"[parity] {name} M={case['M']} K={case['K']} N={case['N']} R={case['R']}")
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    a = _check_quant(run, case, ref["qx"], ref["sx"])
    _check_weights(run, case, ref["qw"], ref["sw"])
    _check_lora_act(a, ref["lora_act"], run.M)
    _check_y(run.host_y()[: run.M, : run.N], ref["y"], name, y64=ref["y64"], ref=ref, case=case)
    # exact per-group integer sums: whole output for the small case, windows otherwise
    Mp = (run.M + 15) // 16 * 16
    if name == "small":
        wins = [(0, Mp, 0, run.N)]
    else:
        wins = [(0, 16, 0, 32), (Mp - 16, 16, run.N - 48, 48), (Mp // 32 * 16, 16, run.N // 32 * 16, 64)]
    for m0, mc, n0, nc in wins:
        got = run.psums(m0, mc, n0, nc)
        rows = np.arange(m0, min(m0 + mc, run.M))
        P = O.group_psums(ref["qx"][rows], ref["qw"][n0: n0 + nc])
        assert np.array_equal(got[: len(rows)], P), (name, m0, n0)
        assert not np.any(got[len(rows):]), "psums of padding rows must be 0"


def test_prefill_parity_full():
    """The largest workload compared in full: codes and scales of all of X
    and W bit-exact, every one of the M x N outputs against the oracle
    (evaluated in row chunks; each row of X is quantized on its own, so a
    chunk is the same definition), the bar's rms taken over all of them, and
    four 128 x 128 windows of group sums (corners, the last tile, an interior
    one) bit-exact."""
    case = workloads.generate("prefill")
    M, K, N = case["M"], case["K"], case["N"]
    _say(f"[parity] prefill M={M} K={K} N={N} R={case['R']}")
    run = GpuLayerRun(case)
    qx, sx = O.quantize_groups(case["x"])
    qw, sw = O.quantize_groups(case["w"])
    a = _check_quant(run, case, qx, sx)
    _check_weights(run, case, qw, sw)
    y = run.host_y()[:M, :N]
    ref = np.empty((M, N), np.float16)
    ref64 = np.empty((M, N))
    la = np.empty((M, case["R"]))
    chunk = 1024
    for r0 in range(0, M, chunk):
        rows = np.arange(r0, min(r0 + chunk, M))
        part = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"],
                        w16=case["w"], rows=rows)
        ref[rows] = part["y"]
        ref64[rows] = part["y64"]
        la[rows] = part["lora_act"]
        _say(f"[parity] prefill oracle rows {r0}..{rows[-1]}")
    _check_lora_act(a, la, M)
    full = dict(qx=qx, sx=sx, qw=qw, sw=sw, lora_act=la)
    _check_y(y, ref, "prefill (all outputs)", y64=ref64, ref=full, case=case)
    for m0, n0 in [(0, 0), (M - 128, N - 128), (4096, 2048), (M - 128, 0)]:
        got = run.psums(m0, 128, n0, 128)
        assert np.array_equal(got, O.group_psums(qx[m0: m0 + 128], qw[n0: n0 + 128])), (m0, n0)


@pytest.mark.parametrize("M,K,N,R", [(1, 128, 16, 16), (17, 128, 48, 0), (33, 256, 64, 64),
                                     (5, 384, 32, 48), (130, 512, 80, 32), (40, 8192, 48, 32),
                                     (40, 8192, 48, 64), (3, 16384, 32, 16)])
def test_ragged_and_rank_edges(M, K, N, R):
    """Ragged M, every rank, and the quantizer's wave counts: K = 8192 at
    M = 40 splits K four ways with 16 k-pairs per workgroup (16 waves at
    rank 32, 8 at rank 64), K = 16384 at M = 3 eight ways (16 waves)."""
    case = workloads.random_case(M, K, N, R, seed=1000 + M + K + R)
    _say(f"[edge] M={M} K={K} N={N} R={R}")
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"] if R else None, case["lora_up"] if R else None,
                   case["col_scale"], case["bias"], w16=case["w"])
    a = _check_quant(run, case, ref["qx"], ref["sx"])
    _check_weights(run, case, ref["qw"], ref["sw"])
    _check_lora_act(a, ref["lora_act"], M)
    _check_y(run.host_y()[:M, :N], ref["y"], f"edge M={M} R={R}", y64=ref["y64"], ref=ref, case=case)
    Mp = (M + 15) // 16 * 16
    got = run.psums(0, Mp, 0, N)
    assert np.array_equal(got[:M], O.group_psums(ref["qx"], ref["qw"]))
    # rows >= M of y are never written
    assert np.all(np.isnan(run.host_y()[M:].astype(np.float64)))


@pytest.mark.parametrize("M,K,N,R", [(1, 128, 48, 0), (2, 384, 32, 64), (1, 1664, 64, 48),
                                     (2, 4864, 48, 32), (1, 4864, 16, 64), (2, 1664, 48, 16),
                                     (3, 1664, 32, 32), (3, 4864, 32, 48), (4, 1664, 32, 64),
                                     (4, 4864, 48, 16), (4, 384, 16, 0), (8, 1664, 32, 32),
                                     (13, 4864, 48, 64), (6, 1664, 8192, 48), (11, 384, 8192, 0),
                                     (16, 4864, 8192, 16), (9, 1664, 8192, 64), (1, 1664, 8192, 48),
                                     (2, 384, 8192, 0), (3, 4864, 8192, 64), (4, 1664, 8192, 16),
                                     (4, 4864, 8192, 64), (1, 8192, 4096, 32), (16, 8192, 4096, 64),
                                     (4, 16384, 2048, 16), (7, 8320, 1024, 48)])
def test_small_m_decode_shapes(M, K, N, R):
    """M <= 16 kernels over uneven per-wave k-pair ranges (a wave with no
    k-pairs, ranges that are not a multiple of the batch), every rank, and
    groups whose scales differ by 16x between odd and even groups, so a
    group / scale mispairing cannot hide inside the tolerance.  N = 8192
    (512 column tiles) takes the two-column-tiles-per-workgroup paths: the
    dot kernel (M <= 3, every rank) and the MFMA decode kernel (M >= 4,
    R <= 48; R = 64 keeps one tile); at N = 8192 M = 4 runs the MFMA decode
    kernel, at narrower N the dot kernel.  K >= 8192 with at most 256
    workgroups (N <= 4096) takes the 8-wave workgroups, whose waves split K
    eight ways (K = 8320: 65 k-pairs, a ragged split)."""
    case = workloads.random_case(M, K, N, R, seed=2000 + M + K + R)
    x = case["x"].astype(np.float64)
    x[:, (np.arange(K) // 64) % 2 == 1] *= 16.0
    case["x"] = x.astype(np.float16)
    w = case["w"].astype(np.float64)
    w[:, (np.arange(K) // 64) % 3 == 2] *= 0.125
    case["w"] = w.astype(np.float16)
    _say(f"[decode-shape] M={M} K={K} N={N} R={R}")
    assert W.w4a4_query_variant(M, N, K, R) == 1
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"] if R else None, case["lora_up"] if R else None,
                   case["col_scale"], case["bias"], w16=case["w"])
    a = _check_quant(run, case, ref["qx"], ref["sx"])
    _check_lora_act(a, ref["lora_act"], M)
    _check_y(run.host_y()[:M, :N], ref["y"], f"decode shape M={M} K={K} R={R}", y64=ref["y64"], ref=ref, case=case)
    assert np.all(np.isnan(run.host_y()[M:].astype(np.float64)))


@pytest.mark.parametrize("cfg,K,R", [(c, 512, 32) for c in range(10)] + [(c, 2048, 32) for c in range(10)] +
                         [(c, 2048, 64) for c in range(10)])
def test_every_tile_shape(cfg, K, R, monkeypatch):
    """Each M > 16 tile shape (forced) on a shape with ragged row and column
    edges for all of them: M = 130 (9 row tiles), N = 208 (13 column tiles);
    K = 512 gives one lora_act partial, K = 2048 two: shapes whose waves
    cannot hold every partial through the K loop (row tiles x rank blocks x
    4 > 16, e.g. all of them at rank 64 but the one-row-tile ones) load and
    sum them in the epilogue instead."""
    M, N = 130, 208
    _, _, ks = W.w4a4_act_layout(M, K, R, with_splits=True)
    assert ks == (1 if K == 512 else 2)
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    case = workloads.random_case(M, K, N, R, seed=3000 + cfg + K + R)
    _say(f"[tile shape {cfg}] M={M} K={K} N={N} R={R} partials={ks}")
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"tile shape {cfg}", y64=ref["y64"], ref=ref, case=case)
    assert np.all(np.isnan(run.host_y()[M:].astype(np.float64)))


@pytest.mark.parametrize("cfg,K,R", [(c, K, R) for c in (0, 1, 2, 3, 5, 8) for K, R in ((512, 32), (2048, 64))])
def test_every_lean_tile_shape(cfg, K, R, monkeypatch):
    """The lean variant (3 workgroups per CU: 3-deep LDS ring, epilogue
    operands and lora_act partials loaded after the K loop, tile-by-tile
    loop body) of each tile shape that has one, forced, on the ragged shape
    of the test above, with one and with two lora_act partials."""
    M, N = 130, 208
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    monkeypatch.setenv("W4A4_TILED_LEAN", "1")
    case = workloads.random_case(M, K, N, R, seed=3500 + cfg + K + R)
    _say(f"[lean tile shape {cfg}] M={M} K={K} N={N} R={R}")
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"lean tile shape {cfg}", y64=ref["y64"], ref=ref, case=case)
    assert np.all(np.isnan(run.host_y()[M:].astype(np.float64)))


@pytest.mark.parametrize("cfg,R", [(c, R) for c in (3, 4, 5, 7, 8) for R in (32, 64)])
def test_every_k_split_tile_shape(cfg, R, monkeypatch):
    """The K-split variant (two sets of waves over the two halves of K, the
    second's accumulators added to the first's in LDS) of each tile shape
    that has one, forced, on the ragged shape above with K = 2560 (20
    k-pairs, 10 per half; two lora_act partials)."""
    M, N, K = 130, 208, 2560
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    monkeypatch.setenv("W4A4_TILED_LEAN", "0")
    monkeypatch.setenv("W4A4_TILED_KSPLIT", "1")
    case = workloads.random_case(M, K, N, R, seed=3700 + cfg + R)
    _say(f"[k-split tile shape {cfg}] M={M} K={K} N={N} R={R}")
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"k-split tile shape {cfg}", y64=ref["y64"], ref=ref, case=case)
    assert np.all(np.isnan(run.host_y()[M:].astype(np.float64)))


def test_strided_x_and_y():
    M, K, N, R = 40, 256, 64, 32
    case = workloads.random_case(M, K, N, R, seed=7)
    run = GpuLayerRun(case, ldx=K + 64, ldy=N + 24)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_quant(run, case, ref["qx"], ref["sx"])
    y = run.host_y()
    _check_y(y[:, :N], ref["y"], "strided", y64=ref["y64"], ref=ref, case=case)
    assert np.all(np.isnan(y[:, N:].astype(np.float64))), "columns beyond N were written"


def test_checkpoint_codes_with_minus_eight():
    """qweight/w_scales input (checkpoint layout), codes spanning -8..7."""
    M, K, N, R = 24, 256, 32, 16
    case = workloads.random_case(M, K, N, R, seed=11)
    rng = np.random.default_rng(12)
    q = rng.integers(-8, 8, size=(N, K))
    q[0, :] = -8
    nib = (q & 0xF).astype(np.uint8)
    case["qweight"] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    case["w_scales"] = (rng.uniform(0.001, 0.01, size=(N, K // 64))).astype(np.float16)
    run = GpuLayerRun(case, use_qweight=True)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"],
                   qweight=case["qweight"], w_scales=case["w_scales"])
    assert np.array_equal(ref["qw"], q.astype(np.int8))
    _check_weights(run, case, ref["qw"], ref["sw"])
    _check_y(run.host_y()[:M], ref["y"], "checkpoint codes", y64=ref["y64"], ref=ref, case=case)
    got = run.psums(0, 32, 0, N)
    assert np.array_equal(got[:M], O.group_psums(ref["qx"], ref["qw"]))


def test_extreme_rows_and_determinism():
    """Zero rows, huge-magnitude rows, subnormal rows; two runs bit-identical."""
    M, K, N, R = 48, 256, 64, 16
    case = workloads.random_case(M, K, N, R, seed=13)
    x = case["x"].astype(np.float64)
    x[3] = 0.0
    x[4] *= 8000.0
    x[5] *= 2.0 ** -20
    x[6, :64] = 0.0
    x[7] = np.where(np.arange(K) % 64 == 0, 60000.0, x[7])
    case["x"] = np.clip(x, -65504, 65504).astype(np.float16)
    case["lora_down"] = (case["lora_down"].astype(np.float64) * 1e-3).astype(np.float16)
    run = GpuLayerRun(case)
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_quant(run, case, ref["qx"], ref["sx"])
    y1 = run.host_y().copy()
    W.w4a4_quantize_act(M, K, R, run.x, run.wblob, run.act)
    W.w4a4_linear(M, N, K, R, run.act, run.wblob, run.y)
    _torch().cuda.synchronize()
    assert np.array_equal(y1.view(np.uint16), run.host_y().view(np.uint16))
    ok = np.ones(M, bool)
    ok[4] = ok[7] = False    # outliers dominate the rms; checked separately below
    _check_y(y1[ok], ref["y"][ok], "extreme rows (ordinary)", y64=ref["y64"][ok], ref=ref, case=case,
             rows=np.flatnonzero(ok))
    for r in (4, 7):
        _check_y(y1[r: r + 1], ref["y"][r: r + 1], f"extreme row {r}", y64=ref["y64"][r: r + 1], ref=ref,
                 case=case, rows=[r])


def test_zero_rows_is_noop():
    torch = _torch()
    W.w4a4_quantize_act(0, 128, 16, None, None, None)
    W.w4a4_linear(0, 16, 128, 16, None, None, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,N,R,eps", [(1, 4096, 64, 32, 1e-6), (3, 1664, 48, 16, 1e-5),
                                         (16, 4096, 32, 32, 1e-6), (13, 384, 32, 0, 1e-6),
                                         (40, 1024, 64, 64, 1e-6), (130, 3072, 48, 48, 1e-6),
                                         (700, 1024, 96, 32, 1e-6), (40, 8192, 64, 32, 1e-6),
                                         (40, 8192, 64, 16, 1e-6)])
def test_rmsnorm_quantize(M, K, N, R, eps):
    """The fused RMSNorm + quantize pass against the oracle's norm-then-
    quantize: codes and scales bit-exact, lora_act within 1e-4 * rms, and the
    layer output within the usual tolerance.  Rows get magnitudes spread
    over 1e-2..1e2 and gamma varies per column, so a norm taken over the
    wrong rows, a K split that misses part of the row (M <= 16 splits K over
    workgroups) or a gamma indexed by row would change codes.  K = 8192 at
    M = 40 gives workgroups 16 k-pairs each: rank 16 runs 16 waves per
    workgroup, rank 32 eight (its 16-wave instance would not fit its
    registers beside the norm's state)."""
    rng = np.random.default_rng(4000 + M + K + R)
    case = workloads.random_case(M, K, N, R, seed=4100 + M + K + R)
    x = case["x"].astype(np.float64) * (10.0 ** rng.uniform(-2, 2, (M, 1)))
    x[:, rng.choice(K, size=4, replace=False)] *= 20.0
    case["x"] = x.astype(np.float16)
    gamma = rng.uniform(0.25, 2.0, K).astype(np.float16)
    _say(f"[rmsnorm] M={M} K={K} N={N} R={R} eps={eps}")
    run = GpuLayerRun(case, norm=(gamma, eps))
    xn, qx, sx, la = O.quantize_act_rmsnorm(case["x"], gamma, eps, case["lora_down"] if R else None)
    a = _check_quant(run, case, qx, sx)
    _check_lora_act(a, la, M)
    ref = O.linear(xn, case["lora_down"] if R else None, case["lora_up"] if R else None,
                   case["col_scale"], case["bias"], w16=case["w"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"rmsnorm M={M} K={K} R={R}", y64=ref["y64"], ref=ref, case=case)


def _double_rounding_rows(M=64, K=8192, eps=1e-6, seed=4300):
    """RMSNorm inputs that expose a one-step fp64 -> fp16 conversion: each
    64-group of row r has one dominant element (|x| in [2, 8], at column
    64 G + r; the rest in [2^-4, 2^-2]), and each column's gamma is picked,
    where one exists in [0.5, 2), so that the element's normalized value t =
    (x inv) gamma rounds to a different fp16 directly than through fp32 --
    the group's scale then shows which rounding the kernel took.  Every
    |x| >= 2^-4 makes the row's sum of squares exact in any order, so the
    kernel's inv is the oracle's."""
    rng = np.random.default_rng(seed)
    G = K // 64
    x = (rng.uniform(2.0 ** -4, 2.0 ** -2, (M, K)) * rng.choice([-1.0, 1.0], (M, K))).astype(np.float16)
    rows = np.arange(M)[:, None]
    tcol = np.arange(G)[None, :] * 64 + rows % 64
    x[rows, tcol] = (rng.uniform(2.0, 8.0, (M, G)) * rng.choice([-1.0, 1.0], (M, G))).astype(np.float16)
    xd = x.astype(np.float64)
    inv = 1.0 / np.sqrt((xd * xd).sum(axis=1) / K + eps)
    gamma = rng.uniform(0.5, 2.0, K).astype(np.float16)
    cand = np.arange(0x3800, 0x4000, dtype=np.uint16).view(np.float16)
    k = np.arange(K)
    base = xd[k % 64, k] * inv[k % 64]                              # x * inv, first rounding
    t = base[:, None] * cand.astype(np.float64)[None, :]            # times gamma, second
    hit = t.astype(np.float32).astype(np.float16) != t.astype(np.float16)
    first = np.argmax(hit, axis=1)
    has = hit[k, first]
    gamma[has] = cand[first[has]]
    return x, gamma, eps, int(has.sum())


def test_rmsnorm_fp32_step_of_the_fp16_conversion():
    """The normalized value is fp16(fp32(t)), two roundings: on inputs built
    so that ~1000 group maxima round differently in one step
    (_double_rounding_rows), codes and scales stay bit-exact.  The same
    check on the CPU shows that a one-step conversion changes many scales,
    so the test can tell the two apart."""
    M, K, N, R = 64, 8192, 64, 16
    x, gamma, eps, hits = _double_rounding_rows(M, K)
    case = workloads.random_case(M, K, N, R, seed=4301)
    case["x"] = x
    xn, qx, sx, la = O.quantize_act_rmsnorm(x, gamma, eps, case["lora_down"])
    xd = x.astype(np.float64)
    t = (xd * (1.0 / np.sqrt((xd * xd).sum(axis=1) / K + eps))[:, None]) * gamma.astype(np.float64)[None, :]
    _, sx_one_step = O.quantize_groups(t.astype(np.float16))
    changed = int(np.sum(sx_one_step.view(np.uint16) != sx.view(np.uint16)))
    _say(f"[rmsnorm double rounding] M={M} K={K}: {hits} targeted maxima, {changed} scales differ in one step")
    assert hits > 400 and changed > 100
    run = GpuLayerRun(case, norm=(gamma, eps))
    a = _check_quant(run, case, qx, sx)
    _check_lora_act(a, la, M)


# Activation-pass launch shapes (M, K, R, RMSNorm): the pass splits K into
# ks ranges (the library's act layout reports ks), gives each workgroup
# NW = 16, 8, 4 or 2 waves by its k-pairs (16 only with < 256 workgroups and
# a rank its registers allow), and wave w takes k-pairs w, w + NW, ... of its
# range: two per loop trip, one more after the loop when the count is odd.
QUANT_SHAPES = [(1, 128, 16, False),     # 1 k-pair, 2 waves: wave 1 has none
                (1, 640, 32, True),      # 5 k-pairs, 4 waves: 2, 1, 1, 1
                (8, 2304, 48, False),    # 4 ranges of 4-5 k-pairs, 4 waves
                (40, 4224, 64, True),    # 4 ranges of 8-9, 8 waves
                (40, 8320, 16, True),    # 4 ranges of 16-17, 16 waves
                (4096, 3072, 32, False),  # 24 k-pairs, 8 waves: 3 each (a trip and a peeled step)
                (4096, 4096, 16, True)]  # 32 k-pairs, 8 waves: 4 each (two trips)


def _quant_waves(M, K, R, norm):
    """(NW, sorted set of k-pairs per wave) of the activation pass's launch."""
    _, _, ks = W.w4a4_act_layout(M, K, R, with_splits=True)
    KP, mt = K // 128, -(-M // 16)
    rh = 16
    while rh > 8 and mt * (16 // rh) * ks < 256:
        rh //= 2
    wgs, kp_wg = mt * ks, KP // ks
    if kp_wg >= 16 and wgs < 256 and R <= (16 if norm else 32):
        nw = 16
    else:
        nw = 8 if kp_wg >= 8 else (4 if kp_wg >= 4 else 2)
    counts = set()
    for j in range(ks):
        n = (j + 1) * KP // ks - j * KP // ks
        counts |= {len(range(w, n, nw)) for w in range(nw)}
    return nw, counts


@pytest.mark.parametrize("M,K,R,norm", QUANT_SHAPES)
def test_quantizer_launch_shapes(M, K, R, norm):
    """Codes and scales bit-exact, lora_act within 1e-4 * rms, for every
    wave count and every number of k-pairs per wave the loop handles."""
    case = workloads.random_case(M, K, 16, R, seed=4400 + M + K + R)
    nw, counts = _quant_waves(M, K, R, norm)
    _say(f"[quant shape] M={M} K={K} R={R} norm={norm}: {nw} waves, k-pairs per wave {sorted(counts)}")
    if norm:
        gamma = np.random.default_rng(4401 + K).uniform(0.5, 2.0, K).astype(np.float16)
        _, qx, sx, la = O.quantize_act_rmsnorm(case["x"], gamma, 1e-6, case["lora_down"])
        run = GpuLayerRun(case, norm=(gamma, 1e-6))
    else:
        qx, sx, la = O.quantize_act(case["x"], case["lora_down"])
        run = GpuLayerRun(case)
    a = _check_quant(run, case, qx, sx)
    _check_lora_act(a, la, M)


def test_svdquant_checkpoint_layer():
    """A checkpoint derived offline (w4a4_gemm_lora_amd.svdquant: RTN int4 plus
    rank-32 factors of the quantization error) packed through the qweight
    path and run: codes, scales and factors as derived, output within the
    usual tolerance of the oracle on the same checkpoint."""
    from w4a4_gemm_lora_amd import svdquant as S
    rng = np.random.default_rng(15)
    M, K, N, R = 48, 1024, 160, 32
    a = rng.standard_normal((N, 4)) @ rng.standard_normal((4, K))
    w = (a * 0.02 + rng.standard_normal((N, K)) * 0.01).astype(np.float16)
    d = S.derive(w, rank=R)
    case = workloads.random_case(M, K, N, R, seed=4200)
    case.update(qweight=d["qweight"], w_scales=d["w_scales"], lora_down=d["proj_down"], lora_up=d["proj_up"])
    _say(f"[svdquant] M={M} K={K} N={N} R={R} residual/rtn={d['residual_norm'] / d['rtn_error_norm']:.3f}")
    run = GpuLayerRun(case, use_qweight=True)
    ref = O.linear(case["x"], d["proj_down"], d["proj_up"], case["col_scale"], case["bias"],
                   qweight=d["qweight"], w_scales=d["w_scales"])
    _check_weights(run, case, d["codes"], d["w_scales"])
    _check_y(run.host_y()[:M, :N], ref["y"], "svdquant checkpoint", y64=ref["y64"], ref=ref, case=case)


@pytest.mark.parametrize("norm", [False, True])
def test_layer_graph_buckets_replay_eager(norm):
    """Bucketed native graphs (LayerGraphs over w4a4_graph_*; "W4A4 CUDA
    Kernel for Voice Clone", section 4.3: pad to the bucket, copy in,
    replay): requests of several row counts, each padded to its bucket and
    replayed, give bit for bit the eager two-call result on the same rows and
    are within the layer bar of the oracle on the request's own rows
    (RMSNorm variant: the oracle's norm-then-layer); buckets are replayed
    repeatedly with new data, with the program's own eager work and
    synchronizations in between, every other replay on a side stream."""
    torch = _torch()
    rng = np.random.default_rng(16)
    N, K, R = 96, 1024, 32
    case = workloads.random_case(16, K, N, R, seed=4300)
    layer = W.PackedLinear(N, K, R, w_fp16=_to_dev(case["w"]), lora_down=_to_dev(case["lora_down"]),
                           lora_up=_to_dev(case["lora_up"]), col_scale=_to_dev(case["col_scale"]),
                           bias=_to_dev(case["bias"]))
    gamma = _to_dev(rng.uniform(0.5, 2.0, K).astype(np.float16)) if norm else None
    graphs = W.LayerGraphs(layer, [1, 4, 16, 64], gamma=gamma, eps=1e-6)   # a chain of one layer
    side = torch.cuda.Stream()
    g_host = None if gamma is None else gamma.cpu().numpy()
    try:
        for it, M in enumerate([1, 3, 16, 40, 1, 64, 3, 40]):
            xh = (rng.standard_normal((M, K)) * (1 + it)).astype(np.float16)
            x = _to_dev(xh)
            # eager reference at the bucket size (rows past M zero, as the graph sees them)
            B = graphs.bucket_for(M)
            xp = torch.zeros((B, K), dtype=torch.float16, device="cuda")
            xp[:M] = x
            act = W.alloc_act_blob(B, K, R)
            y_ref = torch.empty((B, N), dtype=torch.float16, device="cuda")
            if norm:
                W.w4a4_quantize_act_rmsnorm(B, K, R, xp, gamma, 1e-6, layer.wblob, act)
            else:
                W.w4a4_quantize_act(B, K, R, xp, layer.wblob, act)
            W.w4a4_linear(B, N, K, R, act, layer.wblob, y_ref)
            torch.cuda.synchronize()
            y = graphs.run(x, stream=side if it % 2 else None)
            torch.cuda.synchronize()
            _say(f"[graph] norm={norm} M={M} bucket={B} stream={'side' if it % 2 else 'current'}")
            assert torch.equal(y, y_ref[:M]), f"replay {it} (M={M}) differs from eager"
            xin = xh if gamma is None else O.rms_norm(xh, g_host, 1e-6)
            ref = O.linear(xin, case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
            _check_y(y.cpu().numpy(), ref["y"], f"graph replay M={M}", y64=ref["y64"], ref=ref, case=case)
    finally:
        graphs.close()


def test_graph_capture_of_a_layer_chain():
    """w4a4_graph_begin/end around a chain of three layers (the second and
    third reading the previous output) captured on a side stream: every
    replay, with new input written between replays and eager work in between,
    equals the eager chain bit for bit, and each layer's replayed output is
    within the layer bar of the oracle applied to that layer's replayed
    input."""
    import ctypes
    torch = _torch()
    lib = W.load_library()
    M, K = 16, 1024
    dims = [(K, 1024, 32), (1024, 1024, 16), (1024, 2048, 0)]   # (K_in, N, R)
    layers, acts, ys, cases = [], [], [], []
    for j, (k_in, n, r) in enumerate(dims):
        c = workloads.random_case(16, k_in, n, r, seed=4400 + j)
        cases.append(c)
        layers.append(W.PackedLinear(n, k_in, r, w_fp16=_to_dev(c["w"]),
                                     lora_down=_to_dev(c["lora_down"]) if r else None,
                                     lora_up=_to_dev(c["lora_up"]) if r else None,
                                     col_scale=_to_dev(c["col_scale"]), bias=_to_dev(c["bias"])))
        acts.append(W.alloc_act_blob(M, k_in, r))
        ys.append(torch.empty((M, n), dtype=torch.float16, device="cuda"))
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")

    def chain(stream):
        inp = x
        for L, act, y in zip(layers, acts, ys):
            W.w4a4_quantize_act(M, L.K, L.R, inp, L.wblob, act, stream=stream)
            W.w4a4_linear(M, L.N, L.K, L.R, act, L.wblob, y, stream=stream)
            inp = y

    side = torch.cuda.Stream()
    h = ctypes.c_void_p()
    with torch.cuda.stream(side):
        assert lib.w4a4_graph_begin(side.cuda_stream) == 0
        chain(side.cuda_stream)
        assert lib.w4a4_graph_end(side.cuda_stream, ctypes.byref(h)) == 0
    try:
        rng = np.random.default_rng(17)
        for it in range(4):
            x.copy_(_to_dev(rng.standard_normal((M, K)).astype(np.float16)))
            chain(torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            ref = ys[-1].clone()
            ys[-1].fill_(float("nan"))
            assert lib.w4a4_graph_launch(h, torch.cuda.current_stream().cuda_stream) == 0
            torch.cuda.synchronize()
            assert torch.equal(ys[-1], ref), f"replay {it} differs from the eager chain"
            inp = x.cpu().numpy()
            for j, (c, y) in enumerate(zip(cases, ys)):
                r = dims[j][2]
                o = O.linear(inp, c["lora_down"] if r else None, c["lora_up"] if r else None, c["col_scale"],
                             c["bias"], w16=c["w"])
                out = y.cpu().numpy()
                _check_y(out, o["y"], f"chain replay {it} layer {j}", y64=o["y64"], ref=o, case=c)
                inp = out
    finally:
        lib.w4a4_graph_destroy(h)
