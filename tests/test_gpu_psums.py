"""GPU parity of the exact per-group integer sums P[m, n, g] ("W4A4 CUDA
Kernel for Voice Clone", section 3.7: the int32 sum of each 64-group before
the per-group dequant), bit for bit against the oracle.

w4a4_debug_group_psums launches the instance of the kernel, tile shape and
variant that w4a4_linear runs for the same shape (and the same W4A4_TILED_*
overrides) with only the per-group scale-accumulate swapped for a store of P,
so these checks cover the integer path of every production kernel: the
tiled kernel (every tile shape, lean and K-split variants; 3.0f-offset
integer MFMA), the MFMA decode kernel (5 <= M <= 16, and M = 4 on wide
layers) and the dot decode kernel (M <= 4, v_dot8 on the packed nibbles).
Codes -8 (the two's-complement edge, "INT4 Kernel Architecture, in depth",
section "Failure modes") reach every M <= 16 kernel from checkpoint weights
and from activation rows whose fp16 scale is subnormal.
"""
import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from oracle import w4a4_oracle as O
from tests.test_gpu_parity import GpuLayerRun, _check_y, _say, _to_dev, _torch, _workload

pytestmark = pytest.mark.gpu


def _check_window(got, qx, qw, m0, n0, M, what):
    """got [mc][nc][G] against the oracle's P; window rows >= M are padding (0)."""
    mc, nc = got.shape[:2]
    rows = np.arange(m0, min(m0 + mc, M))
    want = O.group_psums(qx[rows], qw[n0: n0 + nc])
    bad = np.argwhere(got[: len(rows)] != want)
    assert bad.size == 0, f"{what}: {len(bad)} group sums differ, first at (m, n, g) = {bad[0] + [m0, n0, 0]}"
    assert not np.any(got[len(rows):]), f"{what}: padding rows of the window are not 0"


def _full_psums(run, glu=False):
    torch = _torch()
    Mp = (run.M + 15) // 16 * 16
    out = torch.full((Mp, run.N, run.K // 64), -(2 ** 31), dtype=torch.int32, device="cuda")
    fn = W.w4a4_debug_group_psums_glu if glu else W.w4a4_debug_group_psums
    fn(run.M, run.N, run.K, run.R, run.act, run.wblob, 0, Mp, 0, run.N, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["small", "mlp_up", "mlp_down", "decode-1", "decode-2", "decode-4", "decode-16"])
def test_psums_whole_output_of_each_workload(name):
    """Every group sum of the whole output of the workloads the oracle
    finishes in seconds (the decode sweep at M = 1, 2, 4, 16: dot kernel,
    dot kernel, MFMA decode kernel with two column tiles per workgroup, MFMA
    decode kernel)."""
    case = _workload(name)
    run = GpuLayerRun(case)
    _say(f"[psums] {name} M={run.M} K={run.K} N={run.N} variant={W.w4a4_query_variant(run.M, run.N, run.K, run.R)}")
    qx, _ = O.quantize_groups(case["x"])
    qw, _ = O.quantize_groups(case["w"])
    _check_window(_full_psums(run), qx, qw, 0, 0, run.M, name)


def _forced(monkeypatch, cfg, lean, ksplit):
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    monkeypatch.setenv("W4A4_TILED_LEAN", str(int(lean)))
    monkeypatch.setenv("W4A4_TILED_KSPLIT", str(int(ksplit)))


TILED_INSTANCES = ([(c, False, False) for c in range(10)] + [(c, True, False) for c in (0, 1, 2, 3, 5, 8)]
                   + [(c, False, True) for c in (3, 4, 5, 7, 8)])


@pytest.mark.parametrize("cfg,lean,ksplit", TILED_INSTANCES)
def test_psums_every_tiled_instance(cfg, lean, ksplit, monkeypatch):
    """Each tile shape of the tiled kernel (forced), its lean variant where
    it has one and its K-split variant where it has one, on a shape with
    ragged row and column edges for all of them (M = 130: 9 row tiles, N =
    208: 13 column tiles; K = 2560: 20 k-pairs, split 10 + 10), with codes
    -8 in the weights: all of P."""
    M, K, N, R = 130, 2560, 208, 32
    _forced(monkeypatch, cfg, lean, ksplit)
    case = workloads.random_case(M, K, N, R, seed=5000 + cfg + 20 * lean + 40 * ksplit)
    rng = np.random.default_rng(5100 + cfg)
    q = rng.integers(-8, 8, size=(N, K))
    q[3, :] = -8
    q[:, 5] = -8
    nib = (q & 0xF).astype(np.uint8)
    case["qweight"] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    case["w_scales"] = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float16)
    _say(f"[psums tiled] cfg={cfg} lean={lean} ksplit={ksplit}")
    run = GpuLayerRun(case, use_qweight=True)
    qx, _ = O.quantize_groups(case["x"])
    _check_window(_full_psums(run), qx, q.astype(np.int8), 0, 0, M, f"cfg {cfg} lean {lean} ksplit {ksplit}")
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"],
                   qweight=case["qweight"], w_scales=case["w_scales"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"tiled cfg {cfg} lean {lean} ksplit {ksplit}", y64=ref["y64"], ref=ref, case=case)


def _subnormal_rows(rng, x, rows):
    """Rows whose every group has absmax 17 * 2^-24: the fp16 scale rounds to
    2 * 2^-24 and codes k / 2 (round half to even, clamped) reach -8 for
    k = -16, -17 (the golden case subnormal_scale_clamp_reaches_minus_8)."""
    K = x.shape[1]
    for r in rows:
        k = rng.integers(-17, 18, size=K)
        k[::64] = -17
        x[r] = (k * 2.0 ** -24).astype(np.float16)
    return x


DECODE_SHAPES = [(1664, 8192), (1664, 48), (8192, 4096)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("K,N", DECODE_SHAPES)
def test_psums_decode_kernels_with_minus_eight(M, K, N):
    """-8 codes through every M <= 16 kernel: checkpoint weights with a whole
    row and scattered entries at -8, and activation rows with subnormal
    scales whose codes reach -8.  N = 8192 takes the two-column-tile paths
    (dot kernel for M <= 3, MFMA decode for M >= 4), N = 48 the one-tile ones
    (dot kernel up to M = 4), K = 8192 at N = 4096 the 8-wave workgroups
    (K split eight ways).  All of P bit-exact, Y within the layer bar."""
    R = 32
    case = workloads.random_case(M, K, N, R, seed=6000 + M + K + N)
    rng = np.random.default_rng(6100 + M + K)
    x = case["x"].copy()
    x = _subnormal_rows(rng, x, range(0, M, 2))
    case["x"] = x
    q = rng.integers(-8, 8, size=(N, K))
    q[1, :] = -8
    q[rng.random((N, K)) < 0.05] = -8
    nib = (q & 0xF).astype(np.uint8)
    case["qweight"] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    case["w_scales"] = rng.uniform(1e-3, 1e-2, size=(N, K // 64)).astype(np.float16)
    _say(f"[psums decode -8] M={M} K={K} N={N}")
    run = GpuLayerRun(case, use_qweight=True)
    qx, _ = O.quantize_groups(case["x"])
    assert np.any(qx == -8), "the subnormal rows must carry -8 codes"
    a = run.host_act()
    assert np.array_equal(a["qx"][:M], qx), "activation codes differ"
    _check_window(_full_psums(run), qx, q.astype(np.int8), 0, 0, M, f"decode M={M} K={K} N={N}")
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"],
                   qweight=case["qweight"], w_scales=case["w_scales"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"decode -8 M={M} K={K} N={N}", y64=ref["y64"], ref=ref, case=case)


def _interleave(gate, up, tile=16):
    n = gate.shape[0]
    g = gate.reshape(n // tile, tile, *gate.shape[1:])
    u = up.reshape(n // tile, tile, *up.shape[1:])
    return np.stack([g, u], axis=1).reshape(2 * n, *gate.shape[1:])


@pytest.mark.parametrize("M", [1, 4, 16, 130])
def test_psums_gated_layer_dispatch(M):
    """The kernels w4a4_linear_glu runs (tile shapes and decode paths that
    hold whole (gate, up) pairs): P of the interleaved packed columns."""
    K, N, R = 1024, 8192 if M == 4 else 96, 32
    torch = _torch()
    g = workloads.random_case(M, K, N // 2, R // 2, seed=7000 + M)
    u = workloads.random_case(M, K, N // 2, R // 2, seed=7100 + M)
    w = _interleave(g["w"], u["w"])
    wblob = W.alloc_weight_blob(N, K, R)
    ld = np.concatenate([g["lora_down"], u["lora_down"]], axis=1)
    lu = np.zeros((N, R), np.float16)
    lu[:, :R // 2] = _interleave(g["lora_up"], np.zeros_like(u["lora_up"]))[:, :R // 2]
    lu[:, R // 2:] = _interleave(np.zeros_like(g["lora_up"]), u["lora_up"])[:, :R // 2]
    W.w4a4_pack_weights(N, K, R, wblob, w_fp16=_to_dev(np.ascontiguousarray(w)), lora_down=_to_dev(ld),
                        lora_up=_to_dev(lu))
    x = _to_dev(g["x"])
    act = W.alloc_act_blob(M, K, R)
    W.w4a4_quantize_act(M, K, R, x, wblob, act)
    Mp = (M + 15) // 16 * 16
    out = torch.zeros((Mp, N, K // 64), dtype=torch.int32, device="cuda")
    W.w4a4_debug_group_psums_glu(M, N, K, R, act, wblob, 0, Mp, 0, N, out)
    torch.cuda.synchronize()
    _say(f"[psums glu] M={M} K={K} N={N}")
    qx, _ = O.quantize_groups(g["x"])
    qw, _ = O.quantize_groups(w)
    _check_window(out.cpu().numpy(), qx, qw, 0, 0, M, f"gated M={M}")


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("tiles", [1, 2])
def test_psums_every_decode_shape_forced(M, waves, tiles, monkeypatch):
    """Each decode workgroup shape forced (W4A4_DECODE_WAVES: K split 4 or 8
    ways; W4A4_DECODE_TILES: one or two column tiles per workgroup) on a
    shape where all of them apply (K = 1664: 13 k-pairs, so with 8 waves the
    last wave has none; N = 8192): all of P bit-exact and Y within the
    layer bar, for the dot kernel (M = 1) and the MFMA decode kernel (M = 4,
    16)."""
    K, N, R = 1664, 8192, 32
    monkeypatch.setenv("W4A4_DECODE_WAVES", str(waves))
    monkeypatch.setenv("W4A4_DECODE_TILES", str(tiles))
    case = workloads.random_case(M, K, N, R, seed=6500 + M + 10 * waves + tiles)
    _say(f"[psums decode forced] M={M} waves={waves} tiles={tiles}")
    run = GpuLayerRun(case)
    qx, _ = O.quantize_groups(case["x"])
    qw, _ = O.quantize_groups(case["w"])
    _check_window(_full_psums(run), qx, qw, 0, 0, M, f"decode forced M={M} waves={waves} tiles={tiles}")
    ref = O.linear(case["x"], case["lora_down"], case["lora_up"], case["col_scale"], case["bias"], w16=case["w"])
    _check_y(run.host_y()[:M, :N], ref["y"], f"decode forced M={M} waves={waves} tiles={tiles}",
             y64=ref["y64"], ref=ref, case=case)
