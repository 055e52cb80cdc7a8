"""GPU parity of the gated-MLP front half: gate and up projections packed as
one layer with SiLU(gate) * up in the GEMM epilogue (w4a4_linear_glu),
against the oracle's two separate layers and gated activation.

"W4A4 CUDA Kernel for Voice Clone", section 3.1: the Qwen3 MLP computes
SiLU(gate_proj(x)) * up_proj(x) and feeds it to down_proj.
"""
import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from oracle import w4a4_oracle as O
from tests.test_gpu_parity import MAX_TOL, MEAN_TOL, _say, _to_dev, _torch

pytestmark = pytest.mark.gpu


def _fp16_ulp(v):
    """Spacing of fp16 values at |v| (subnormal spacing below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _check_h(h_gpu, h_ref, what):
    """The layer bar on h (mean error <= MEAN_TOL rms; max error <= MAX_TOL rms)
    with two fp16 ulps of slack per element on the max: h = fp16(SiLU(g) u)
    comes from the fp16-rounded g and u, and a g or u lying within rounding
    error of an fp16 rounding boundary may round to the neighbouring value
    (moving h by up to ~1 ulp of h), after which h's own rounding may flip
    too.  At |h| >= 32 one ulp (2^-5) alone exceeds 2e-2 rms for rms ~ 1."""
    hg = h_gpu.astype(np.float64)
    hr = h_ref.astype(np.float64)
    assert np.all(np.isfinite(hg)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(hr ** 2))
    err = np.abs(hg - hr)
    _say(f"{what}: rms={rms:.4g} max|dh|/rms={err.max() / rms:.3g} mean|dh|/rms={err.mean() / rms:.3g}")
    bound = MAX_TOL * rms + 2.0 * _fp16_ulp(hr)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), f"{what}: err {err.flat[worst]} > bound {bound.flat[worst]} at h={hr.flat[worst]}"
    assert err.mean() <= MEAN_TOL * rms, f"{what}: mean err {err.mean()} > {MEAN_TOL}*{rms}"


def _half(case, R):
    """One projection's oracle arguments (rank R may be 0)."""
    return dict(lora_down16=case["lora_down"] if R else None, lora_up16=case["lora_up"] if R else None,
                col_scale=case["col_scale"], bias=case["bias"], w16=case["w"])


def _run_glu(x, gate, up, Rg, Ru, ldy=None):
    """Pack (gate, up) through GatedMLPUp, quantize x, run the gated GEMM
    into a NaN-filled output of row stride ldy; returns host h [M, ldy]."""
    torch = _torch()
    M, K = x.shape
    N = gate["w"].shape[0]
    d = lambda a: _to_dev(a)
    layer = W.GatedMLPUp(N, K, d(gate["w"]), d(up["w"]),
                         lora_down_gate=d(gate["lora_down"]) if Rg else None,
                         lora_up_gate=d(gate["lora_up"]) if Rg else None,
                         lora_down_up=d(up["lora_down"]) if Ru else None,
                         lora_up_up=d(up["lora_up"]) if Ru else None,
                         a_gate=d(gate["col_scale"]), b_gate=d(gate["bias"]),
                         a_up=d(up["col_scale"]), b_up=d(up["bias"]))
    ldy = N if ldy is None else ldy
    xd = d(x)
    act = W.alloc_act_blob(M, K, layer.R)
    h = torch.full((max(M, 1), ldy), float("nan"), dtype=torch.float16, device="cuda")
    W.w4a4_quantize_act(M, K, layer.R, xd, layer.wblob, act)
    W.w4a4_linear_glu(M, 2 * N, K, layer.R, layer.r_gate, act, layer.wblob, h, ldy=ldy)
    torch.cuda.synchronize()
    return h.cpu().numpy()


def _cases(M, K, N, Rg, Ru, seed):
    g = workloads.random_case(M, K, N, Rg, seed=seed)
    u = workloads.random_case(M, K, N, Ru, seed=seed + 1)
    return g["x"], g, u


@pytest.mark.parametrize("M,K,N,Rg,Ru", [(1, 1024, 64, 32, 32), (3, 640, 48, 16, 0),
                                         (4, 4096, 1024, 32, 32), (7, 1024, 80, 0, 16),
                                         (16, 4096, 1024, 32, 32), (12, 1536, 272, 16, 16),
                                         (17, 384, 48, 0, 0), (40, 384, 80, 16, 16),
                                         (130, 3072, 48, 32, 16), (300, 1024, 208, 32, 32),
                                         (3, 8192, 2048, 32, 32), (9, 8192, 2048, 16, 16),
                                         (24, 1024, 64, 8, 8), (5, 1024, 64, 8, 24), (40, 512, 96, 24, 8)])
def test_glu_layer_against_oracle(M, K, N, Rg, Ru):
    """h = fp16(SiLU(g) * u) within the layer tolerance (taken on h) of the
    oracle's separate gate and up layers; decode (M <= 16) and tiled (M > 16)
    kernels, ragged row counts, either projection without LoRA, unequal
    ranks (also ranks that share a 16-wide rank block of the packed L_up,
    where no block can be skipped), column counts that are and are not
    multiples of 64."""
    x, g, u = _cases(M, K, N, Rg, Ru, seed=5000 + M + K + N + Rg)
    _say(f"[glu] M={M} K={K} N={N} Rg={Rg} Ru={Ru} -> variant {W.w4a4_query_variant(M, 2 * N, K, Rg + Ru)}")
    h = _run_glu(x, g, u, Rg, Ru)
    _, _, ref = O.mlp_gate_up(x, _half(g, Rg), _half(u, Ru))
    _check_h(h[:M, :N], ref, f"glu M={M} K={K} N={N} R={Rg}+{Ru}")
    assert np.all(np.isnan(h[M:].astype(np.float64)))


def test_glu_mlp_workload_full_output():
    """The MLP up-projection workload (M=700 tokens, K=1024, 3072 columns per
    projection, rank 32 each, X with x20 outlier channels): gate and up
    drawn from two seeds of the workload recipe, the full h compared."""
    g = workloads.generate("mlp_up")
    u = workloads.generate("mlp_up", seed=workloads.WORKLOADS["mlp_up"].seed + 7)
    x = g["x"]
    M, K, N, R = g["M"], g["K"], g["N"], g["R"]
    _say(f"[glu workload] M={M} K={K} N={N} R={R}+{R}")
    h = _run_glu(x, g, u, R, R)
    _, _, ref = O.mlp_gate_up(x, _half(g, R), _half(u, R))
    _check_h(h[:M, :N], ref, "glu mlp workload")


@pytest.mark.parametrize("M", [5, 64])
def test_glu_strided_output(M):
    """A row stride above the output width: the columns past N stay as they
    were (NaN), rows below M too."""
    K, N, R = 512, 96, 16
    x, g, u = _cases(M, K, N, R, R, seed=5200 + M)
    h = _run_glu(x, g, u, R, R, ldy=N + 40)
    _, _, ref = O.mlp_gate_up(x, _half(g, R), _half(u, R))
    _check_h(h[:M, :N], ref, f"glu strided M={M}")
    assert np.all(np.isnan(h[:, N:].astype(np.float64)))


@pytest.mark.parametrize("cfg,lean", [(c, "0") for c in range(10)] + [(c, "1") for c in (0, 1, 2, 3, 8)])
def test_glu_every_tile_shape(cfg, lean, monkeypatch):
    """Each M > 16 tile shape forced in turn, in the 4-stage and (where it
    exists) the lean variant (shapes whose waves hold an odd number of
    column tiles cannot pair gate with up and fall back to the model's
    pick); 13 row tiles and 14 fused column tiles leave ragged edges for
    every shape."""
    M, K, N, R = 200, 1024, 112, 16
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    monkeypatch.setenv("W4A4_TILED_LEAN", lean)
    x, g, u = _cases(M, K, N, R, R, seed=5300 + cfg)
    _say(f"[glu tile shape {cfg} lean={lean}] M={M} K={K} N={N}")
    h = _run_glu(x, g, u, R, R)
    _, _, ref = O.mlp_gate_up(x, _half(g, R), _half(u, R))
    _check_h(h[:M, :N], ref, f"glu tile shape {cfg}")


def test_glu_matches_separate_layers_on_gpu():
    """The fused layer against the library's own two layers plus the
    oracle's gated activation of their fp16 outputs: the integer work is
    the same, so h differs only where the fp32 accumulation order of the
    two launches rounds g or u to a neighbouring fp16 value."""
    torch = _torch()
    M, K, N, R = 16, 2048, 256, 32
    x, g, u = _cases(M, K, N, R, R, seed=5400)
    outs = []
    for c in (g, u):
        wb = W.alloc_weight_blob(N, K, R)
        W.w4a4_pack_weights(N, K, R, wb, w_fp16=_to_dev(c["w"]), lora_down=_to_dev(c["lora_down"]),
                            lora_up=_to_dev(c["lora_up"]), col_scale=_to_dev(c["col_scale"]),
                            bias=_to_dev(c["bias"]))
        act = W.alloc_act_blob(M, K, R)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        W.w4a4_quantize_act(M, K, R, _to_dev(x), wb, act)
        W.w4a4_linear(M, N, K, R, act, wb, y)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    h_sep = O.glu(outs[0], outs[1])
    h = _run_glu(x, g, u, R, R)[:M, :N]
    d = np.abs(h.astype(np.float64) - h_sep.astype(np.float64))
    rms = np.sqrt(np.mean(h_sep.astype(np.float64) ** 2))
    _say(f"glu vs separate layers: max|d|/rms={d.max() / rms:.3g}, differing {np.count_nonzero(d)} of {d.size}")
    assert d.max() <= 4e-3 * rms
    assert np.count_nonzero(d) <= d.size // 20
