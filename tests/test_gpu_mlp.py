"""GPU parity of the gated-MLP front half: gate and up projections packed as
one layer with SiLU(gate) * up in the GEMM epilogue (w4a4_linear_glu),
against the oracle's two separate layers and gated activation.

"W4A4 CUDA Kernel for Voice Clone", section 3.1: the Qwen3 MLP computes
SiLU(gate_proj(x)) * up_proj(x) and feeds it to down_proj.
"""
import os

import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from oracle import w4a4_oracle as O
from tests.parity_bar import MEAN_TOL, near_tie_flips
from tests.test_gpu_parity import _check_y, _say, _to_dev, _torch

pytestmark = pytest.mark.gpu


def _interleave_cols(yp):
    """Split a packed gated output [M, 2N] (column tiles of 16 alternating
    gate, up) into g [M, N] and u [M, N]."""
    M, N2 = yp.shape
    t = yp.reshape(M, N2 // 32, 2, 16)
    return t[:, :, 0, :].reshape(M, N2 // 2), t[:, :, 1, :].reshape(M, N2 // 2)


def _decode_waves(workgroups, K):
    """The decode kernels' K split for a launch of `workgroups` workgroups
    (8 waves when there are few workgroups and many k-pairs, else 4)."""
    return 8 if workgroups <= 256 and K // 128 >= 64 else 4


class _env:
    """Set environment variables for a block (tuning overrides the library
    reads at every launch), restoring them afterwards."""

    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _plain_env(M, N, K, R):
    """Overrides under which w4a4_linear on the packed gated blob (2N
    columns, rank R) runs the per-tile arithmetic of the kernel
    w4a4_linear_glu picks: for M > 16 every tiled shape without a K split
    accumulates a tile in the same order, so one is forced unless the gated
    run forces its own (then the same one); for M <= 16 the gated kernels
    hold one (gate, up) pair of tiles per workgroup, so two tiles and the
    same K split."""
    if M <= 16:
        return dict(W4A4_DECODE_TILES=2, W4A4_DECODE_WAVES=_decode_waves(2 * N // 32, K))
    cfg = os.environ.get("W4A4_TILED_CFG", "")
    if cfg == "":
        # the gated pick is never the wide kernel at these sizes (it needs
        # 512 workgroups of 256 x 128)
        assert ((M + 255) // 256) * (2 * N // 128) < 512 or R > 32, (M, N)
        cfg = "0"
    return dict(W4A4_TILED_CFG=cfg, W4A4_TILED_KSPLIT=0)


def _check_glu(h_gpu, gu_gpu, x, gate, up, Rg, Ru, what):
    """The gated layer against the oracle:
    - g and u (from w4a4_linear on the packed blob, the gated kernel's own
      per-tile arithmetic, see _plain_env) each at the layer bar against the
      oracle's gate and up layers (parity_bar, near ties judged against the
      kernel's error bound);
    - h equal to fp16(SiLU(g) * u) of those g and u, bit for bit except at
      near ties of that rounding: the kernel's fp32 SiLU from the hardware
      exp2 and reciprocal is within ~1e-6 relative of the exact value for
      |g| <= 20 and within ~6e-6 beyond (the exponent's argument rounded),
      so a flip is accepted only between the two fp16 neighbours of the
      exact value and within 1e-5 relative of their midpoint;
    - h against the oracle's h (from the oracle's g and u): the mean bar."""
    M, N = h_gpu.shape
    g_gpu, u_gpu = gu_gpu
    for name, c, R, y in (("g", gate, Rg, g_gpu), ("u", up, Ru, u_gpu)):
        ref = O.linear(x, **_half(c, R))
        _check_y(y, ref["y"], f"{what} {name}", y64=ref["y64"], ref=ref,
                 case=dict(lora_up=c["lora_up"] if R else None, col_scale=c["col_scale"], bias=c["bias"]))
    exact = O.silu(g_gpu.astype(np.float64)) * u_gpu.astype(np.float64)
    want = O.to_fp16(exact)
    differ = h_gpu.astype(np.float64) != want.astype(np.float64)
    tie = near_tie_flips(h_gpu, want, exact, 1e-5 * np.abs(exact) + 2.0 ** -30)
    bad = differ & ~tie
    _say(f"{what}: h vs fp16(SiLU(g) u) of the GPU's g, u: {int(differ.sum())} differ, all near ties: {not bad.any()}")
    assert not bad.any(), (f"{what}: h differs from the gated activation of g, u beyond a near tie at "
                           f"{np.argwhere(bad)[0]}: {h_gpu[bad][0]} vs {want[bad][0]} (exact {exact[bad][0]})")
    _, _, h_ref = O.mlp_gate_up(x, _half(gate, Rg), _half(up, Ru))
    hr = h_ref.astype(np.float64)
    err = np.abs(h_gpu.astype(np.float64) - hr)
    rms = np.sqrt(np.mean(hr ** 2))
    _say(f"{what}: h vs oracle h: max|dh|/rms={err.max() / rms:.3g} mean|dh|/rms={err.mean() / rms:.3g}")
    assert err.mean() <= MEAN_TOL * rms, f"{what}: mean err {err.mean()} > {MEAN_TOL}*{rms}"


def _half(case, R):
    """One projection's oracle arguments (rank R may be 0)."""
    return dict(lora_down16=case["lora_down"] if R else None, lora_up16=case["lora_up"] if R else None,
                col_scale=case["col_scale"], bias=case["bias"], w16=case["w"])


def _run_glu(x, gate, up, Rg, Ru, ldy=None, with_gu=False):
    """Pack (gate, up) through GatedMLPUp, quantize x, run the gated GEMM
    into a NaN-filled output of row stride ldy; returns host h [M, ldy], and
    with with_gu also (g, u) [M, N] from w4a4_linear on the same packed
    blob and activation blob (see _plain_env)."""
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
    if not with_gu:
        return h.cpu().numpy()
    yp = torch.empty((max(M, 1), 2 * N), dtype=torch.float16, device="cuda")
    with _env(**_plain_env(M, N, K, layer.R)):
        W.w4a4_linear(M, 2 * N, K, layer.R, act, layer.wblob, yp)
    torch.cuda.synchronize()
    return h.cpu().numpy(), _interleave_cols(yp.cpu().numpy()[:M])


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
    h, gu = _run_glu(x, g, u, Rg, Ru, with_gu=True)
    _check_glu(h[:M, :N], gu, x, g, u, Rg, Ru, f"glu M={M} K={K} N={N} R={Rg}+{Ru}")
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
    h, gu = _run_glu(x, g, u, R, R, with_gu=True)
    _check_glu(h[:M, :N], gu, x, g, u, R, R, "glu mlp workload")


@pytest.mark.parametrize("M", [5, 64])
def test_glu_strided_output(M):
    """A row stride above the output width: the columns past N stay as they
    were (NaN), rows below M too."""
    K, N, R = 512, 96, 16
    x, g, u = _cases(M, K, N, R, R, seed=5200 + M)
    h, gu = _run_glu(x, g, u, R, R, ldy=N + 40, with_gu=True)
    _check_glu(h[:M, :N], gu, x, g, u, R, R, f"glu strided M={M}")
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
    h, gu = _run_glu(x, g, u, R, R, with_gu=True)
    _check_glu(h[:M, :N], gu, x, g, u, R, R, f"glu tile shape {cfg}")


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
