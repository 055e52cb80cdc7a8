"""GPU parity of the gated layer whose output goes straight into the down
projection's activation blob (w4a4_linear_glu_quant), and of the whole
gated MLP built on it.

"W4A4 CUDA Kernel for Voice Clone", section 3.1: the Qwen3 MLP computes
down_proj(SiLU(gate_proj(x)) * up_proj(x)), every projection W4A4; section
3.6: the activation pass of a layer's input (per-group codes and scales,
LoRA-down).  For M > 16 the gated GEMM's epilogue quantizes h itself, so
its codes and scales must equal, bit for bit, what the activation pass
writes from the h that w4a4_linear_glu stores, and those must equal the
oracle's quantizer applied to that h; lora_act differs from the activation
pass's only by the order of its fp32 sums.
"""
import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from oracle import w4a4_oracle as O
from tests.layout_unpack import split_act_blob
from tests.test_gpu_parity import _check_y, _say, _to_dev, _torch

pytestmark = pytest.mark.gpu


def _layers(M, K, H, Nd, Rg, Ru, Rd, seed, x_scale=1.0):
    """Seeded gate, up and down projections (the workload recipe's random
    layers) and x [M, K]."""
    g = workloads.random_case(M, K, H, Rg, seed=seed, x_scale=x_scale)
    u = workloads.random_case(M, K, H, Ru, seed=seed + 1)
    d = workloads.random_case(M, H, Nd, Rd, seed=seed + 2)
    return g["x"], g, u, d


def _pack(g, u, d, Rg, Ru, Rd):
    dev = _to_dev
    K, H, Nd = g["w"].shape[1], g["w"].shape[0], d["w"].shape[0]
    up = W.GatedMLPUp(H, K, dev(g["w"]), dev(u["w"]),
                      lora_down_gate=dev(g["lora_down"]) if Rg else None,
                      lora_up_gate=dev(g["lora_up"]) if Rg else None,
                      lora_down_up=dev(u["lora_down"]) if Ru else None,
                      lora_up_up=dev(u["lora_up"]) if Ru else None,
                      a_gate=dev(g["col_scale"]), b_gate=dev(g["bias"]),
                      a_up=dev(u["col_scale"]), b_up=dev(u["bias"]))
    down = W.PackedLinear(Nd, H, Rd, w_fp16=dev(d["w"]), lora_down=dev(d["lora_down"]) if Rd else None,
                          lora_up=dev(d["lora_up"]) if Rd else None, col_scale=dev(d["col_scale"]),
                          bias=dev(d["bias"]))
    return up, down


def _blob(M, K, R, fill):
    b = W.alloc_act_blob(M, K, R)
    b.fill_(fill)   # every byte the call owns must be written
    return b


def _run_both(x, up, down):
    """The quantized-output call and, for reference, the unfused pair
    (w4a4_linear_glu into h, then w4a4_quantize_act of h), both from the
    same activation blob of x.  Returns host (act_q, act_ref, h)."""
    torch = _torch()
    M, K, H, Rd = x.shape[0], up.K, up.N, down.R
    act = W.alloc_act_blob(M, K, up.R)
    W.w4a4_quantize_act(M, K, up.R, _to_dev(x), up.wblob, act)
    act_q = _blob(M, H, Rd, 0xA5)
    ws = torch.empty(max(W.w4a4_glu_quant_workspace(M, 2 * H, Rd), 256), dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    W.w4a4_linear_glu_quant(M, 2 * H, K, up.R, up.r_gate, act, up.wblob, Rd, down.wblob if Rd else None,
                            act_q, ws)
    h = torch.empty((M, H), dtype=torch.float16, device="cuda")
    W.w4a4_linear_glu(M, 2 * H, K, up.R, up.r_gate, act, up.wblob, h)
    act_r = _blob(M, H, Rd, 0x3C)
    W.w4a4_quantize_act(M, H, Rd, h, down.wblob, act_r)
    torch.cuda.synchronize()
    return act_q, act_r, h


def _lora_bound(h, ld):
    """Two fp32 summations of the same K fp16 x fp16 products (each exact in
    fp32) in different orders differ by at most 2 K 2^-24 sum_k |h_k ld_k|."""
    a = np.abs(h.astype(np.float64)) @ np.abs(ld.astype(np.float64))
    return 2.0 * h.shape[1] * 2.0 ** -24 * a + 1e-30


def _compare(act_q, act_r, h, M, H, Rd, ld, what):
    """Codes and scales of the whole blob (padding rows too) bit for bit
    against the activation pass and the oracle's quantizer of h; lora_act
    partial by partial against the activation pass's and, summed, against
    the oracle's fp64 h L_down, within the reordering bound."""
    _, offs, ks = W.w4a4_act_layout(M, H, Rd, with_splits=True)
    qb, rb = act_q.cpu().numpy(), act_r.cpu().numpy()
    Mp = (M + 15) // 16 * 16
    n_codes, n_scales = Mp * H // 2, Mp * (H // 64) * 2
    assert np.array_equal(qb[offs[0]: offs[0] + n_codes], rb[offs[0]: offs[0] + n_codes]), f"{what}: codes differ"
    assert np.array_equal(qb[offs[1]: offs[1] + n_scales], rb[offs[1]: offs[1] + n_scales]), f"{what}: scales differ"
    a = split_act_blob(qb, M, H, Rd, offs, ks)
    qx, sx = O.quantize_groups(h)
    assert np.array_equal(a["qx"][:M], qx), f"{what}: codes differ from the oracle's quantizer of h"
    assert np.array_equal(a["sx"][:M].view(np.uint16), sx.view(np.uint16)), f"{what}: scales differ from the oracle's"
    assert not np.any(a["qx"][M:]) and not np.any(a["sx"][M:].view(np.uint16)), f"{what}: padding rows not 0"
    if Rd == 0:
        return
    r = split_act_blob(rb, M, H, Rd, offs, ks)
    # each K-range partial covers the same groups in both blobs
    KP = H // 128
    for j in range(ks):
        cols = slice(128 * (j * KP // ks), 128 * ((j + 1) * KP // ks))
        bound = _lora_bound(h[:, cols], ld[cols])
        dq = np.abs(a["lora_parts"][j][:M].astype(np.float64) - r["lora_parts"][j][:M])
        assert np.all(dq <= bound), f"{what}: lora_act partial {j} beyond the reordering bound"
        assert not np.any(a["lora_parts"][j][M:]), f"{what}: padding rows of lora_act partial {j} not 0"
    exact = O.lora_act(h, ld)
    d = np.abs(a["lora_act"][:M].astype(np.float64) - exact)
    bound = _lora_bound(h, ld) * (1 + ks) + 2.0 ** -24 * np.abs(exact) * ks
    _say(f"{what}: codes/scales bit-exact; lora_act max|d| {d.max():.3g} (bound {bound.max():.3g})")
    assert np.all(d <= bound), f"{what}: lora_act beyond its bound against the oracle"


CASES = [
    # M, K, H, Rg, Ru, Rd
    (17, 384, 128, 16, 16, 16), (40, 512, 256, 32, 32, 32), (130, 1024, 384, 32, 16, 64),
    (300, 1024, 640, 0, 0, 0), (300, 768, 256, 16, 16, 48), (701, 1024, 1024, 32, 32, 32),
    (1, 1024, 256, 32, 32, 32), (4, 4096, 1024, 32, 32, 32), (16, 1024, 384, 16, 16, 16),
]


@pytest.mark.parametrize("M,K,H,Rg,Ru,Rd", CASES)
def test_glu_quant_matches_activation_pass(M, K, H, Rg, Ru, Rd, monkeypatch):
    """Quantized gated output against the unfused pair and the oracle's
    quantizer: ragged rows (17, 130, 701: padding inside the last tile),
    several groups and k-pairs of h, every down rank (0, 16, 32, 48, 64,
    one lora_act split or more), no LoRA at all -- the quantizing epilogue
    forced for M > 16 -- and M <= 16 (the route through the workspace)."""
    monkeypatch.setenv("W4A4_GLU_QUANT_EPILOGUE", "1")
    Nd = 64
    x, g, u, d = _layers(M, K, H, Nd, Rg, Ru, Rd, seed=8000 + M + H + Rd)
    up, down = _pack(g, u, d, Rg, Ru, Rd)
    _say(f"[glu quant] M={M} K={K} H={H} R={Rg}+{Ru} R_down={Rd}")
    act_q, act_r, h = _run_both(x, up, down)
    _compare(act_q, act_r, h.cpu().numpy(), M, H, Rd, d["lora_down"] if Rd else None, f"glu quant M={M} H={H}")


@pytest.mark.parametrize("cfg,lean", [(0, "0"), (0, "1"), (1, "0"), (1, "1")])
def test_glu_quant_every_instance(cfg, lean, monkeypatch):
    """Both tile shapes that hold whole groups of h (128 x 128, 64 x 128),
    each in the 4-stage and the lean variant, forced; 9 row tiles (ragged
    for both) and 6 groups (3 k-pairs) of h; ranks 16 + 16 and 32 down."""
    monkeypatch.setenv("W4A4_TILED_CFG", str(cfg))
    monkeypatch.setenv("W4A4_TILED_LEAN", lean)
    monkeypatch.setenv("W4A4_GLU_QUANT_EPILOGUE", "1")
    M, K, H, R, Rd = 140, 640, 384, 16, 32
    x, g, u, d = _layers(M, K, H, 64, R, R, Rd, seed=8100 + cfg + 10 * int(lean))
    up, down = _pack(g, u, d, R, R, Rd)
    _say(f"[glu quant forced] cfg={cfg} lean={lean}")
    act_q, act_r, h = _run_both(x, up, down)
    _compare(act_q, act_r, h.cpu().numpy(), M, H, Rd, d["lora_down"], f"glu quant cfg {cfg} lean {lean}")


@pytest.mark.parametrize("M,route", [(64, "0"), (200, "1"), (64, ""), (200, "")])
def test_glu_quant_routes(M, route, monkeypatch):
    """Both routes at a size where each is the natural choice (H = 3072:
    M = 64 gives 48 workgroups of one group each and goes through the
    activation pass, M = 200 gives 192 and quantizes in the epilogue),
    forced ("0" / "1") and natural: the same codes and scales."""
    if route:
        monkeypatch.setenv("W4A4_GLU_QUANT_EPILOGUE", route)
    K, H, R, Rd = 512, 3072, 16, 32
    x, g, u, d = _layers(M, K, H, 64, R, R, Rd, seed=8300 + M)
    up, down = _pack(g, u, d, R, R, Rd)
    _say(f"[glu quant route] M={M} route={route or 'natural'}")
    act_q, act_r, h = _run_both(x, up, down)
    _compare(act_q, act_r, h.cpu().numpy(), M, H, Rd, d["lora_down"], f"glu quant M={M} route {route or 'natural'}")


def test_glu_quant_reuses_buffers(monkeypatch):
    """Two calls in a row on the same output blob and workspace, the second
    with fewer rows (its own layout inside the same buffers): the second
    result is that of a fresh call."""
    monkeypatch.setenv("W4A4_GLU_QUANT_EPILOGUE", "1")
    torch = _torch()
    K, H, R, Rd = 512, 256, 16, 32
    x, g, u, d = _layers(300, K, H, 64, R, R, Rd, seed=8200)
    up, down = _pack(g, u, d, R, R, Rd)
    big = W.alloc_act_blob(300, H, Rd)
    ws = torch.empty(W.w4a4_glu_quant_workspace(300, 2 * H, Rd), dtype=torch.uint8, device="cuda")
    for M in (300, 37):
        act = W.alloc_act_blob(M, K, up.R)
        W.w4a4_quantize_act(M, K, up.R, _to_dev(x[:M]), up.wblob, act)
        W.w4a4_linear_glu_quant(M, 2 * H, K, up.R, up.r_gate, act, up.wblob, Rd, down.wblob, big, ws)
    torch.cuda.synchronize()
    _, act_r, h = _run_both(x[:37], up, down)
    total, _ = W.w4a4_act_layout(37, H, Rd)
    _compare(big[:total].clone(), act_r, h.cpu().numpy(), 37, H, Rd, d["lora_down"], "glu quant second call")


def test_gated_mlp_workload_chain():
    """The whole MLP at the workload's shapes (M=700 tokens, hidden 1024,
    intermediate 3072, rank 32 on gate, up and down; X with x20 outlier
    channels; gate and up from two seeds of the up-projection recipe, down
    from the down-projection recipe), stage by stage: h's codes and scales
    bit-exact against the oracle's quantizer of the GPU's h, lora_act within
    its bound, and y (GatedMLP.forward: the quantized-output path) at the
    layer bar against the oracle's down layer on that h.  (g, u and h
    themselves are checked against the oracle in test_gpu_mlp.)

    End to end against the oracle's own chain the difference is reported,
    not barred: re-quantizing h amplifies the near-tie differences of h (a
    one-ulp change of a group's absmax moves that group's scale and so all
    its 64 codes), so the oracle chain fed the GPU's h moves by as much; the
    test checks that the GPU's y is no further from the oracle chain than
    that sensitivity plus one layer's bar."""
    g = workloads.generate("mlp_up")
    u = workloads.generate("mlp_up", seed=workloads.WORKLOADS["mlp_up"].seed + 7)
    dcase = workloads.generate("mlp_down")
    x, M, K, H, R = g["x"], g["M"], g["K"], g["N"], g["R"]
    Nd, Rd = dcase["N"], dcase["R"]
    assert dcase["K"] == H
    up, down = _pack(g, u, dcase, R, R, Rd)
    _say(f"[mlp chain] M={M} K={K} H={H} N_down={Nd} R={R}/{Rd}")
    act_q, act_r, h = _run_both(x, up, down)
    hh = h.cpu().numpy()
    _compare(act_q, act_r, hh, M, H, Rd, dcase["lora_down"], "mlp chain h")
    mlp = W.GatedMLP(up, down)
    y = mlp.forward(_to_dev(x))
    _torch().cuda.synchronize()
    y = y.cpu().numpy()
    dargs = dict(col_scale=dcase["col_scale"], bias=dcase["bias"], w16=dcase["w"])
    ref = O.linear(hh, dcase["lora_down"], dcase["lora_up"], **dargs)
    _check_y(y, ref["y"], "mlp chain y on the GPU's h", y64=ref["y64"], ref=ref, case=dcase)
    half = lambda c: dict(lora_down16=c["lora_down"], lora_up16=c["lora_up"], col_scale=c["col_scale"],
                          bias=c["bias"], w16=c["w"])
    _, _, h_or = O.mlp_gate_up(x, half(g), half(u))
    ref2 = O.linear(h_or, dcase["lora_down"], dcase["lora_up"], **dargs)
    y2 = ref2["y"].astype(np.float64)
    rms = np.sqrt(np.mean(y2 ** 2))
    e_gpu = np.abs(y.astype(np.float64) - y2)
    e_or = np.abs(ref["y"].astype(np.float64) - y2)   # the oracle chain on the GPU's h vs on its own
    _say(f"mlp chain end to end: GPU y vs oracle chain max {e_gpu.max() / rms:.3g} mean {e_gpu.mean() / rms:.3g} "
         f"(x rms); oracle chain on the GPU's h vs on its own h: max {e_or.max() / rms:.3g} "
         f"mean {e_or.mean() / rms:.3g}")
    assert e_gpu.max() <= e_or.max() + 2e-2 * rms
    assert e_gpu.mean() <= e_or.mean() + 2e-3 * rms
