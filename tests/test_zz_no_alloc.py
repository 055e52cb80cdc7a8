"""GPU check of w4a4_linear_glu_quant_noalloc (the allocation-free variant
of the quantized gated output, whose workspace is a library-owned device
array) against w4a4_linear_glu_quant with a workspace of its own: the same
activation blob bit for bit, on two calls in a row, the second with a
smaller input (the array then holds the first call's contents)."""
import numpy as np
import pytest

import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from tests.test_gpu_parity import _say, _to_dev, _torch

pytestmark = pytest.mark.gpu


def _layers(M, K, H, R, Rd, seed):
    g = workloads.random_case(M, K, H, R, seed=seed)
    u = workloads.random_case(M, K, H, R, seed=seed + 1)
    d = workloads.random_case(M, H, 64, Rd, seed=seed + 2)
    dev = _to_dev
    up = W.GatedMLPUp(H, K, dev(g["w"]), dev(u["w"]), dev(g["lora_down"]), dev(g["lora_up"]),
                      dev(u["lora_down"]), dev(u["lora_up"]), dev(g["col_scale"]), dev(g["bias"]),
                      dev(u["col_scale"]), dev(u["bias"]))
    down = W.PackedLinear(64, H, Rd, w_fp16=dev(d["w"]), lora_down=dev(d["lora_down"]), lora_up=dev(d["lora_up"]))
    return g["x"], up, down


def test_noalloc_matches_workspace_variant_twice():
    """First call: M=700, 3072 columns of h (the quantizing epilogue, 4.3 MB
    of LoRA-down shares in the array); second: M=40 (h through the array and
    the activation pass), each against the variant with its own workspace."""
    torch = _torch()
    K, H, R, Rd = 1024, 3072, 16, 32
    x, up, down = _layers(700, K, H, R, Rd, seed=9100)
    for M in (700, 40):
        act = W.alloc_act_blob(M, K, up.R)
        W.w4a4_quantize_act(M, K, up.R, _to_dev(x[:M]), up.wblob, act)
        ref = W.alloc_act_blob(M, H, Rd)
        ref.fill_(0xA5)
        ws = torch.empty(W.w4a4_glu_quant_workspace(M, 2 * H, Rd), dtype=torch.uint8, device="cuda")
        W.w4a4_linear_glu_quant(M, 2 * H, K, up.R, up.r_gate, act, up.wblob, Rd, down.wblob, ref, ws)
        got = W.alloc_act_blob(M, H, Rd)
        got.fill_(0x3C)
        W.w4a4_linear_glu_quant_noalloc(M, 2 * H, K, up.R, up.r_gate, act, up.wblob, Rd, down.wblob, got)
        torch.cuda.synchronize()
        same = np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
        _say(f"[noalloc] M={M}: activation blob identical to the workspace variant's: {same}")
        assert same, f"M={M}: the allocation-free variant's activation blob differs"
