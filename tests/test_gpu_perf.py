"""Performance regression limits ("High-Performance Kernel Design for W4A4
... on Blackwell", section 5: passing smoke tests does not make a kernel
fast; "INT4 Kernel Architecture, in depth", "Why INT4 kernels exist": small
batches are bound by HBM, large ones by the matrix cores).

Each test times the layer's GEMM the way bench.py reports it -- a graph of
50 back-to-back launches after the clocks have settled, divided into the
method's algorithmic operations or bytes (bench.algorithmic_counts) -- and
holds it to a floor some 15-20% below what the kernels measure on MI355X
(prefill 0.29 of the dense int8 peak; decode 0.55 / 0.48 / 0.48 of HBM at
M = 1 / 4 / 16; the prefill activation pass 0.55 of HBM), so that box-to-box
spread passes and a real regression does not.  Decode rotates the weights
through 12 blobs (384 MB, beyond the 256 MB last-level cache) so that they
stream from HBM.
"""
import numpy as np
import pytest

import bench
import w4a4_gemm_lora_amd as W
from w4a4_gemm_lora_amd import workloads
from tests.test_gpu_parity import _say, _torch

pytestmark = pytest.mark.gpu

PREFILL_INT8_FRAC_FLOOR = 0.25
DECODE_HBM_FRAC_FLOOR = {1: 0.45, 4: 0.40, 16: 0.40}
ACT_PASS_HBM_FRAC_FLOOR = 0.45


def _linear_ms(case, rotate):
    torch = _torch()
    M, K, N, R = case["M"], case["K"], case["N"], case["R"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    src = dict(w_fp16=dev(case["w"]), lora_down=dev(case["lora_down"]), lora_up=dev(case["lora_up"]),
               col_scale=dev(case["col_scale"]), bias=dev(case["bias"]))
    blobs = []
    for _ in range(rotate):   # the same packed weights at `rotate` addresses
        wb = W.alloc_weight_blob(N, K, R)
        W.w4a4_pack_weights(N, K, R, wb, **src)
        blobs.append(wb)
    del src
    act = W.alloc_act_blob(M, K, R)
    W.w4a4_quantize_act(M, K, R, dev(case["x"]), blobs[0], act)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    return bench.graph_avg_ms(torch, lambda i, cs: W.w4a4_linear(M, N, K, R, act, blobs[i % rotate], y, stream=cs),
                              50, settle_ms=300.0)


def test_prefill_int8_fraction_floor():
    """M=8192, K=N=4096, rank 32: the GEMM's layer operations per second
    against the 5.0 POP/s dense int8 peak."""
    case = workloads.generate("prefill")
    ms = _linear_ms(case, 1)
    c = bench.algorithmic_counts(case["M"], case["N"], case["K"], case["R"])
    frac = c["lin_ops"] / (ms * 1e-3) / 1e12 / bench.PEAK_INT8_TOPS
    _say(f"[perf] prefill linear {ms * 1e3:.1f} us = {frac:.3f} of the int8 peak (floor {PREFILL_INT8_FRAC_FLOOR})")
    assert frac >= PREFILL_INT8_FRAC_FLOOR


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_hbm_fraction_floor(M):
    """K=4096, N=14336, rank 32: the GEMM's algorithmic bytes per second
    against the 8 TB/s HBM peak."""
    case = workloads.generate("decode", M=M)
    ms = _linear_ms(case, 12)
    c = bench.algorithmic_counts(case["M"], case["N"], case["K"], case["R"])
    frac = c["lin_bytes"] / (ms * 1e-3) / 1e9 / bench.PEAK_HBM_GBPS
    _say(f"[perf] decode M={M} linear {ms * 1e3:.2f} us = {frac:.3f} of HBM (floor {DECODE_HBM_FRAC_FLOOR[M]})")
    assert frac >= DECODE_HBM_FRAC_FLOOR[M]


def test_prefill_activation_pass_hbm_floor():
    """M=8192, K=4096, rank 32: the activation pass's algorithmic bytes (X,
    L_down, codes, scales, lora_act) per second against the 8 TB/s HBM peak."""
    torch = _torch()
    case = workloads.generate("prefill")
    M, K, N, R = case["M"], case["K"], case["N"], case["R"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    wb = W.alloc_weight_blob(N, K, R)
    W.w4a4_pack_weights(N, K, R, wb, w_fp16=dev(case["w"]), lora_down=dev(case["lora_down"]),
                        lora_up=dev(case["lora_up"]), col_scale=dev(case["col_scale"]), bias=dev(case["bias"]))
    x = dev(case["x"])
    act = W.alloc_act_blob(M, K, R)
    torch.cuda.synchronize()
    ms = bench.graph_avg_ms(torch, lambda i, cs: W.w4a4_quantize_act(M, K, R, x, wb, act, stream=cs), 50,
                            settle_ms=300.0)
    c = bench.algorithmic_counts(M, N, K, R)
    frac = c["q_bytes"] / (ms * 1e-3) / 1e9 / bench.PEAK_HBM_GBPS
    _say(f"[perf] prefill activation pass {ms * 1e3:.1f} us = {frac:.3f} of HBM (floor {ACT_PASS_HBM_FRAC_FLOOR})")
    assert frac >= ACT_PASS_HBM_FRAC_FLOOR
