"""Offline derivation of a W4A4 + LoRA checkpoint from an fp16 weight (host side).

"W4A4 CUDA Kernel for Voice Clone", sections 2.1-2.3: the int4 weight leaves
an error E = W - Q(W) that a rank-R product proj_up @ proj_down^T absorbs at
run time, and the factors are refined by re-quantizing W minus the current
low-rank part (up to 3 rounds, stopping when the residual stops shrinking).
The pages round with GPTQ, which needs calibration activations that are not
available here; this module rounds to nearest with the same per-(row,
64-group) rule the activation quantizer uses (scale = fp16(fp32(absmax / 7)),
a zero scale replaced by 2^-24, q = clamp(rint(w / scale), -8, 7)).

This runs once per layer at load time, on the host, like the checkpoint
conversion in the pages; it is not on the forward path.  Its outputs are the
checkpoint tensors w4a4_pack_weights takes (qweight [N, K/2] uint8 with the
even k in the low nibble, w_scales [N, K/64] fp16, proj_down [K, R] and
proj_up [N, R] fp16) plus the error figures the pages quote (the share of the
quantization error's energy the low-rank term captures).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def _rtn_groups(w: np.ndarray):
    """Round-to-nearest int4 codes and fp16 scales of each (row, 64-group)."""
    n, k = w.shape
    g = w.astype(np.float16).astype(np.float32).reshape(n, k // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    scale = (amax / np.float32(7.0)).astype(np.float16)
    scale[scale == 0] = np.float16(2.0 ** -24)
    s32 = scale.astype(np.float32)[:, :, None]
    q = np.clip(np.rint(g / s32), -8, 7).astype(np.int8)   # np.rint: half to even
    return q.reshape(n, k), scale


def _dequant(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    n, k = q.shape
    return (q.reshape(n, k // GROUP, GROUP).astype(np.float64) *
            scale.astype(np.float64)[:, :, None]).reshape(n, k)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """int4 codes [N, K] -> qweight [N, K/2]: byte j holds k = 2j in the low
    nibble and k = 2j + 1 in the high nibble, two's complement."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def derive(w16, rank: int, rounds: int = 3):
    """Quantize W (fp16 [N, K]) and derive rank-`rank` LoRA factors.

    Each round quantizes W - L (L = the previous round's low-rank term, 0 at
    first), takes the residual E = W - deq(Q), and sets L to the best rank-R
    approximation of E (truncated SVD); a round whose error
    ||W - deq(Q) - L||_F is not smaller than the previous round's is
    discarded.  Returns a dict with the checkpoint tensors and the error
    figures: rtn_error_norm = ||W - deq(RTN(W))||_F (plain int4, no LoRA),
    first_round_captured = the share of that error's energy the first
    rank-R SVD absorbs (the figure the pages quote for trained weights), and
    residual_norm = ||W - deq(Q) - L||_F of the kept round (factors in fp16)."""
    w = np.asarray(w16, np.float16).astype(np.float64)
    n, k = w.shape
    if k % GROUP or rank < 0 or rank > min(n, k):
        raise ValueError("K must be a multiple of 64 and 0 <= rank <= min(N, K)")
    low = np.zeros_like(w)
    best = None
    history = []
    for _ in range(max(1, rounds)):
        q, scale = _rtn_groups((w - low).astype(np.float16))
        e = w - _dequant(q, scale)
        if rank:
            u, s, vt = np.linalg.svd(e, full_matrices=False)
            up = u[:, :rank] * s[:rank]
            down = vt[:rank].T
        else:
            up = np.zeros((n, 0))
            down = np.zeros((k, 0))
        # the factors as the kernels will see them (fp16)
        up16, down16 = up.astype(np.float16), down.astype(np.float16)
        low_new = up16.astype(np.float64) @ down16.astype(np.float64).T
        resid = float(np.linalg.norm(e - low_new))
        e2 = float(np.sum(e * e))
        captured = 1.0 - resid * resid / e2 if e2 > 0 else 1.0
        if best is not None and resid >= best["residual_norm"]:
            break
        best = dict(q=q, scale=scale, up16=up16, down16=down16, residual_norm=resid,
                    error_norm=float(np.sqrt(e2)), captured=captured)
        history.append(dict(residual_norm=resid, error_norm=float(np.sqrt(e2)), captured=captured))
        low = low_new
    return dict(qweight=pack_nibbles(best["q"]), w_scales=best["scale"],
                proj_down=best["down16"], proj_up=best["up16"], codes=best["q"],
                residual_norm=best["residual_norm"], rtn_error_norm=history[0]["error_norm"],
                first_round_captured=history[0]["captured"], rounds=history,
                weight_norm=float(np.linalg.norm(w)))


def _main(argv=None):
    """python -m w4a4_gemm_lora_amd.svdquant N K R [seed] [lowrank]: derive a
    checkpoint for a seeded synthetic W (N(0, 0.02), or with `lowrank` a
    rank-4 component of the same scale added) and print its error figures."""
    import json
    import sys
    import time
    a = sys.argv[1:] if argv is None else argv
    n, k, r = int(a[0]), int(a[1]), int(a[2])
    seed = int(a[3]) if len(a) > 3 else 20261202
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)) * 0.02
    if len(a) > 4 and a[4] == "lowrank":
        w = w + (rng.standard_normal((n, 4)) @ rng.standard_normal((4, k))) * 0.02 / 2
    t0 = time.perf_counter()
    d = derive(w.astype(np.float16), r)
    print(json.dumps({"N": n, "K": k, "R": r, "weights": "lowrank+N(0,0.02)" if len(a) > 4 else "N(0,0.02)",
                      "rounds_kept": len(d["rounds"]), "first_round_captured": round(d["first_round_captured"], 4),
                      "residual_over_rtn_error": round(d["residual_norm"] / d["rtn_error_norm"], 4),
                      "rtn_error_over_weight": round(d["rtn_error_norm"] / d["weight_norm"], 4),
                      "seconds": round(time.perf_counter() - t0, 2)}))


if __name__ == "__main__":
    _main()
