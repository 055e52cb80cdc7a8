"""Plain, slow, obviously correct CPU oracle for the W4A4 + LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may.  It shares no code, table or constant generator with the HIP
kernels in ``w4a4_gemm_lora_amd/csrc``.

What it computes (numpy; fp64 wherever the method does not fix a precision):

    Y[m,n] = fp16( a[n] * ( sum_g s_x[m,g] s_w[n,g] P[m,n,g]
                            + sum_r lora_act[m,r] L_up[n,r] ) + b[n] )
    P[m,n,g]       = sum_{k in group g} q_x[m,k] q_w[n,k]        (exact int)
    lora_act[m,r]  = sum_k X[m,k] L_down[k,r]                    (unquantized X)

Sources (the pages a reader of this file has):

* "W4A4 CUDA Kernel for Voice Clone: From Profiling to 2.6x Faster Than FP16"
  - section 2.1: the low-rank correction Y = INT4_GEMM(X, Q(W)) +
    X @ proj_down @ proj_up^T with proj_down [K, R], proj_up [N, R];
  - section 2.3: checkpoint tensors qweight [N, K/2] (two int4 per byte),
    w_scales [N, K/64] fp16;
  - section 3.2: quantization group size 64 along K;
  - section 3.6, quantize path: per (row, 64-group) absmax, scale =
    absmax / 7, q = round-to-nearest of x / scale clamped to [-8, 7], stored
    as the low 4 bits of q (two's complement);
  - section 3.6, LoRA-down branch: reads the fp16 X tile (not the quantized one);
  - section 3.7, per-group dequant: int32 group sum times activation scale
    times weight scale, accumulated over groups; LoRA-up added to the same
    accumulator.
* "High-Performance Kernel Design for W4A4 Quantized Matrix Multiplication on
  Blackwell Architecture", section 1: output = scaled low-bit matmul +
  low-rank residual + column-wise affine.
* "INT4 Kernel Architecture, in depth", section "Failure modes" and the
  per-layer validation listing: check each layer against a dequantized
  reference.

Readings where the pages are silent or inconsistent (each is listed with its
reason in the design notes of this repository):

1. The value divided by is the *stored* fp16 scale (converted exactly to fp32),
   so the integer grid the GEMM multiplies by is the grid the value was
   rounded to.  The scale itself is fp32(absmax / 7) rounded to fp16 (RNE).
2. The pages floor the fp32 scale at 1e-10, which is 0 in fp16; the floor is
   applied to the fp16 scale instead: a zero scale becomes 2^-24 (the
   smallest positive fp16), so an all-zero group quantizes to q = 0.
3. Rounding is round-half-to-even (the pages' round-to-nearest intrinsic),
   after an IEEE fp32 division.
4. Accumulation over groups is exact-ish (fp64) rather than the pages' fp16.
5. The column-wise affine is y = a[n] * (main + lora) + b[n], a and b fp32.
6. checkpoint nibble order: low nibble = even k; two's complement.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
QMIN, QMAX = -8, 7
FP16_MIN_SUBNORMAL = np.float16(2.0 ** -24)   # bit pattern 0x0001


def to_fp16(v) -> np.ndarray:
    """Round to IEEE binary16, nearest-even (numpy's float->half conversion)."""
    return np.asarray(v).astype(np.float16)


# ----------------------------------------------------------------------------
# Quantizer ("W4A4 CUDA Kernel for Voice Clone", section 3.6, quantize path)
# ----------------------------------------------------------------------------
def quantize_groups(v16: np.ndarray):
    """Symmetric signed int4 quantization, one scale per (row, 64-wide group).

    v16: float16 [rows, K], K a multiple of 64.
    Returns (q int8 [rows, K] in [-8, 7], s float16 [rows, K/64]).

    Per group: amax = max |v| (exact); s = fp16(fp32(amax / 7)), with a zero
    scale replaced by 2^-24; q = clamp(rint(fp32(v) / fp32(s)), -8, 7) where
    the division is IEEE fp32 and rint is half-to-even.
    """
    v16 = np.asarray(v16, dtype=np.float16)
    rows, K = v16.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    G = K // GROUP
    v32 = v16.astype(np.float32).reshape(rows, G, GROUP)      # exact widening
    amax = np.max(np.abs(v32), axis=2)                         # exact
    s32 = amax / np.float32(7.0)                               # IEEE fp32 division
    s16 = s32.astype(np.float16)                               # RNE to fp16
    s16 = np.where(s16 == 0, FP16_MIN_SUBNORMAL, s16).astype(np.float16)
    ratio = v32 / s16.astype(np.float32)[:, :, None]           # IEEE fp32 division
    q = np.clip(np.rint(ratio), QMIN, QMAX).astype(np.int8)    # half-to-even
    return q.reshape(rows, K), s16


def unpack_qweight(qweight: np.ndarray, K: int) -> np.ndarray:
    """Checkpoint nibbles [N, K/2] uint8 -> int8 [N, K].

    Byte j of a row holds k = 2j in its low nibble and k = 2j+1 in its high
    nibble; each nibble is a two's-complement 4-bit integer
    ("W4A4 CUDA Kernel for Voice Clone", section 2.3 and the nibble store in
    section 3.6)."""
    qweight = np.asarray(qweight, dtype=np.uint8)
    N = qweight.shape[0]
    assert qweight.shape[1] * 2 == K
    lo = (qweight & 0x0F).astype(np.int16)
    hi = (qweight >> 4).astype(np.int16)
    nib = np.empty((N, K), np.int16)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


# ----------------------------------------------------------------------------
# Integer group sums and the scaled main term (section 3.7, per-group dequant)
# ----------------------------------------------------------------------------
def group_psums(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P[m, n, g] = sum over k in group g of qx[m,k] * qw[n,k]  (int32).

    The per-group products are formed as fp64 matrix products of small
    integers: every partial sum is an integer of magnitude <= 64*64 < 2^53, so
    the library matmul is exact in any summation order."""
    M, K = qx.shape
    N = qw.shape[0]
    G = K // GROUP
    P = np.empty((M, N, G), np.int32)
    for g in range(G):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        a = qx[:, ks].astype(np.float64)
        b = qw[:, ks].astype(np.float64)
        P[:, :, g] = np.rint(a @ b.T).astype(np.int32)
    return P


def main_term(qx, sx, qw, sw) -> np.ndarray:
    """main[m,n] = sum_g s_x[m,g] * s_w[n,g] * P[m,n,g], evaluated in fp64."""
    M, K = qx.shape
    N = qw.shape[0]
    G = K // GROUP
    sx64 = np.asarray(sx, np.float16).astype(np.float64)
    sw64 = np.asarray(sw, np.float16).astype(np.float64)
    out = np.zeros((M, N), np.float64)
    for g in range(G):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        Pg = np.rint(qx[:, ks].astype(np.float64) @ qw[:, ks].astype(np.float64).T)
        out += (sx64[:, g][:, None] * sw64[:, g][None, :]) * Pg
    return out


# ----------------------------------------------------------------------------
# Low-rank correction (section 2.1; LoRA-down on fp16 X, section 3.6)
# ----------------------------------------------------------------------------
def lora_act(x16: np.ndarray, lora_down16: np.ndarray) -> np.ndarray:
    """lora_act[m, r] = sum_k X[m,k] * L_down[k,r] in fp64 (unquantized X)."""
    return np.asarray(x16).astype(np.float64) @ np.asarray(lora_down16).astype(np.float64)


def lora_term(la: np.ndarray, lora_up16: np.ndarray) -> np.ndarray:
    """lora[m, n] = sum_r lora_act[m,r] * L_up[n,r] in fp64."""
    return la @ np.asarray(lora_up16).astype(np.float64).T


# ----------------------------------------------------------------------------
# The whole layer (column-wise affine: Blackwell article, section 1)
# ----------------------------------------------------------------------------
def quantize_weights(w16=None, qweight=None, w_scales=None, K=None):
    """Weight codes and scales: RTN of fp16 W by the activation rule, or the
    checkpoint pair (qweight, w_scales) taken as given."""
    if w16 is not None:
        return quantize_groups(w16)
    qw = unpack_qweight(qweight, K)
    return qw, np.asarray(w_scales, np.float16)


def linear(x16, lora_down16, lora_up16, col_scale=None, bias=None,
           w16=None, qweight=None, w_scales=None, rows=None, cols=None):
    """Evaluate the layer; returns a dict with Y (fp16) and every intermediate.

    rows / cols: optional index arrays selecting output rows / columns (each
    row of X and each row of W is quantized on its own, so a subset gives the
    same values as the full evaluation restricted to it).
    """
    x16 = np.asarray(x16, np.float16)
    K = x16.shape[1]
    if rows is not None:
        x16 = x16[np.asarray(rows)]
    if w16 is not None:
        w16 = np.asarray(w16, np.float16)
        if cols is not None:
            w16 = w16[np.asarray(cols)]
    else:
        qweight = np.asarray(qweight, np.uint8)
        w_scales = np.asarray(w_scales, np.float16)
        if cols is not None:
            qweight = qweight[np.asarray(cols)]
            w_scales = w_scales[np.asarray(cols)]
    qx, sx = quantize_groups(x16)
    qw, sw = quantize_weights(w16, qweight, w_scales, K)
    N = qw.shape[0]
    a = np.ones(N) if col_scale is None else np.asarray(col_scale, np.float32).astype(np.float64)
    b = np.zeros(N) if bias is None else np.asarray(bias, np.float32).astype(np.float64)
    if cols is not None:
        if col_scale is not None:
            a = a[np.asarray(cols)]
        if bias is not None:
            b = b[np.asarray(cols)]
    main = main_term(qx, sx, qw, sw)
    R = 0 if lora_down16 is None else np.asarray(lora_down16).shape[1]
    if R:
        lu = np.asarray(lora_up16, np.float16)
        if cols is not None:
            lu = lu[np.asarray(cols)]
        la = lora_act(x16, lora_down16)
        lo = lora_term(la, lu)
    else:
        la = np.zeros((x16.shape[0], 0))
        lo = np.zeros_like(main)
    y64 = a[None, :] * (main + lo) + b[None, :]
    return dict(y=to_fp16(y64), y64=y64, main=main, lora=lo, lora_act=la,
                qx=qx, sx=sx, qw=qw, sw=sw)


def quantize_act(x16, lora_down16):
    """What the activation pass produces: q_x, s_x and lora_act."""
    qx, sx = quantize_groups(x16)
    la = lora_act(x16, lora_down16) if lora_down16 is not None else None
    return qx, sx, la


def rms_norm(x16, gamma16, eps: float) -> np.ndarray:
    """Row-wise RMSNorm of fp16 X into fp16, the way the fused norm +
    quantize pass defines it.

    Sources: "W4A4 CUDA Kernel for Voice Clone", section 3.1 (every projection
    input of the Qwen3 layer comes out of an RMSNorm: input_layernorm before
    q/k/v, post_attention_layernorm before gate/up) and section 3.9 (kernel 5
    computes 1 / sqrt(mean(x^2) + eps) per row over all K columns, which the
    quantizer then reads).  The pages give no formula for the learned weight;
    the reading here is the usual RMSNorm y = x * inv_rms * gamma[k].

    Fixed arithmetic (so that the codes are reproducible bit for bit):
        ms    = (sum_k x[m,k]^2) / K          fp64
        inv   = 1 / sqrt(ms + eps)            fp64
        t     = (x * inv) * gamma[k]          fp64, two roundings, in this order
        x_out = fp16(fp32(t))                 round to fp32 first, then to fp16 (RNE)
    """
    x = np.asarray(x16, np.float16).astype(np.float64)
    g = np.asarray(gamma16, np.float16).astype(np.float64)
    K = x.shape[1]
    ss = (x * x).sum(axis=1)                    # each x^2 is exact in fp64
    inv = 1.0 / np.sqrt(ss / K + eps)
    t = (x * inv[:, None]) * g[None, :]
    return t.astype(np.float32).astype(np.float16)


def quantize_act_rmsnorm(x16, gamma16, eps, lora_down16):
    """The fused pass: RMSNorm (rms_norm above), then the activation
    quantizer and LoRA-down on the normalized fp16 rows.  Returns
    (x_norm, q_x, s_x, lora_act)."""
    xn = rms_norm(x16, gamma16, eps)
    qx, sx, la = quantize_act(xn, lora_down16)
    return xn, qx, sx, la


def silu(v) -> np.ndarray:
    """SiLU(v) = v / (1 + exp(-v)) in fp64 ("W4A4 CUDA Kernel for Voice
    Clone", section 3.1: the Qwen3 MLP computes SiLU(gate) * up)."""
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def glu(g16, u16) -> np.ndarray:
    """The MLP's gated activation on the fp16 outputs of the gate and up
    projections: h = fp16(SiLU(g) * u), SiLU and the product in fp64."""
    g = np.asarray(g16, np.float16).astype(np.float64)
    u = np.asarray(u16, np.float16).astype(np.float64)
    return to_fp16(silu(g) * u)


def mlp_gate_up(x16, gate: dict, up: dict):
    """Gate and up projections of the same X (each a dict of linear()'s
    keyword arguments: lora_down16, lora_up16, col_scale, bias, w16 or
    qweight/w_scales) and the gated activation.  Returns (g, u, h)."""
    g = linear(x16, **gate)["y"]
    u = linear(x16, **up)["y"]
    return g, u, glu(g, u)


def ops_count(M, N, K, R) -> int:
    """Useful operations of one layer evaluation: 2MNK for the int4 product
    plus 2MR(K+N) for the two low-rank products."""
    return 2 * M * N * K + 2 * M * R * (K + N)
