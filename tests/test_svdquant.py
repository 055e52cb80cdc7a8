"""Offline LoRA-factor derivation (w4a4_gemm_lora_amd.svdquant) on the host:
its round-to-nearest agrees with the oracle's quantizer, its factors are a
truncated SVD of the quantization error, and the derived checkpoint makes the
layer more accurate than plain int4 (checked with the oracle)."""
import numpy as np

from oracle import w4a4_oracle as O
from w4a4_gemm_lora_amd import svdquant as S


def test_rtn_matches_oracle_quantizer_and_checkpoint_packing():
    """Two independent implementations of the pages' rounding rule give the
    same codes and scales bit for bit, including ties and all-zero groups;
    qweight unpacks (oracle's checkpoint reader) to the same codes."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((48, 320)) * 0.05).astype(np.float16)
    w[3, :64] = 0                                    # all-zero group
    w[5, 64:128] = np.float16(0.7)                   # constant group
    w[7, 128:192] = (np.arange(64) % 16 - 7).astype(np.float16) * np.float16(0.125)   # grid values and ties
    d = S.derive(w, rank=0, rounds=1)
    qx, sx = O.quantize_groups(w)
    assert np.array_equal(d["codes"], qx)
    assert np.array_equal(d["w_scales"].view(np.uint16), sx.view(np.uint16))
    assert np.array_equal(O.unpack_qweight(d["qweight"], 320), qx)
    assert d["proj_down"].shape == (320, 0) and d["proj_up"].shape == (48, 0)


def test_factors_are_truncated_svd_of_the_error():
    """With one refinement round (rounds=1) the factors are the best rank-R
    approximation of E = W - deq(Q) (Eckart-Young): the residual equals the
    norm of E's trailing singular values (up to the fp16 rounding of the
    factors), and full rank leaves almost nothing."""
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((64, 128)) * 0.02).astype(np.float16)
    q, s = O.quantize_groups(w)
    e = w.astype(np.float64) - q.astype(np.float64) * np.repeat(s.astype(np.float64), 64, axis=1)
    sv = np.linalg.svd(e, compute_uv=False)
    for R in (4, 16):
        d = S.derive(w, rank=R, rounds=1)
        tail = np.sqrt(np.sum(sv[R:] ** 2))
        assert abs(d["residual_norm"] - tail) <= 2e-3 * np.linalg.norm(e)
        assert abs(d["first_round_captured"] - (1 - tail ** 2 / np.sum(sv ** 2))) < 1e-2
    d = S.derive(w, rank=64, rounds=1)
    assert d["residual_norm"] <= 2e-3 * np.linalg.norm(e)


def test_rounds_never_increase_the_residual():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((96, 6)) @ rng.standard_normal((6, 256))
    w = (a * 0.01 + rng.standard_normal((96, 256)) * 0.01).astype(np.float16)
    d = S.derive(w, rank=8, rounds=3)
    res = [r["residual_norm"] for r in d["rounds"]]
    assert all(b < a_ for a_, b in zip(res, res[1:]))
    assert d["residual_norm"] == res[-1] < d["rtn_error_norm"]


def test_derived_checkpoint_recovers_accuracy():
    """The point of the LoRA branch (pages, section 2.1): with the derived
    factors the W4A4 layer is closer to the fp16 matmul X W^T than plain
    int4 is."""
    rng = np.random.default_rng(14)
    M, K, N, R = 32, 512, 96, 32
    a = rng.standard_normal((N, 4)) @ rng.standard_normal((4, K))
    w = (a * 0.02 + rng.standard_normal((N, K)) * 0.01).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    d = S.derive(w, rank=R)
    y_lora = O.linear(x, d["proj_down"], d["proj_up"], qweight=d["qweight"], w_scales=d["w_scales"])["y64"]
    d0 = S.derive(w, rank=0, rounds=1)
    y_rtn = O.linear(x, None, None, qweight=d0["qweight"], w_scales=d0["w_scales"])["y64"]
    err_lora = np.linalg.norm(y_lora - exact)
    err_rtn = np.linalg.norm(y_rtn - exact)
    assert err_lora < err_rtn, (err_lora, err_rtn)
