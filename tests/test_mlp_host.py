"""Host-side pieces of the gated MLP front half (no GPU): the (gate, up)
row interleave that w4a4_linear_glu pairs, and GatedMLPUp's argument checks."""
import pytest
import torch

import w4a4_gemm_lora_amd as W


def test_interleave_gate_up_row_order():
    """Rows [32j, 32j+16) of the packed layer are gate rows [16j, 16j+16),
    rows [32j+16, 32j+32) up rows [16j, 16j+16); 1-D vectors (a, b) follow
    the same order, and the interleave of the identity pair inverts."""
    n, k = 48, 5
    gate = torch.arange(n * k, dtype=torch.float32).reshape(n, k)
    up = -1.0 - gate
    w = W.interleave_gate_up(gate, up)
    assert w.shape == (2 * n, k)
    for j in range(n // 16):
        assert torch.equal(w[32 * j:32 * j + 16], gate[16 * j:16 * j + 16])
        assert torch.equal(w[32 * j + 16:32 * j + 32], up[16 * j:16 * j + 16])
    a = W.interleave_gate_up(torch.arange(n), torch.arange(n) + 1000)
    assert a[:16].tolist() == list(range(16)) and a[16:32].tolist() == list(range(1000, 1016))
    back = w.reshape(n // 16, 2, 16, k)
    assert torch.equal(back[:, 0].reshape(n, k), gate) and torch.equal(back[:, 1].reshape(n, k), up)


def test_gated_layer_argument_checks():
    w = torch.zeros((40, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        W.GatedMLPUp(40, 128, w, w)                        # 40 columns: not whole 16-column tiles
    w = torch.zeros((32, 128), dtype=torch.float16)
    ld = torch.zeros((128, 16), dtype=torch.float16)
    with pytest.raises(ValueError):
        W.GatedMLPUp(32, 128, w, w, lora_down_gate=ld)     # L_down without L_up
