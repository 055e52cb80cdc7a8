"""The test-side unpacker against hand-placed bytes (CPU)."""
import numpy as np

from tests.layout_unpack import unpack_codes, unpack_scales, unpack_lora_up, unpack_lora_down


def test_unpack_codes_hand_placed_nibbles():
    K = 256
    buf = np.zeros(2 * 1024, np.uint8)  # 16 rows, two k-pairs
    # tile p=1, lane l = r + 16c with r=5, c=2; group 1 (bytes 8..15); byte b=3
    lane = 5 + 16 * 2
    buf[1024 + 16 * lane + 8 + 3] = 0x9A   # low nibble 0xA = -6, high 0x9 = -7
    q = unpack_codes(buf, 16, K)
    k_lo = 128 * 1 + 64 * 1 + 16 * 2 + 2 * 3
    assert q[5, k_lo] == -6 and q[5, k_lo + 1] == -7
    assert np.count_nonzero(q) == 2


def test_unpack_scales_and_lora_layouts():
    K, R, N = 256, 32, 32
    s = np.arange(2 * 2 * 16 * 2, dtype=np.uint16)  # [mt=2][p=2][16][2]
    out = unpack_scales(s.view(np.float16), 32, K).view(np.uint16)
    assert out[16 + 3, 2 * 1 + 1] == ((1 * 2 + 1) * 16 + 3) * 2 + 1
    lu = np.arange(N * R, dtype=np.uint16)
    up = unpack_lora_up(lu.view(np.float16), N, R).view(np.uint16)
    # (nt=1, t=1, l = i + 16c with i=7, c=3, j=2) -> L_up[16+7][16+12+2]
    assert up[23, 30] == ((1 * 2 + 1) * 64 + (7 + 16 * 3)) * 4 + 2
    ld = np.arange(K * R, dtype=np.uint16)
    dn = unpack_lora_down(ld.view(np.float16), K, R).view(np.uint16)
    # (p=1, t=0, s=3, l = n + 16c with n=9, c=1, j=5) -> L_down[128+64+16+8+5][9]
    assert dn[221, 9] == (((1 * 2 + 0) * 4 + 3) * 64 + (9 + 16)) * 8 + 5
