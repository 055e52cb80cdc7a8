"""Unpack the library's blobs into plain row-major arrays (test helper).

Written from the layout description in include/w4a4.h, independently of the
HIP packers, so that comparing unpacked GPU blobs against the oracle checks
the packers too.  numpy only; no method arithmetic.
"""
import numpy as np


def unpack_codes(buf, rows_p, K):
    """Code tiles [rows_p/16][K/128][1024 B] -> int8 [rows_p, K].

    Lane l = r + 16c owns bytes [16l, 16l+16); bytes 0..7 = group 0 of the
    tile, 8..15 = group 1; byte b holds k = 16c + 2b (low nibble) and
    16c + 2b + 1 (high nibble) within its group."""
    MT, KP = rows_p // 16, K // 128
    t = np.asarray(buf, np.uint8)[: MT * KP * 1024].reshape(MT, KP, 4, 16, 2, 8)  # mt p c r j b
    nib = np.stack([t & 0xF, t >> 4], axis=-1)                                   # ... e
    nib = nib.transpose(0, 3, 1, 4, 2, 5, 6)                                     # mt r p j c b e
    q = nib.reshape(rows_p, K).astype(np.int16)
    return np.where(q >= 8, q - 16, q).astype(np.int8)


def unpack_scales(buf, rows_p, K):
    """fp16 [rows_p/16][K/128][16][2] -> fp16 [rows_p, K/64]."""
    MT, KP = rows_p // 16, K // 128
    s = np.asarray(buf).view(np.uint16)[: MT * KP * 32].reshape(MT, KP, 16, 2)
    return s.transpose(0, 2, 1, 3).reshape(rows_p, K // 64).view(np.float16)


def unpack_lora_up(buf, N, R):
    """fp16 [N/16][R/16][64][4], (nt, t, l=i+16c, j) = L_up[16nt+i][16t+4c+j]."""
    u = np.asarray(buf).view(np.uint16)[: N * R].reshape(N // 16, R // 16, 4, 16, 4)  # nt t c i j
    return u.transpose(0, 3, 1, 2, 4).reshape(N, R).view(np.float16)


def unpack_lora_down(buf, K, R):
    """fp16 [K/128][R/16][4][64][8],
    (p, t, s, l=n+16c, j) = L_down[128p + 64(s/2) + 16c + 8(s%2) + j][16t+n]."""
    d = np.asarray(buf).view(np.uint16)[: K * R].reshape(K // 128, R // 16, 2, 2, 4, 16, 8)  # p t sj sh c n j
    return d.transpose(0, 2, 4, 3, 6, 1, 5).reshape(K, R).view(np.float16)


def split_weight_blob(blob, N, K, R, offsets):
    """Slice a host copy (uint8) of a weight blob into its sections."""
    b = np.asarray(blob, np.uint8)
    o = offsets
    G = K // 64
    return dict(
        lora_down=unpack_lora_down(b[o[0]: o[0] + K * R * 2], K, R) if R else None,
        qw=unpack_codes(b[o[1]: o[1] + N * K // 2], N, K),
        sw=unpack_scales(b[o[2]: o[2] + N * G * 2], N, K),
        lora_up=unpack_lora_up(b[o[3]: o[3] + N * R * 2], N, R) if R else None,
        a=b[o[4]: o[4] + 4 * N].view(np.float32),
        b=b[o[5]: o[5] + 4 * N].view(np.float32),
    )


def split_act_blob(blob, M, K, R, offsets, splits=1):
    """Sections of an activation blob; lora_act is the in-order sum of the
    `splits` fp32 partials [splits][Mp][R]."""
    b = np.asarray(blob, np.uint8)
    o = offsets
    Mp = (M + 15) // 16 * 16
    G = K // 64
    parts = b[o[2]: o[2] + splits * Mp * R * 4].view(np.float32).reshape(splits, Mp, R)
    la = np.zeros((Mp, R), np.float32)
    for j in range(splits):
        la = (la + parts[j]).astype(np.float32)
    return dict(
        qx=unpack_codes(b[o[0]: o[0] + Mp * K // 2], Mp, K),
        sx=unpack_scales(b[o[1]: o[1] + Mp * G * 2], Mp, K),
        lora_act=la, lora_parts=parts,
        Mp=Mp,
    )
