"""Writer of the library's Q1 plane layout, for the byte-for-byte check of
the repack kernel (test infrastructure; not part of the oracle, which holds
only the pages' arithmetic). The layout is the library's own, declared in
include/gemm_decode.h ("Q1 planes"); the page "browseml-gpu.js" (packQ1)
fixes only what it must carry: each block's f16 scale and its 128 sign bits.
Integer byte moves in numpy, from that declaration:

  R64 = rows rounded up to 64, nb = K/128, nb8 = nb rounded up to 8.
  bits  : u32 [R64/64][nb][2 halves][64][2]; word m of half h of (row r,
          block i) holds the sign bits of elements 32k + 4l + j with
          l = 4h + jj (jj < 4), k = 2m + kk (kk < 2), j < 4, at bit
          (8*jj + 2 + 4*kk + j) mod 32.
  scales: u16 [R64/64][nb8/8][64][8]; entry (r, i) = the f16 bits of d0.
  Padding rows and padding blocks are zero.
"""
import numpy as np


def plane_sizes(rows: int, K: int):
    nb = K // 128
    nb8 = (nb + 7) // 8 * 8
    r64 = (rows + 63) // 64 * 64
    return r64 * nb * 4, r64 * nb8


def element_position(e: int):
    """(half h, word m, bit) that element e (0..127) of a block occupies."""
    k, l, j = e // 32, (e % 32) // 4, e % 4
    h, jj, m, kk = l // 4, l % 4, k // 2, k % 2
    return h, m, (8 * jj + 2 + 4 * kk + j) % 32


def q1_planes(w_aos, rows: int, K: int):
    """(bits u32 [...], scales u16 [...]) of AoS Q1_0 weight bytes."""
    nb = K // 128
    nb8 = (nb + 7) // 8 * 8
    r64 = (rows + 63) // 64 * 64
    W = np.ascontiguousarray(w_aos, dtype=np.uint8).reshape(rows, nb, 18)
    signs = np.unpackbits(W[:, :, 2:], axis=2, bitorder="little").astype(np.uint32)   # [rows, nb, 128]
    bits = np.zeros((r64 // 64, nb, 2, 64, 2), dtype=np.uint32)
    words = np.zeros((rows, nb, 2, 2), dtype=np.uint32)
    for e in range(128):
        h, m, pos = element_position(e)
        words[:, :, h, m] |= signs[:, :, e] << np.uint32(pos)
    r = np.arange(rows)
    bits[r // 64, :, :, r % 64, :] = words                     # [rows, nb, 2, 2] into (t, i, h, lane, m)
    scales = np.zeros((r64 // 64, nb8 // 8, 64, 8), dtype=np.uint16)
    d0 = W[:, :, 0:2].copy().view("<u2")[:, :, 0]              # [rows, nb]
    i = np.arange(nb)
    scales[(r // 64)[:, None], (i // 8)[None, :], (r % 64)[:, None], (i % 8)[None, :]] = d0
    return bits.reshape(-1), scales.reshape(-1)
