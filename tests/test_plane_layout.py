"""Pins for the test helper that writes the library's Q1 plane layout
(tests/q1_layout.py), the reference the repack kernel is compared with byte
for byte.

The layout is the library's own (declared in include/gemm_decode.h, "Q1
planes"); the page "browseml-gpu.js" (packQ1) only fixes what it must carry:
each block's f16 scale and its 128 sign bits. Pinned here by single-element
closed forms (one sign bit set lands at exactly the declared position) and a
full round trip back to the AoS bytes.
"""
import numpy as np
import pytest

import workloads as wl
from q1_layout import q1_planes


def declared_pos(e):
    """(u32 index within the block for row 0, bit) of element e of a block."""
    k, l, j = e // 32, (e % 32) // 4, e % 4
    h, jj, m, kk = l // 4, l % 4, k // 2, k % 2
    return h * 128 + m, (8 * jj + 2 + 4 * kk + j) % 32


def test_each_element_lands_at_declared_bit():
    rows, K = 1, 128
    for e in range(128):
        W = np.zeros((1, 1, 18), dtype=np.uint8)
        W[0, 0, 0:2] = [0x00, 0x3C]
        W[0, 0, 2 + e // 8] = 1 << (e % 8)
        bits, scales = q1_planes(W, rows, K)
        idx, pos = declared_pos(e)
        want = np.zeros(64 * 4, dtype=np.uint32)
        want[idx] = np.uint32(1) << np.uint32(pos)   # row 0 -> lane 0
        assert np.array_equal(bits, want), e
        assert scales[0] == 0x3C00 and not scales[1:].any()


def test_positions_are_a_permutation():
    seen = set()
    for e in range(128):
        seen.add(declared_pos(e))
    assert len(seen) == 128


def _decode_planes(bits, scales, rows, K):
    """Inverse map written from the declared layout."""
    nb = K // 128
    nb8 = (nb + 7) // 8 * 8
    W = np.zeros((rows, nb, 18), dtype=np.uint8)
    for r in range(rows):
        t, lane = divmod(r, 64)
        for i in range(nb):
            h = int(scales[((t * (nb8 // 8) + i // 8) * 64 + lane) * 8 + i % 8])
            W[r, i, 0], W[r, i, 1] = h & 0xFF, h >> 8
            for e in range(128):
                idx, pos = declared_pos(e)
                h, m = divmod(idx, 128)
                word = int(bits[(((t * nb + i) * 2 + h) * 64 + lane) * 2 + m])
                if (word >> pos) & 1:
                    W[r, i, 2 + e // 8] |= 1 << (e % 8)
    return W


@pytest.mark.parametrize("rows,K", [(1, 128), (65, 384), (130, 1152)])
def test_round_trip_and_zero_padding(rows, K):
    W = wl.q1_weights_aos(rows, K, seed=rows + K)
    bits, scales = q1_planes(W, rows, K)
    assert np.array_equal(_decode_planes(bits, scales, rows, K), W)
    nb = K // 128
    nb8 = (nb + 7) // 8 * 8
    r64 = (rows + 63) // 64 * 64
    b4 = bits.reshape(r64 // 64, nb, 2, 64, 2).transpose(0, 1, 3, 2, 4).reshape(r64 // 64, nb, 64, 4)
    s8 = scales.reshape(r64 // 64, nb8 // 8, 64, 8)
    pad_rows = [r for r in range(rows, r64)]
    for r in pad_rows:
        t, lane = divmod(r, 64)
        assert not b4[t, :, lane].any() and not s8[t, :, lane].any()
    if nb8 > nb:
        s_flat = s8.transpose(0, 2, 1, 3).reshape(r64 // 64, 64, nb8)
        assert not s_flat[:, :, nb:].any()
