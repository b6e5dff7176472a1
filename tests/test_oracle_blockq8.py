"""Pins for the block-Q8 matmul_nt oracle (CPU only).

The oracle follows the page "block_q8_matmul_nt.wgsl": quants packed four per
u32, element t in byte t%4 of word t/4, sign-extended (PACKING, quant_at);
per output, acc = 0, then per 32-block block_sum = sum x*quant in order and
acc = acc + scale*block_sum (ACCUMULATION ORDER, main), in f32 with each
product and add rounded separately. Pinned against numpy's f64 matmul
within the rounding bound, closed forms and an integer-exact case.
"""
import math

import numpy as np
import pytest

import workloads as wl


def dequant(quants, scales):
    n = quants.shape[0]
    q = np.ascontiguousarray(quants).view(np.int8).reshape(n, -1).astype(np.float64)
    return q * np.repeat(scales.astype(np.float64), 32, axis=1)


def gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


@pytest.mark.parametrize("m,k,n,seed", [(1, 960, 257, 1), (16, 960, 64, 2), (3, 64, 5, 3)])
def test_within_bound_of_numpy_f64(orc, m, k, n, seed):
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed)
    y = orc.blockq8_f32(x, quants, scales, nthreads=4).astype(np.float64)
    D = dequant(quants, scales)
    ref = x.astype(np.float64) @ D.T
    absum = np.abs(x.astype(np.float64)) @ np.abs(D).T
    # a term's path: 1 product, <= 31 adds, 1 scale product, <= k/32 adds
    assert np.all(np.abs(y - ref) <= gamma(33 + k // 32) * absum)


def test_sign_extension_and_byte_order(orc):
    """0xFF reads as -1, not +255; element t lives in byte t%4 of word t/4."""
    k, n = 32, 1
    for t in range(32):
        q = np.zeros(k, dtype=np.uint8)
        q[t] = 0xFF
        quants = q.view("<u4").reshape(n, k // 4)
        word = int(quants[0, t // 4])
        assert (word >> (8 * (t % 4))) & 0xFF == 0xFF
        x = np.zeros((1, k), dtype=np.float32)
        x[0, t] = 3.0
        y = orc.blockq8_f32(x, quants, np.ones((1, 1), dtype=np.float32))
        assert y[0, 0] == -3.0


def test_quants_one_scales_one_gives_row_sums(orc):
    m, k, n = 4, 960, 3
    x, _, _ = wl.blockq8_inputs(m, k, n, 7)
    quants = np.full((n, k // 4), 0x01010101, dtype=np.uint32)
    scales = np.ones((n, k // 32), dtype=np.float32)
    y = orc.blockq8_f32(x, quants, scales)
    for r in range(m):
        s = math.fsum(x[r].astype(np.float64))
        bound = gamma(k) * np.abs(x[r]).astype(np.float64).sum()
        assert np.all(np.abs(y[r].astype(np.float64) - s) <= bound)


def test_integer_exact_case(orc):
    """|x| <= 4 integers and power-of-two scales: every f32 step exact."""
    m, k, n = 5, 960, 40
    rng = np.random.default_rng(11)
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
    q = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
    quants = q.view("<u4").reshape(n, k // 4)
    scales = (2.0 ** rng.integers(-8, -3, size=(n, k // 32))).astype(np.float32)
    y = orc.blockq8_f32(x, quants, scales)
    ref = x.astype(np.float64) @ dequant(quants, scales).T
    assert np.array_equal(y.astype(np.float64), ref)
