"""Pins for the sign-bit GEMM oracle (CPU only).

Definition (page "BonsaiのWebGPUカーネルを読み解く", figure on PrismML's
kernels: q1_bits holds 32 weights' sign bits per u32, q1_scales one scale per
32 weights, bit 1 -> +1.0 and 0 -> -1.0):
    y[m, n] = sum_g scale[n, g] * sum_j x[m, 32g + j] * sign(n, 32g + j).
The oracle accumulates in f64 (page "web-xpu-ops", "The reference is the
point") and rounds once. Pinned against numpy's f64 matmul on the
dequantized weights, closed forms and an integer-exact case.
"""
import math

import numpy as np
import pytest

import workloads as wl


def dequant(bits, scales):
    N, G = bits.shape
    b = np.unpackbits(np.ascontiguousarray(bits).view(np.uint8), bitorder="little").reshape(N, G * 32)
    sign = 2.0 * b.astype(np.float64) - 1.0
    return sign * np.repeat(scales.astype(np.float64), 32, axis=1)


@pytest.mark.parametrize("M,N,K,seed", [(7, 33, 128, 1), (16, 64, 512, 2), (3, 5, 4096, 3)])
def test_matches_numpy_f64_matmul(orc, M, N, K, seed):
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed)
    y = orc.sign_gemm_f64(x, bits, scales, nthreads=4).astype(np.float64)
    ref = x.astype(np.float64) @ dequant(bits, scales).T
    # both are f64 sums of the same exact-in-f64 terms, then one f32 rounding
    assert np.all(np.abs(y - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-12 * np.abs(ref).max())


def test_all_bits_one_scale_one_gives_row_sums(orc):
    M, N, K = 5, 3, 1024
    x, _, _ = wl.sign_gemm_inputs(M, N, K, 9)
    bits = np.full((N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    scales = np.ones((N, K // 32), dtype=np.float32)
    y = orc.sign_gemm_f64(x, bits, scales)
    for m in range(M):
        s = np.float32(math.fsum(x[m].astype(np.float64)))
        for n in range(N):
            assert abs(float(y[m, n]) - float(s)) <= np.spacing(np.abs(s))
    bits0 = np.zeros_like(bits)
    y0 = orc.sign_gemm_f64(x, bits0, scales)
    assert np.array_equal(y0, -y)


def test_single_weight_sign_convention(orc):
    """x = unit vector at k: y = +scale where the bit is 1, -scale where 0,
    with bit j of word g <-> weight 32g + j."""
    K, N = 96, 4
    bits = np.zeros((N, 3), dtype=np.uint32)
    bits[1, 2] = 1 << 5          # row 1, weight 69 = +1
    scales = np.arange(1, N * 3 + 1, dtype=np.float32).reshape(N, 3) / 8
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 69] = 1.0
    y = orc.sign_gemm_f64(x, bits, scales)[0]
    assert y[1] == scales[1, 2]
    for n in (0, 2, 3):
        assert y[n] == -scales[n, 2]


def test_integer_exact_case(orc):
    """Integer x (|x| <= 8) and power-of-two scales: every partial sum is exact,
    so the result equals numpy's exact f64 value rounded once to f32."""
    M, N, K = 9, 17, 2048
    rng = np.random.default_rng(5)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = (2.0 ** rng.integers(-6, -1, size=(N, K // 32))).astype(np.float32)
    y = orc.sign_gemm_f64(x, bits, scales)
    ref = (x.astype(np.float64) @ dequant(bits, scales).T).astype(np.float32)
    assert np.array_equal(y, ref)
    y32 = orc.sign_gemm_f32(x, bits, scales)
    assert np.array_equal(y32, ref)


def test_f32_group_order_within_1e6(orc):
    """The f32 group-order evaluation stays within 1e-6 of ||y||_inf of the f64
    oracle at the prefill shape's K: the 1e-5 tolerance has margin."""
    M, N, K = 8, 64, 4096
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, 2)
    y64 = orc.sign_gemm_f64(x, bits, scales, nthreads=8)
    y32 = orc.sign_gemm_f32(x, bits, scales, nthreads=8)
    assert np.max(np.abs(y32 - y64)) / np.max(np.abs(y64)) < 1e-6
