"""Checks of the seeded input generators: formats, bit order, ranges,
distribution moments and reproducibility (no method arithmetic here)."""
import numpy as np

import workloads as wl


def test_q1_aos_format_and_distribution():
    W = wl.q1_weights_aos(512, 1024, seed=0)
    assert W.shape == (512, 8, 18) and W.dtype == np.uint8
    d0 = W[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all(d0 >= 0)
    assert abs(np.sqrt(np.mean(d0 ** 2)) - 0.02) < 0.001   # |N(0, 0.02)|
    bits = np.unpackbits(W[:, :, 2:], axis=-1)
    assert abs(bits.mean() - 0.5) < 0.01
    assert np.array_equal(W, wl.q1_weights_aos(512, 1024, seed=0))
    assert not np.array_equal(W, wl.q1_weights_aos(512, 1024, seed=1))


def test_q8_aos_format_and_distribution():
    A = wl.q8_acts_aos(4096, seed=1000, n_act=3)
    assert A.shape == (3, 128, 34)
    d1 = A[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    assert d1.min() >= 0.00099 and d1.max() <= 0.0501
    q = A[:, :, 2:].copy().view(np.int8)
    assert q.min() >= -127 and q.max() <= 127


def test_mulberry32_uniform_and_random_case_format():
    r = wl.Mulberry32(1)
    v = np.array([r() for _ in range(20000)])
    assert v.min() >= 0 and v.max() < 1 and abs(v.mean() - 0.5) < 0.01
    W, A = wl.random_case(8, 2048, 1)
    assert W.size == 8 * 16 * 18 and A.size == 64 * 34
    h = np.concatenate([W.reshape(-1, 18)[:, :2], A.reshape(-1, 34)[:, :2]]).copy().view(np.uint16)
    e = (h >> 10) & 0x1F
    assert e.min() >= 3 and e.max() <= 16
    q = A.reshape(-1, 34)[:, 2:]
    frac128 = np.mean(q == 128)
    assert 0.01 < frac128 < 0.035
    W2, A2 = wl.random_case(8, 2048, 1)
    assert np.array_equal(W, W2) and np.array_equal(A, A2)


def test_packed_bit_order():
    b = np.zeros((1, 64), dtype=np.uint8)
    b[0, 33] = 1
    w = wl.pack_bits_lsb(b)
    assert w.tolist() == [[0, 2]]


def test_blockq8_and_sign_inputs():
    x, quants, scales = wl.blockq8_inputs(2, 960, 8, 3)
    assert quants.shape == (8, 240) and scales.shape == (8, 30) and x.shape == (2, 960)
    q = quants.view(np.int8).reshape(8, 960)
    assert q.min() >= -128 and q.max() <= 127
    x, bits, scales = wl.sign_gemm_inputs(4, 8, 128, 2)
    assert bits.shape == (8, 4) and scales.shape == (8, 4) and np.all(scales >= 0)


def test_ternary_inputs_and_absmax():
    P, N, ws, xq, xs = wl.ternary_inputs(100, 2560, 4000)
    assert P.shape == (100, 80) and not np.any(P & N)
    frac = np.mean(np.unpackbits(P.view(np.uint8)))
    assert abs(frac - 1 / 3) < 0.01
    assert np.max(np.abs(xq.astype(np.int64))) == 127 and xs > 0
    q, s = wl.absmax_int8(np.array([0.5, -1.0, 0.25, 0.003937007874015748]))
    assert q.tolist() == [64, -127, 32, 1]   # 63.5 ties upward to 64; 0.5 -> 1
    assert len(wl.bitnet_step_shapes()) == 210
