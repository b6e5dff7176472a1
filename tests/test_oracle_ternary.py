"""Pins for the ternary bitplane oracle (CPU only).

The page "BonsaiのWebGPUカーネルを読み解く" (section on Bonsai) states the
identity dot = 2(pc(P&X) - pc(N&X)) - pc(P) + pc(N) for P (w=+1) and N (w=-1)
bitplanes against a binary plane X. The oracle (T2) applies it to the eight
offset-binary planes of int8 x; T1 is the direct int64 sum. Pinned: T1 == T2,
both equal numpy's int64 matmul, closed forms.
"""
import numpy as np
import pytest

import workloads as wl


def unpack_w(P, N):
    rows, W = P.shape
    p = np.unpackbits(np.ascontiguousarray(P).view(np.uint8), bitorder="little").reshape(rows, W * 32)
    n = np.unpackbits(np.ascontiguousarray(N).view(np.uint8), bitorder="little").reshape(rows, W * 32)
    return p.astype(np.int64) - n.astype(np.int64)


@pytest.mark.parametrize("rows,K,seed", [(64, 2560, 1), (17, 6912, 2), (5, 32, 3)])
def test_identity_equals_direct_and_numpy(orc, rows, K, seed):
    P, N, ws, xq, xs = wl.ternary_inputs(rows, K, seed)
    assert not np.any(P & N)
    t1 = orc.ternary_dot_direct(P, N, xq)
    y, t2 = orc.ternary_gemv(P, N, ws, xq, xs, nthreads=4)
    ref = unpack_w(P, N) @ xq.astype(np.int64)
    assert np.array_equal(t1, ref)
    assert np.array_equal(t2.astype(np.int64), ref)
    s = np.float32(np.float32(ws) * np.float32(xs))
    assert np.array_equal(y, ref.astype(np.float32) * s)


def test_minus_128_and_extremes(orc):
    rng = np.random.default_rng(4)
    rows, K = 9, 256
    w = rng.integers(-1, 2, size=(rows, K))
    P = wl.pack_bits_lsb((w == 1).astype(np.uint8))
    N = wl.pack_bits_lsb((w == -1).astype(np.uint8))
    x = rng.integers(-128, 128, size=K).astype(np.int8)
    x[::7] = -128
    x[::11] = 127
    _, t2 = orc.ternary_gemv(P, N, 1.0, x, 1.0)
    assert np.array_equal(t2.astype(np.int64), w @ x.astype(np.int64))


def test_closed_forms(orc):
    rows, K = 6, 320
    P, N, _, _, _ = wl.ternary_inputs(rows, K, 5)
    pcP = np.array([sum(bin(int(v)).count("1") for v in r) for r in P])
    pcN = np.array([sum(bin(int(v)).count("1") for v in r) for r in N])
    minus1 = np.full(K, -1, dtype=np.int8)
    _, d = orc.ternary_gemv(P, N, 1.0, minus1, 1.0)
    assert np.array_equal(d, -(pcP - pcN))          # all x = -1
    x = np.random.default_rng(6).integers(-127, 128, size=K).astype(np.int8)
    ones = np.full((rows, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    zeros = np.zeros_like(ones)
    _, d = orc.ternary_gemv(ones, zeros, 1.0, x, 1.0)
    assert np.all(d == int(x.astype(np.int64).sum()))  # all w = +1
    _, d = orc.ternary_gemv(zeros, zeros, 1.0, x, 1.0)
    assert not d.any()                                # P = N = 0
    _, d = orc.ternary_gemv(P, N, 1.0, np.zeros(K, dtype=np.int8), 1.0)
    assert not d.any()                                # x = 0
