"""Pins for the Q1_0 . q8_0 oracle (CPU only).

The oracle (oracle.c, F1 and F2) follows the arithmetic that the page
"browseml-gpu.js" states in its header comment: integer s per 4 elements,
ab = d1*s then sequential rounded adds over the four 32-element sub-blocks,
acc = fma(d0, ab, acc) per block, and the fixed tree
((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7)). These tests tie it to things other
than itself: numpy's f16 conversion, exact integer sums, exact f64 sums when
every f32 step is exact, an f64 brute force within the first-order rounding
bound, closed-form cases crafted so that a different rounding order, an
unfused acc step or a different tree pairing gives a different answer, and
invariants.
"""
import math

import numpy as np
import pytest

import workloads as wl


# --------------------------------------------------------------- helpers

def f16_bits(v: float) -> int:
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def build_aos(d0_bits, signs, d1_bits, q):
    """AoS bytes from explicit fields.

    d0_bits: [rows, nb] u16; signs: [rows, K] 0/1; d1_bits: [K/32] u16;
    q: [K] int8. Layout per the page: weight block = d0 LE + bits (element j at
    byte 2 + j//8, bit j%8); activation block = d1 LE + 32 int8."""
    d0_bits = np.asarray(d0_bits, dtype=np.uint16)
    rows, nb = d0_bits.shape
    K = nb * 128
    signs = np.asarray(signs, dtype=np.uint8).reshape(rows, nb, 128)
    W = np.zeros((rows, nb, 18), dtype=np.uint8)
    W[:, :, 0] = d0_bits & 0xFF
    W[:, :, 1] = d0_bits >> 8
    W[:, :, 2:] = np.packbits(signs, axis=-1, bitorder="little")
    d1_bits = np.asarray(d1_bits, dtype=np.uint16)
    A = np.zeros((K // 32, 34), dtype=np.uint8)
    A[:, 0] = d1_bits & 0xFF
    A[:, 1] = d1_bits >> 8
    A[:, 2:] = np.asarray(q, dtype=np.int8).reshape(K // 32, 32).view(np.uint8)
    return W, A


def decode_fields(W, A, rows, K):
    """Inverse of build_aos using numpy's own f16 conversion."""
    nb = K // 128
    W = np.asarray(W, dtype=np.uint8).reshape(rows, nb, 18)
    d0 = W[:, :, 0:2].copy().view(np.float16).reshape(rows, nb).astype(np.float64)
    signs = np.unpackbits(W[:, :, 2:], axis=-1, bitorder="little").reshape(rows, K)
    A = np.asarray(A, dtype=np.uint8).reshape(-1, K // 32, 34)
    d1 = A[:, :, 0:2].copy().view(np.float16).reshape(A.shape[0], K // 32).astype(np.float64)
    q = A[:, :, 2:].copy().view(np.int8).reshape(A.shape[0], K).astype(np.int64)
    return d0, signs, d1, q


def wrapped_terms(signs, q):
    """c_e = q if bit 1 else the int8-wrapping negation of q (-(-128) = -128)."""
    neg = np.where(q == -128, -128, -q)
    return np.where(signs == 1, q, neg)


def f64_brute(W, A, rows, K):
    """Per row: math.fsum of the exact f64 terms d0*d1*c_e, and sum |terms|."""
    d0, signs, d1, q = decode_fields(W, A, rows, K)
    c = wrapped_terms(signs, q[0])
    d0e = np.repeat(d0, 128, axis=1)
    d1e = np.repeat(d1[0], 32)
    terms = d0e * d1e[None, :] * c  # each exact: 11 + 11 + 8 significant bits
    y = np.array([math.fsum(t) for t in terms])
    return y, np.abs(terms).sum(axis=1)


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)


# --------------------------------------------------------------- pins

def test_f16_decode_matches_numpy_all_patterns(orc):
    """f16 -> f32 decode equals numpy's conversion for all 65536 patterns
    (NaNs compared as a class)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(v)) for v in h], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("K", [128, 256, 1024])
def test_integer_exact_unit_scales(orc, K):
    """d0 = d1 = 1.0: every f32 op is exact (|partial| < 2^24), so the oracle
    equals the exact integer sum of the wrapped terms, -128 quants included."""
    rows = 32
    rng = np.random.default_rng(K)
    signs = rng.integers(0, 2, size=(rows, K))
    q = rng.integers(-128, 128, size=K)
    q[rng.random(K) < 0.05] = -128
    W, A = build_aos(np.full((rows, K // 128), 0x3C00), signs, np.full(K // 32, 0x3C00), q)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0]
    exact = wrapped_terms(signs, q[None, :]).sum(axis=1)
    assert np.array_equal(y.astype(np.int64), exact)
    assert np.array_equal(y, exact.astype(np.float32))


@pytest.mark.parametrize("K", [128, 512, 1024])
def test_power_of_two_scales_exact(orc, K):
    """d in {2^-3, 2^-2, 2^-1}, |q| <= 15: every partial sum is a multiple of
    2^-6 below 2^15, so every f32 step is exact and the oracle must equal the
    exact f64 dequantize-then-dot."""
    rows = 24
    rng = np.random.default_rng(7 + K)
    pw = np.array([f16_bits(0.125), f16_bits(0.25), f16_bits(0.5)])
    d0b = rng.choice(pw, size=(rows, K // 128))
    d1b = rng.choice(pw, size=K // 32)
    signs = rng.integers(0, 2, size=(rows, K))
    q = rng.integers(-15, 16, size=K)
    W, A = build_aos(d0b, signs, d1b, q)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0]
    ref, _ = f64_brute(W, A, rows, K)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("K,seed", [(128, 1), (256, 2), (1024, 3), (2048, 4)])
def test_brute_force_within_rounding_bound(orc, K, seed):
    """Random f16 scales (the page's randomCase, -128 at 2%): the oracle is
    within gamma(nb + 6) * sum|terms| of the f64 sum of exact terms (3 rounded
    adds in ab, nb fused acc steps, 3 tree adds on any term's path)."""
    rows = 16
    W, A = wl.random_case(rows, K, seed)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0].astype(np.float64)
    ref, absum = f64_brute(W, A, rows, K)
    bound = gamma(K // 128 + 6) * absum + 2.0 ** -149
    assert np.all(np.abs(y - ref) <= bound)


def test_brute_force_config_distribution(orc):
    """Same bound on the decode configs' distributions (|N(0,0.02)| d0,
    U(0.001,0.05) d1, quants in [-127,127])."""
    rows, K = 64, 4096
    W = wl.q1_weights_aos(rows, K, seed=11)
    A = wl.q8_acts_aos(K, seed=12)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0].astype(np.float64)
    ref, absum = f64_brute(W, A, rows, K)
    assert np.all(np.abs(y - ref) <= gamma(K // 128 + 6) * absum)


# ---- closed forms that fix the rounding order -----------------------------

def _crafted(d0_list, subblocks):
    """Build a one-row case. d0_list: d0 per block (floats exact in f16).
    subblocks: per block, list of 4 (d1, {l: s}) pairs; s in [-127, 127] is
    placed as element 4l of the sub-block (q = |s|, bit = 1 if s >= 0 else 0),
    every other quant 0."""
    nb = len(d0_list)
    K = nb * 128
    signs = np.ones((1, K), dtype=np.int64)
    q = np.zeros(K, dtype=np.int64)
    d1b = np.zeros(K // 32, dtype=np.int64)
    for i, blk in enumerate(subblocks):
        for k, (d1, sv) in enumerate(blk):
            d1b[4 * i + k] = f16_bits(d1)
            for l, s in sv.items():
                e = 128 * i + 32 * k + 4 * l
                q[e] = abs(s)
                signs[0, e] = 1 if s >= 0 else 0
    d0b = np.array([[f16_bits(v) for v in d0_list]])
    return build_aos(d0b, signs, d1b, q), K


def test_order_ab_adds_are_sequential_in_k(orc):
    """ab = ((p0 + p1) + p2) + p3. With d0 = 2^10, p0 = 2^14, p1 = p2 = 2^-10:
    2^14 + 2^-10 is a tie (ulp(2^14) = 2^-9) and rounds to even, twice, so
    ab = 2^14 and y = 2^24. Pairing p1 with p2 first would give 2^24 + 2."""
    (W, A), K = _crafted([2.0 ** 10], [[(2.0 ** 14, {0: 1}), (2.0 ** -10, {0: 1}),
                                        (2.0 ** -10, {0: 1}), (1.0, {})]])
    y = orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0]
    assert y == np.float32(2.0 ** 24)


def test_order_acc_step_is_fused(orc):
    """Block 0 leaves acc = -1; block 1 has d0 = 1 + 2^-10 and
    ab = 1 + 2^-20, so d0*ab = 1 + 2^-10 + 2^-20 + 2^-30. A fused step gives
    exactly 2^-10 + 2^-20 + 2^-30; multiply-then-add would lose the 2^-30."""
    sub = 2.0 ** -20  # an f16 subnormal (16 * 2^-24)
    (W, A), K = _crafted(
        [1.0, 1.0 + 2.0 ** -10],
        [[(1.0, {0: -1}), (1.0, {}), (1.0, {}), (1.0, {})],
         [(1.0, {0: 1}), (sub, {0: 1}), (1.0, {}), (1.0, {})]])
    y = orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0]
    assert float(y) == 2.0 ** -10 + 2.0 ** -20 + 2.0 ** -30


def test_order_tree_pairs_lane2_with_lane6(orc):
    """acc0 = 2^24, acc2 = acc6 = 1, other lanes 0. The tree adds
    (acc2 + acc6) = 2 before meeting 2^24, giving 2^24 + 2 exactly; a
    left-to-right sum or ((a0+a1)+(a2+a3)) pairing gives 2^24."""
    (W, A), K = _crafted([2.0 ** 10], [[(2.0 ** 14, {0: 1}), (2.0 ** -10, {2: 1, 6: 1}),
                                        (1.0, {}), (1.0, {})]])
    y = orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0]
    assert float(y) == 2.0 ** 24 + 2


def test_order_tree_pairs_lane1_with_lane5(orc):
    """acc0 = 2^24, acc1 = acc5 = 1: the right subtree (a1+a5) = 2 gives
    2^24 + 2; pairing a1 with a0 or a5 with a4 first gives 2^24."""
    (W, A), K = _crafted([2.0 ** 10], [[(2.0 ** 14, {0: 1}), (2.0 ** -10, {1: 1, 5: 1}),
                                        (1.0, {}), (1.0, {})]])
    y = orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0]
    assert float(y) == 2.0 ** 24 + 2


def test_element_to_lane_mapping(orc):
    """Lane l of sub-block k covers elements 32k + 4l .. 32k + 4l + 3: with
    acc0 = 2^24, a unit placed at element 4*2 (lane 2) and another at element
    4*6 + 3 (lane 6) is 2^24 + 2, but placed at elements of lanes 0 and 4 the
    two units are absorbed (2^24)."""
    def case(e_a, e_b):
        K = 128
        signs = np.ones((1, K), dtype=np.int64)
        q = np.zeros(K, dtype=np.int64)
        q[0] = 1  # lane 0, sub-block 0 carries 2^14 (via d1_0)
        q[32 + e_a] = 1
        q[32 + e_b] = 1
        d1b = np.array([f16_bits(2.0 ** 14), f16_bits(2.0 ** -10), 0x3C00, 0x3C00])
        W, A = build_aos(np.array([[f16_bits(2.0 ** 10)]]), signs, d1b, q)
        return float(orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0])
    assert case(8, 27) == 2.0 ** 24 + 2     # lanes 2 and 6
    assert case(1, 17) == 2.0 ** 24         # lanes 0 and 4: a0+a4 absorbs


def test_wrap_of_minus_128(orc):
    """A -128 quant under a 0 bit contributes -128 (int8 wrapping negation),
    not +128: one element, d0 = d1 = 1."""
    K = 128
    signs = np.ones((1, K), dtype=np.int64)
    q = np.zeros(K, dtype=np.int64)
    q[5] = -128
    signs[0, 5] = 0
    W, A = build_aos(np.array([[0x3C00]]), signs, np.full(4, 0x3C00), q)
    assert orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0] == -128.0
    signs[0, 5] = 1
    W, A = build_aos(np.array([[0x3C00]]), signs, np.full(4, 0x3C00), q)
    assert orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0] == -128.0
    q[5] = 127
    signs[0, 5] = 0
    W, A = build_aos(np.array([[0x3C00]]), signs, np.full(4, 0x3C00), q)
    assert orc.q1_q8_gemv_aos(W, A, 1, K)[0, 0] == -127.0


# ---- invariants -----------------------------------------------------------

def test_flip_all_bits_negates(orc):
    """Without -128 quants, flipping every sign bit gives exactly -y (every
    rounding is sign-symmetric)."""
    rows, K = 32, 1024
    W = wl.q1_weights_aos(rows, K, seed=5)
    A = wl.q8_acts_aos(K, seed=6)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0]
    Wf = W.copy()
    Wf[:, :, 2:] ^= 0xFF
    yf = orc.q1_q8_gemv_aos(Wf, A, rows, K)[0]
    assert np.array_equal(yf, -y)


def test_scale_d0_by_two_doubles(orc):
    """Doubling every d0 (exactly, in f16) doubles y exactly."""
    rows, K = 32, 1024
    W = wl.q1_weights_aos(rows, K, seed=8)
    A = wl.q8_acts_aos(K, seed=9)
    y = orc.q1_q8_gemv_aos(W, A, rows, K)[0]
    W2 = W.copy()
    d0 = W2[:, :, 0:2].copy().view(np.float16)
    W2[:, :, 0:2] = (d0 * np.float16(2)).view(np.uint8)
    y2 = orc.q1_q8_gemv_aos(W2, A, rows, K)[0]
    assert np.array_equal(y2, 2 * y)


def test_columns_equal_single_column(orc):
    """n_act > 1: column c equals the batch-1 result on activation c."""
    rows, K, n = 40, 512, 5
    W = wl.q1_weights_aos(rows, K, seed=3)
    A = wl.q8_acts_aos(K, seed=4, n_act=n)
    Y = orc.q1_q8_gemv_aos(W, A, rows, K, n_act=n, nthreads=4)
    for c in range(n):
        yc = orc.q1_q8_gemv_aos(W, A[c], rows, K)[0]
        assert np.array_equal(Y[c].view(np.uint32), yc.view(np.uint32))


@pytest.mark.parametrize("rows,K,seed", [(256, 2048, 1), (37, 384, 9), (1, 128, 3)])
def test_F1_equals_F2_bitwise(orc, rows, K, seed):
    """F1 (AoS walk, 8 chains per row) and F2 (P1's packed layouts, one chain
    per (row, lane)) agree bit for bit, -128 quants included (randomCase)."""
    W, A = wl.random_case(rows, K, seed)
    As = [A] + [wl.random_case(1, K, seed * 100 + k)[1] for k in range(1, 5)]
    Acat = np.concatenate(As)
    y1 = orc.q1_q8_gemv_aos(W, Acat, rows, K, n_act=5, nthreads=8)
    y2 = orc.q1_q8_gemv_p1packed(W, Acat, rows, K, n_act=5, nthreads=8)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_thread_count_does_not_change_bits(orc):
    rows, K = 96, 1024
    W = wl.q1_weights_aos(rows, K, seed=21)
    A = wl.q8_acts_aos(K, seed=22, n_act=2)
    y1 = orc.q1_q8_gemv_aos(W, A, rows, K, 2, nthreads=1)
    y8 = orc.q1_q8_gemv_aos(W, A, rows, K, 2, nthreads=8)
    assert np.array_equal(y1.view(np.uint32), y8.view(np.uint32))
