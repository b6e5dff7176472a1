"""Pins for the oracle's decode attention (softmax(scale q k^T) v per query
head, grouped KV heads), checked against closed forms and against scipy's
softmax, an independent library routine."""
import numpy as np
import pytest

import oracle

scipy_special = pytest.importorskip("scipy.special")


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((2, 1, 8))
    v = rng.standard_normal((2, 1, 8))
    out = oracle.attention_decode(q, k, v, 0.3)
    assert np.array_equal(out, v[[0, 0, 1, 1], 0])


def test_zero_scale_is_the_mean_of_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 16))
    k = rng.standard_normal((3, 50, 16))
    v = rng.standard_normal((3, 50, 16))
    out = oracle.attention_decode(q, k, v, 0.0)
    assert np.allclose(out, v.mean(axis=1), rtol=0, atol=1e-15)


def test_dominant_key():
    """One key scored 1000 above the rest takes all the weight."""
    D, L = 8, 20
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((1, L, D))
    k[0, 7, 0] = 1000.0
    v = np.arange(L * D, dtype=np.float64).reshape(1, L, D)
    out = oracle.attention_decode(q, k, v, 1.0)
    assert np.array_equal(out[0], v[0, 7])


def test_against_scipy_softmax_and_grouping():
    rng = np.random.default_rng(3)
    Hq, Hkv, L, D = 8, 2, 33, 16
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((Hkv, L, D)) * 3
    v = rng.standard_normal((Hkv, L, D))
    out = oracle.attention_decode(q, k, v, 0.25)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        w = scipy_special.softmax(0.25 * np.einsum("d,ld->l", q[h], k[kv]))
        assert np.allclose(out[h], w @ v[kv], rtol=1e-13, atol=1e-14)


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 8))
    k = rng.standard_normal((1, 40, 8))
    v = rng.standard_normal((1, 40, 8))
    out = oracle.attention_decode(q, k, v, 0.5)
    perm = rng.permutation(40)
    assert np.allclose(oracle.attention_decode(q, k[:, perm], v[:, perm], 0.5), out, rtol=0, atol=1e-14)
    # scores shifted by a constant (a key component along a zero query dim does
    # nothing; a common offset along q does): q . (k + c q/|q|^2) = q.k + c
    c = 37.0
    k2 = k + c * q[0] / (q[0] @ q[0])
    out2 = oracle.attention_decode(q[:1], k2, v, 0.5)
    assert np.allclose(out2, out[:1], rtol=0, atol=1e-12)


def test_large_scores_are_stable():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 8)) * 100
    k = rng.standard_normal((1, 64, 8)) * 100
    v = rng.standard_normal((1, 64, 8))
    out = oracle.attention_decode(q, k, v, 1.0)
    assert np.all(np.isfinite(out))
    assert np.all(np.abs(out) <= np.abs(v).max(axis=1) + 1e-12)   # a convex combination of values
