"""GPU parity for split-K decode attention, through the C ABI.

Bar: max|out_gpu - out_oracle| / ||out_oracle||_inf <= 1e-5 + 2^-22 max|s|
against the f64 definition (softmax(scale q k^T) v per query head, grouped KV
heads). The second term is the f32 arithmetic's own: a score of magnitude
|s| is computed to about ulp(|s|), and softmax turns that absolute error into
the same relative error of the weights; at the usual scale (|s| of a few
units) it adds under 1e-6. Cases cover
GQA groups 1/2/4/8, lengths that leave ragged tiles and empty splits, split
counts from 1 to more than the tiles, a cache stride past kv_len, and large
scores.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = 1e-5
D = 128


@pytest.fixture(scope="module")
def gd():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible HIP device")
    import gemm_decode_amd
    return gemm_decode_amd


def inputs(Hq, Hkv, L, stride, seed, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((Hq, D)) * qscale).astype(np.float32)
    k = rng.standard_normal((Hkv, stride, D)).astype(np.float32)
    v = rng.standard_normal((Hkv, stride, D)).astype(np.float32)
    return q, k, v


def run(gd, q, k, v, Hq, Hkv, L, stride, scale, splits=0):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    out = torch.full((Hq * D,), float("nan"), device="cuda")
    gd.attn_decode_splitk(dev(q), dev(k), dev(v), out, Hq, Hkv, D, L, stride, scale, splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(Hq, D)


def rel_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want)) / np.max(np.abs(want)))


def tol(q, k, scale, Hkv):
    """1e-5 + 2^-22 * the largest |score| (f64)."""
    G = q.shape[0] // Hkv
    smax = max(float(np.max(np.abs(scale * (k[h // G].astype(np.float64) @ q[h].astype(np.float64)))))
               for h in range(q.shape[0]))
    return TOL + smax * 2.0 ** -22


@pytest.mark.parametrize("Hq,Hkv,L,splits", [
    (4, 1, 1, 0),          # one key
    (8, 2, 37, 0),         # one ragged tile
    (32, 8, 4096, 0),      # the 8B-class decode shape, 64 splits
    (32, 8, 4113, 0),      # a ragged last tile
    (16, 16, 1000, 0),     # no grouping
    (16, 8, 777, 5),       # groups of 2, five splits
    (64, 8, 2049, 0),      # groups of 8
    (32, 8, 300, 64),      # more splits than keys allow: trailing splits empty
    (32, 8, 5000, 1),      # one split over every tile
    (32, 8, 32768, 0),     # the long-context decode shape the benchmark times
])
def test_parity(gd, Hq, Hkv, L, splits):
    q, k, v = inputs(Hq, Hkv, L, L, seed=Hq + L + splits)
    scale = 1.0 / np.sqrt(D)
    got = run(gd, q, k, v, Hq, Hkv, L, L, scale, splits)
    want = oracle.attention_decode(q, k[:, :L], v[:, :L], scale)
    assert rel_err(got, want) <= tol(q, k[:, :L], scale, Hkv)


def test_stride_past_length(gd):
    """Rows past kv_len (within kv_stride) are never read: fill them with NaN."""
    Hq, Hkv, L, stride = 32, 8, 1500, 2048
    q, k, v = inputs(Hq, Hkv, L, stride, seed=7)
    k[:, L:] = np.nan
    v[:, L:] = np.nan
    scale = 1.0 / np.sqrt(D)
    got = run(gd, q, k, v, Hq, Hkv, L, stride, scale)
    assert np.all(np.isfinite(got))
    assert rel_err(got, oracle.attention_decode(q, k[:, :L], v[:, :L], scale)) <= tol(q, k[:, :L], scale, Hkv)


def test_large_scores(gd):
    """Scores in the thousands: the running maximum keeps every exp finite,
    and the split holding the dominant keys sets the result."""
    Hq, Hkv, L = 8, 2, 3000
    q, k, v = inputs(Hq, Hkv, L, L, seed=9, qscale=30.0)
    got = run(gd, q, k, v, Hq, Hkv, L, L, 1.0)
    want = oracle.attention_decode(q, k, v, 1.0)
    assert np.all(np.isfinite(got))
    assert rel_err(got, want) <= tol(q, k, 1.0, Hkv)


def test_split_counts_agree(gd):
    """The same inputs at 1, 7, 64 and the default split counts."""
    Hq, Hkv, L = 32, 8, 3333
    q, k, v = inputs(Hq, Hkv, L, L, seed=11)
    want = oracle.attention_decode(q, k, v, 0.1)
    for s in (1, 7, 64, 0):
        assert rel_err(run(gd, q, k, v, Hq, Hkv, L, L, 0.1, s), want) <= tol(q, k, 0.1, Hkv), s


def test_workspace_reuse_across_shapes(gd):
    """One workspace serves calls of different shapes and split counts in
    turn, each meeting the bar (nothing in it carries over between calls)."""
    cases = [(32, 8, 4096, 0), (16, 2, 777, 5), (8, 8, 130, 3), (16, 16, 1000, 0), (64, 8, 2049, 0),
             (32, 8, 4096, 0)]
    need = max(gd.attn_decode_workspace_bytes(Hq, Hkv, D, L, s) for Hq, Hkv, L, s in cases)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for n, (Hq, Hkv, L, s) in enumerate(cases):
        q, k, v = inputs(Hq, Hkv, L, L, seed=100 + n)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        out = torch.full((Hq * D,), float("nan"), device="cuda")
        gd.attn_decode_splitk(dev(q), dev(k), dev(v), out, Hq, Hkv, D, L, L, 0.1, s, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(Hq, D)
        assert rel_err(got, oracle.attention_decode(q, k, v, 0.1)) <= tol(q, k, 0.1, Hkv), (Hq, Hkv, L, s)
