"""GPU parity at the launch-size limits of the entry points whose second grid
dimension is a count the caller chooses: q1_q8_gemv's n_act, and the
problem counts of q1_q8_gemv_grouped and ternary_gemv_grouped (each at most
65535). Every output is checked bit for bit against the oracle, and the
guard elements past each problem's rows must stay untouched.

The launches re-use a few weights and activations across their many
problems (each problem still has its own output), so the oracle runs once
per distinct pair.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LIMIT = 65535


@pytest.fixture(scope="module")
def gd():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible HIP device")
    import gemm_decode_amd
    return gemm_decode_amd


class _Ptr:
    """A device address for the problem-array builders (which read data_ptr())."""

    def __init__(self, p):
        self.p = int(p)

    def data_ptr(self):
        return self.p


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_q1_grouped_at_the_problem_limit(gd, K):
    """65535 problems in one grouped launch (the one-group, two-unit and
    multi-unit kernels by K), rows 1..64 per problem and some rows = 0 (the
    launch's 64): each output bit-exact, nothing written past its rows."""
    rows_max, n_w, n_a = 64, 4, 8
    Ws = [wl.q1_weights_aos(rows_max, K, 300 + w + K) for w in range(n_w)]
    As = [wl.q8_acts_aos(K, 700 + a + K) for a in range(n_a)]
    planes = []
    for W in Ws:
        b, s = gd.q1_alloc_planes(rows_max, K)
        gd.q1_repack(dev(W.reshape(-1)), rows_max, K, b, s)
        planes.append((b, s))
    a_dev = [dev(A.reshape(-1)) for A in As]
    want = {(w, a): oracle.q1_q8_gemv_aos(Ws[w], As[a], rows_max, K).reshape(-1)
            for w in range(n_w) for a in range(n_a)}
    y = torch.full((LIMIT * rows_max,), float("nan"), device="cuda")
    y0 = y.data_ptr()
    entries, expect = [], np.full((LIMIT, rows_max), np.nan, dtype=np.float32)
    for i in range(LIMIT):
        w, a = i % n_w, (i // n_w) % n_a
        rows = 1 + (i * 37) % rows_max
        field = 0 if i % 97 == 0 else rows
        eff = rows_max if field == 0 else rows
        b, s = planes[w]
        entries.append((b, s, a_dev[a], _Ptr(y0 + 4 * i * rows_max), field))
        expect[i, :eff] = want[(w, a)][:eff]
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, LIMIT, rows_max, K)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(LIMIT, rows_max)
    bad = np.nonzero((_bits(got) != _bits(expect)).any(axis=1))[0]
    assert bad.size == 0, f"K {K}: {bad.size} problems differ, first {bad[:5].tolist()}"


def test_q1_columns_at_the_limit(gd):
    """q1_q8_gemv with n_act = 65535 columns (one grid row each on the
    four-chain kernel): every column bit-exact with its own batch-1 GEMV."""
    rows, K = 5, 128
    W = wl.q1_weights_aos(rows, K, 17)
    few = np.stack([wl.q8_acts_aos(K, 900 + c).reshape(-1) for c in range(16)])
    A = np.concatenate([few] * ((LIMIT + 15) // 16))[:LIMIT]
    b, s = gd.q1_alloc_planes(rows, K)
    gd.q1_repack(dev(W.reshape(-1)), rows, K, b, s)
    y = torch.full((LIMIT * rows + 64,), float("nan"), device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y[:LIMIT * rows], rows, K, LIMIT)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = oracle.q1_q8_gemv_aos(W, A.reshape(-1), rows, K, n_act=LIMIT, nthreads=oracle.max_threads()).reshape(-1)
    assert np.array_equal(_bits(got[:LIMIT * rows]), _bits(want))
    assert np.all(np.isnan(got[LIMIT * rows:])), "wrote past the last column"


def test_ternary_grouped_at_the_problem_limit(gd):
    """65535 ternary problems in one grouped launch: every output and dot
    product equal to the oracle's, nothing written past the rows."""
    rows, K, n_w, n_a = 64, 256, 4, 8
    W = K // 32
    ins = [wl.ternary_inputs(rows, K, 500 + w) for w in range(n_w)]
    xq = [wl.ternary_inputs(8, K, 600 + a)[3] for a in range(n_a)]
    xs = [0.01 * (a + 1) for a in range(n_a)]
    wdev = [(dev(P.view(np.int32)), dev(N.view(np.int32))) for P, N, _, _, _ in ins]
    xp = torch.empty(n_a * 8 * W, dtype=torch.int32, device="cuda")
    gd.ternary_act_bitplanes(dev(np.stack(xq)), n_a, K, xp)
    want = {(w, a): oracle.ternary_gemv(ins[w][0], ins[w][1], ins[w][2], xq[a], xs[a])
            for w in range(n_w) for a in range(n_a)}
    y = torch.full((LIMIT * rows + 64,), float("nan"), device="cuda")
    d = torch.full((LIMIT * rows + 64,), -7, dtype=torch.int32, device="cuda")
    y0, d0, x0 = y.data_ptr(), d.data_ptr(), xp.data_ptr()
    entries = []
    ey = np.empty((LIMIT, rows), dtype=np.float32)
    ed = np.empty((LIMIT, rows), dtype=np.int32)
    for i in range(LIMIT):
        w, a = i % n_w, (i // n_w) % n_a
        entries.append((wdev[w][0], wdev[w][1], _Ptr(x0 + 4 * a * 8 * W), _Ptr(y0 + 4 * i * rows),
                        _Ptr(d0 + 4 * i * rows), ins[w][2], xs[a]))
        ey[i], ed[i] = want[(w, a)]
    probs = gd.make_ternary_problems(entries)
    gd.ternary_gemv_grouped(probs, LIMIT, rows, K)
    torch.cuda.synchronize()
    gy, gdot = y.cpu().numpy(), d.cpu().numpy()
    assert np.array_equal(gdot[:LIMIT * rows].reshape(LIMIT, rows), ed)
    assert np.array_equal(_bits(gy[:LIMIT * rows]).reshape(LIMIT, rows), _bits(ey))
    assert np.all(np.isnan(gy[LIMIT * rows:])) and np.all(gdot[LIMIT * rows:] == -7), "wrote past the last problem"
