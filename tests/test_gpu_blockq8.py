"""GPU parity for block-scaled int8 matmul_nt, through the C ABI.

Bar: max|y_gpu - y_oracle| / ||y_oracle||_inf <= 1e-5, the oracle being the
page "block_q8_matmul_nt.wgsl" order in f32; plus an integer-exact case that
must match bit for bit (every f32 step exact in any order).
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def gd():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible HIP device")
    import gemm_decode_amd
    return gemm_decode_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run(gd, x, quants, scales):
    m, k = x.shape
    n = quants.shape[0]
    y = torch.full((m * n,), float("nan"), device="cuda")
    gd.blockq8_matmul_nt(dev(x), dev(quants.view(np.int32)), dev(scales), y, m, k, n)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(m, n)


def rel_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want)) / np.max(np.abs(want)))


@pytest.mark.parametrize("m", [1, 16])
def test_lm_head_shape_full(gd, m):
    """k=960, n=49152 (the output-projection shape) at full size, launched as
    the benchmark launches it: every one of the m x 49152 outputs against the
    oracle."""
    cfg = wl.BLOCKQ8_LMHEAD
    k, n = cfg["k"], cfg["n"]
    x, quants, scales = wl.blockq8_inputs(m, k, n, cfg["seed"])
    y = run(gd, x, quants, scales)
    assert np.all(np.isfinite(y))
    assert rel_err(y, oracle.blockq8_f32(x, quants, scales, nthreads=oracle.max_threads())) <= TOL


def offset_inputs(m, k, n, x_kind, q_kind, seed):
    """Activations with a large common part and small quants: the case where
    a sum of x*q is far smaller than the sum of |x|, so any rewriting of
    x*q that carries a multiple of sum(x) through f32 loses the result.
    x_kind: "c10" / "c100" (c + N(0,1)) or "absn" (|N(0,1)|); q_kind:
    "pm1" (uniform on {-1,0,1}) or "pm8" (uniform on [-8,8])."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(size=(m, k))
    x = {"c10": 10.0 + z, "c100": 100.0 + z, "absn": np.abs(z)}[x_kind].astype(np.float32)
    lim = {"pm1": 1, "pm8": 8}[q_kind]
    q = rng.integers(-lim, lim + 1, size=(n, k)).astype(np.int8)
    quants = np.ascontiguousarray(q).view("<u4").reshape(n, k // 4)
    scales = rng.uniform(1e-3, 1e-2, size=(n, k // 32)).astype(np.float32)
    return x, quants, scales


@pytest.mark.parametrize("q_kind", ["pm1", "pm8"])
@pytest.mark.parametrize("x_kind", ["c10", "c100", "absn"])
@pytest.mark.parametrize("m", [1, 16])
def test_offset_activations_small_quants(gd, m, x_kind, q_kind):
    """The 1e-5 bar holds for any finite x, not only for zero-mean x against
    full-range quants ("block_q8_matmul_nt.wgsl", PACKING: a quant is its
    sign-extended byte; ACCUMULATION ORDER: a block's 32 products summed,
    then scaled once)."""
    k, n = 960, 4096
    x, quants, scales = offset_inputs(m, k, n, x_kind, q_kind, seed=100 * m + 10 * ["c10", "c100", "absn"].index(x_kind) + len(q_kind) + (q_kind == "pm8"))
    y = run(gd, x, quants, scales)
    err = rel_err(y, oracle.blockq8_f32(x, quants, scales, nthreads=oracle.max_threads()))
    assert err <= TOL, f"m={m} x={x_kind} q={q_kind}: {err:.3e} of ||y||_inf"


@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (3, 64, 130), (5, 992, 77), (16, 960, 300), (2, 2048, 257)])
def test_small_shapes_full(gd, m, k, n):
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed=m * 1000 + k + n)
    y = run(gd, x, quants, scales)
    assert rel_err(y, oracle.blockq8_f32(x, quants, scales)) <= TOL


def test_integer_exact_bitwise(gd):
    m, k, n = 4, 960, 512
    rng = np.random.default_rng(11)
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float32)
    q = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
    quants = q.view("<u4").reshape(n, k // 4)
    scales = (2.0 ** rng.integers(-8, -3, size=(n, k // 32))).astype(np.float32)
    y = run(gd, x, quants, scales)
    assert np.array_equal(y, oracle.blockq8_f32(x, quants, scales))


def test_sign_extension(gd):
    """Quant bytes 0xFF and 0x80 read as -1 and -128."""
    k, n = 32, 2
    q = np.zeros((n, k), dtype=np.uint8)
    q[0, 3] = 0xFF
    q[1, 17] = 0x80
    quants = q.view("<u4").reshape(n, k // 4)
    x = np.ones((1, k), dtype=np.float32)
    y = run(gd, x, quants, np.ones((n, 1), dtype=np.float32))
    assert y.tolist() == [[-1.0, -128.0]]


@pytest.mark.parametrize("m", [2, 3, 7, 8, 9, 15, 16])
@pytest.mark.parametrize("k", [32, 256, 288, 512, 544, 1024])
def test_small_m_tiles(gd, m, k):
    """2 <= m <= 16 with k <= 1024 (the matrix-core path): every block-count
    bucket edge, m across partial row groups, n ragged over 16-feature
    tiles and twelve-tile workgroups."""
    n = 16 * 13 + 5
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed=7 * m + k)
    y = run(gd, x, quants, scales)
    assert rel_err(y, oracle.blockq8_f32(x, quants, scales)) <= TOL


@pytest.mark.parametrize("m,k", [(1, 2048), (2, 1056), (4, 4096)])
def test_long_rows(gd, m, k):
    """k above 1024 (the staged-activation VALU path)."""
    n = 150
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed=m + k)
    y = run(gd, x, quants, scales)
    assert rel_err(y, oracle.blockq8_f32(x, quants, scales)) <= TOL


def test_row_magnitudes(gd):
    """Activation rows 40 decades apart and an all-zero row: each output row
    meets the bar against its own largest value, and the zero row is 0."""
    m, k, n = 7, 512, 200
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed=5)
    mags = np.array([1e-20, 1e-4, 1.0, 1e4, 7e4, 1e20, 0.0], dtype=np.float64)
    x = (x * mags[:, None]).astype(np.float32)
    y = run(gd, x, quants, scales)
    want = oracle.blockq8_f32(x, quants, scales)
    for r in range(m):
        if mags[r] == 0.0:
            assert np.all(y[r] == 0.0)
        else:
            assert rel_err(y[r:r + 1], want[r:r + 1]) <= TOL, r
