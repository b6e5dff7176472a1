"""GPU parity for the sign-bit prefill GEMM (matrix-core path), via the C ABI.

Bar: max|y_gpu - y_oracle| / ||y_oracle||_inf <= 1e-5 against the f64 oracle
of the plain definition; an integer-valued case must match bit for bit (hi/lo
split exact, every f32 accumulation exact), which pins the MFMA tiling.
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


def run(gd, x, bits, scales):
    M, K = x.shape
    N = bits.shape[0]
    y = torch.full((M * N,), float("nan"), device="cuda")
    gd.q1_sign_gemm(dev(x), dev(bits.view(np.int32)), dev(scales), y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(M, N)


def rel_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want)) / np.max(np.abs(want)))


def test_integer_exact_pins_tiling(gd):
    M, N, K = 144, 160, 256
    rng = np.random.default_rng(5)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = (2.0 ** rng.integers(-6, -1, size=(N, K // 32))).astype(np.float32)
    y = run(gd, x, bits, scales)
    assert np.array_equal(y, oracle.sign_gemm_f64(x, bits, scales))


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 16, 32), (17, 33, 96), (130, 129, 512), (64, 256, 4096),
                                   (33, 70, 8224)])
def test_ragged_shapes(gd, M, N, K):
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=M + N + K)
    y = run(gd, x, bits, scales)
    assert rel_err(y, oracle.sign_gemm_f64(x, bits, scales, nthreads=8)) <= TOL


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_shape_full(gd, packed):
    """M=512 tokens, N=4096, K=4096 at full size, as the benchmark calls it
    (the caller's sign words and scales, or weights packed once by
    q1_sign_pack): all 512 x 4096 outputs against the f64 oracle."""
    cfg = wl.SIGN_PREFILL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, cfg["seed"])
    if packed:
        wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        gd.q1_sign_pack(dev(bits.view(np.int32)), dev(scales), N, K, wp)
        yt = torch.full((M * N,), float("nan"), device="cuda")
        gd.q1_sign_gemm_packed(dev(x), wp, yt, M, N, K)
        torch.cuda.synchronize()
        y = yt.cpu().numpy().reshape(M, N)
    else:
        y = run(gd, x, bits, scales)
    assert np.all(np.isfinite(y))
    want = oracle.sign_gemm_f64(x, bits, scales, nthreads=oracle.max_threads())
    assert rel_err(y, want) <= TOL


def test_all_ones_row_sums(gd):
    M, N, K = 32, 48, 1024
    x, _, _ = wl.sign_gemm_inputs(M, N, K, 1)
    bits = np.full((N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    y = run(gd, x, bits, np.ones((N, K // 32), dtype=np.float32))
    want = x.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(y - want[:, None])) <= 1e-5 * np.max(np.abs(want))


def test_row_magnitudes(gd):
    """Token rows 40 decades apart and an all-zero row: each output row meets
    the bar against its own largest value, and the zero row is 0."""
    M, N, K = 7, 150, 512
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=9)
    mags = np.array([1e-20, 1e-4, 1.0, 1e4, 7e4, 1e20, 0.0])
    x = (x.astype(np.float64) * mags[:, None]).astype(np.float32)
    y = run(gd, x, bits, scales)
    want = oracle.sign_gemm_f64(x, bits, scales)
    for r in range(M):
        if mags[r] == 0.0:
            assert np.all(y[r] == 0.0)
        else:
            assert rel_err(y[r:r + 1], want[r:r + 1]) <= TOL, r


@pytest.mark.parametrize("packed", [False, True])
def test_output_scale_magnitudes(gd, packed):
    """Outputs whose scales sit 40 decades apart, an all-zero output, and an
    output whose own scales span 23 decades: each output column meets the
    bar against its own largest value and the zero output is 0 (each output
    has its own power-of-two normalisation)."""
    M, N, K = 40, 8, 1024
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=11)
    mags = np.array([1e-20, 1e-4, 1.0, 1e4, 1e20, 0.0, 1.0, 1.0])
    sc = scales.astype(np.float64) * mags[:, None]
    sc[6] = np.geomspace(1e-20, 1e3, K // 32)
    sc[7, ::3] *= -1.0
    sc = sc.astype(np.float32)
    want = oracle.sign_gemm_f64(x, bits, sc)
    if packed:
        wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        gd.q1_sign_pack(dev(bits.view(np.int32)), dev(sc), N, K, wp)
        yt = torch.full((M * N,), float("nan"), device="cuda")
        gd.q1_sign_gemm_packed(dev(x), wp, yt, M, N, K)
        torch.cuda.synchronize()
        y = yt.cpu().numpy().reshape(M, N)
    else:
        y = run(gd, x, bits, sc)
    for n in range(N):
        if mags[n] == 0.0:
            assert np.all(y[:, n] == 0.0)
        else:
            assert rel_err(y[:, n:n + 1], want[:, n:n + 1]) <= TOL, n


def test_explicit_workspace_and_reuse(gd):
    """A caller-owned workspace of exactly the reported size gives the same
    bits as the cached one, and reusing it for a second, smaller call on the
    same stream leaves no trace of the first."""
    M, N, K = 100, 200, 640
    need = gd.q1_sign_gemm_workspace_bytes(M, N, K)
    assert need == 112 * K * 4 + 112 * 32 + N * (K // 64) * 16 + N * 4
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=3)
    y1 = torch.empty(M * N, device="cuda")
    gd.q1_sign_gemm(dev(x), dev(bits.view(np.int32)), dev(scales), y1, M, N, K, workspace=ws)
    y0 = run(gd, x, bits, scales)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().reshape(M, N), y0)
    x2, bits2, scales2 = wl.sign_gemm_inputs(20, 40, 96, seed=4)
    y2 = torch.empty(20 * 40, device="cuda")
    gd.q1_sign_gemm(dev(x2), dev(bits2.view(np.int32)), dev(scales2), y2, 20, 40, 96, workspace=ws)
    torch.cuda.synchronize()
    assert rel_err(y2.cpu().numpy().reshape(20, 40), oracle.sign_gemm_f64(x2, bits2, scales2)) <= TOL
    with pytest.raises(gd.GemmDecodeError):
        gd.q1_sign_gemm(dev(x), dev(bits.view(np.int32)), dev(scales), y1, M, N, K, workspace=ws[:need - 16])
