"""GPU parity for the packed sign-bit paths, via the C ABI: the one-time
pack, the matrix-core GEMM on packed weights, the decode GEMV and the LUT4
prefill GEMM (table lookup of signed 4-element sums).

Bar: the packed layout byte for byte against the header's definition; the
packed GEMM bit for bit against q1_sign_gemm; the lookup paths within
max|y_gpu - y_oracle| / ||y_oracle||_inf <= 1e-5 of the f64 oracle, and bit
for bit on integer-valued inputs (every table entry and partial sum exact),
which pins the nibble -> table-entry map.
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


def rel_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want)) / np.max(np.abs(want)))


def pack(gd, bits, scales):
    N, G = bits.shape
    K = 32 * G
    wp = torch.full((gd.q1_sign_packed_bytes(N, K),), 0xCD, dtype=torch.uint8, device="cuda")
    gd.q1_sign_pack(dev(bits.view(np.int32)), dev(scales), N, K, wp)
    return wp


def packed_ref(bits, scales):
    """The packed layout written from the header's definition: the table
    kernels' section, the matrix-core section (only its first 8*N*G bytes
    are defined) and the per-output exponents, as uint32 arrays."""
    N, G = bits.shape
    G2 = (G + 1) // 2
    out = np.zeros((G2, N, 4), dtype=np.uint32)
    sb = scales.view(np.uint32)
    for p in range(G2):
        out[p, :, 0] = bits[:, 2 * p]
        out[p, :, 2] = sb[:, 2 * p]
        if 2 * p + 1 < G:
            out[p, :, 1] = bits[:, 2 * p + 1]
            out[p, :, 3] = sb[:, 2 * p + 1]
    smax = np.max(np.abs(scales), axis=1)
    c = np.where(smax > 0, 15 - np.frexp(smax)[1], 0).astype(np.int32)
    v = np.ldexp(scales, c[:, None]).astype(np.float32)            # exact: a power-of-two scaling
    sh = v.astype(np.float16)
    sl = (v - sh.astype(np.float32)).astype(np.float16)           # v - sh is exact in f32
    hl = sh.view(np.uint16).astype(np.uint32) | (sl.view(np.uint16).astype(np.uint32) << 16)
    mc = np.zeros((G, N, 2), dtype=np.uint32)
    mc[:, :, 0] = bits.T
    mc[:, :, 1] = hl.T
    return out.reshape(-1), mc.reshape(-1), c.view(np.uint32)


def check_packed(wp, bits, scales):
    N, G = bits.shape
    words = wp.cpu().numpy().view(np.uint32)
    tab, mc, cexp = packed_ref(bits, scales)
    sec = tab.size                                   # 4 words per output and group pair
    assert words.size == 2 * sec + N
    assert np.array_equal(words[:sec], tab), "table kernels' section"
    assert np.array_equal(words[sec:sec + mc.size], mc), "matrix-core section"
    assert np.array_equal(words[2 * sec:], cexp), "output exponents"


def run(gd, fn, x, wp, N):
    M, K = x.shape
    y = torch.full((M * N,), float("nan"), device="cuda")
    getattr(gd, fn)(dev(x), wp, y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(M, N)


@pytest.mark.parametrize("N,K", [(1, 32), (65, 96), (130, 2048), (64, 4096 + 32), (17, 16384), (20, 16384 + 32)])
def test_pack_layout(gd, N, K):
    _, bits, scales = wl.sign_gemm_inputs(1, N, K, seed=N + K)
    wp = pack(gd, bits, scales)
    torch.cuda.synchronize()
    check_packed(wp, bits, scales)


def test_pack_layout_extreme_scales(gd):
    """Outputs whose scales span many decades, an all-zero output, negative
    and subnormal scales: the matrix-core section's exponents and fp16
    pairs follow the definition exactly."""
    N, K = 6, 256
    _, bits, scales = wl.sign_gemm_inputs(1, N, K, seed=77)
    scales = scales.astype(np.float64)
    scales[0] *= 1e-30
    scales[1] *= 1e30
    scales[2] = 0.0
    scales[3] *= -1.0
    scales[4, ::2] = 1e-41                    # f32 subnormals beside normal values
    scales[5] = np.geomspace(1e-20, 1e3, K // 32)
    scales = scales.astype(np.float32)
    wp = pack(gd, bits, scales)
    torch.cuda.synchronize()
    check_packed(wp, bits, scales)


@pytest.mark.parametrize("M,N,K", [(17, 33, 96), (130, 129, 512), (512, 4096, 4096)])
def test_packed_gemm_matches_unpacked(gd, M, N, K):
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=3 * M + N)
    wp = pack(gd, bits, scales)
    y1 = torch.empty(M * N, device="cuda")
    y2 = torch.full((M * N,), float("nan"), device="cuda")
    xd = dev(x)
    gd.q1_sign_gemm(xd, dev(bits.view(np.int32)), dev(scales), y1, M, N, K)
    gd.q1_sign_gemm_packed(xd, wp, y2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))


GEMV_SHAPES = [(1, 1, 32), (1, 63, 96), (1, 4096, 4096), (1, 14336, 4096), (1, 4096, 14336), (3, 130, 8224),
               (2, 200, 4096 + 64), (1, 8192, 2080), (2, 8193, 2080)]


@pytest.mark.parametrize("M,N,K", GEMV_SHAPES)
def test_gemv_parity(gd, M, N, K):
    """Decode shapes (4096x4096, 14336x4096, and 4096x14336 over several
    table chunks), an odd group count, K past a chunk by one pair, and N on
    both sides of the switch from 16 to 64 outputs per workgroup."""
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=M * 7 + N + K)
    y = run(gd, "q1_sign_gemv", x, pack(gd, bits, scales), N)
    assert rel_err(y, oracle.sign_gemm_f64(x, bits, scales, nthreads=oracle.max_threads())) <= TOL


@pytest.mark.parametrize("fn", ["q1_sign_gemv", "q1_sign_gemm_lut4"])
@pytest.mark.parametrize("M,N,K", [(1, 70, 4096 + 96), (20, 530, 1056)])
def test_integer_exact(gd, fn, M, N, K):
    """Small integer activations and power-of-two scales make every table
    entry, partial sum and fma exact: the result must equal the oracle's bit
    for bit, whatever the order, so a wrong nibble or entry shows."""
    rng = np.random.default_rng(M + N)
    x = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = (2.0 ** rng.integers(-6, -1, size=(N, K // 32))).astype(np.float32)
    y = run(gd, fn, x, pack(gd, bits, scales), N)
    assert np.array_equal(y, oracle.sign_gemm_f64(x, bits, scales))


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (17, 33, 96), (130, 600, 512), (16, 512, 4096), (33, 1000, 2080)])
def test_lut4_parity(gd, M, N, K):
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=M + 5 * N + K)
    y = run(gd, "q1_sign_gemm_lut4", x, pack(gd, bits, scales), N)
    assert rel_err(y, oracle.sign_gemm_f64(x, bits, scales, nthreads=oracle.max_threads())) <= TOL


def test_lut4_prefill_shape_sampled(gd):
    """M=512 tokens, N=4096, K=4096 at full size, 96 output columns checked."""
    cfg = wl.SIGN_PREFILL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, cfg["seed"])
    y = run(gd, "q1_sign_gemm_lut4", x, pack(gd, bits, scales), N)
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 64, replace=False)]))
    want = oracle.sign_gemm_f64(x, bits[cols], scales[cols], nthreads=oracle.max_threads())
    assert rel_err(y[:, cols], want) <= TOL


@pytest.mark.parametrize("fn", ["q1_sign_gemv", "q1_sign_gemm_lut4"])
def test_row_magnitudes(gd, fn):
    """Activation rows 40 decades apart and an all-zero row: each output row
    meets the bar against its own largest value; the zero row is 0."""
    M, N, K = 7, 300, 512
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed=5)
    mags = np.array([1e-20, 1e-4, 1.0, 1e4, 7e4, 1e20, 0.0])
    x = (x * mags[:, None]).astype(np.float32)
    y = run(gd, fn, x, pack(gd, bits, scales), N)
    want = oracle.sign_gemm_f64(x, bits, scales)
    for r in range(M):
        if mags[r] == 0.0:
            assert np.all(y[r] == 0.0)
        else:
            assert rel_err(y[r:r + 1], want[r:r + 1]) <= TOL, r
