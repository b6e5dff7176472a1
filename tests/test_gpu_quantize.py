"""GPU parity for on-device activation quantization, through the C ABI.

Bar: bit-exact. Codes, f16 block scales, f32 token scales and bit-plane
words must equal the oracle's (page "web-xpu-ops" quantize rule: reciprocal
127/absmax in f64, Math.round ties toward +infinity, clamp to [-127, 127]),
and the quantize-then-GEMV pipelines must give the oracle's GEMV of the
oracle's quantization bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gd():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible HIP device")
    import gemm_decode_amd
    return gemm_decode_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def planes_of(q):
    """Two's-complement bit planes [count][8][K/32] of int8 codes [count][K],
    from the header's definition (bit j of word m of plane b = bit b of
    element 32m + j)."""
    count, K = q.shape
    u = q.view(np.uint8).astype(np.uint32).reshape(count, K // 32, 32)
    w = np.arange(32, dtype=np.uint32)
    out = np.zeros((count, 8, K // 32), dtype=np.uint32)
    for b in range(8):
        out[:, b] = (((u >> b) & 1) << w).sum(axis=2).astype(np.uint32)
    return out


def acts(n, K, seed):
    """N(0,1) rows at magnitudes 1e-3 .. 1e3, with a zero block, exact ties
    and a row reaching its absmax at a negative value."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(n, K)) * (10.0 ** rng.uniform(-3, 3, size=(n, 1)))
    x = x.astype(np.float32)
    if K >= 64:
        x[0, 32:64] = 0.0                                      # a zero block
        x[0, 64 % K:64 % K + 32] = np.arange(-16, 16) + 0.5    # ties once scaled by 127/absmax = 127/15.5
    if n > 1:
        x[1, K // 2] = -4.0 * np.max(np.abs(x[1]))
    return x


def run_q8(gd, x):
    n, K = x.shape
    out = torch.full((n * (K // 32) * 34,), 0xEE, dtype=torch.uint8, device="cuda")
    gd.q8_0_quantize(dev(x), out, n, K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_act(gd, x):
    count, K = x.shape
    planes = torch.full((count * 8 * (K // 32),), -1, dtype=torch.int32, device="cuda")
    scale = torch.full((count,), float("nan"), device="cuda")
    gd.ternary_quantize_act(dev(x), count, K, planes, scale)
    torch.cuda.synchronize()
    return planes, scale


@pytest.mark.parametrize("n,K", [(1, 32), (1, 4096), (3, 96), (32, 4096), (2, 14336), (5, 1152)])
def test_q8_0_bit_exact(gd, n, K):
    x = acts(n, K, seed=n * 100 + K)
    got = run_q8(gd, x)
    want = oracle.quantize_q8_0(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_q8_0_scale_extremes(gd):
    """Block scales that round to f16 subnormals, to zero and to infinity,
    and blocks whose values tie under the reciprocal."""
    K = 32 * 6
    x = np.zeros((1, K), dtype=np.float32)
    rng = np.random.default_rng(3)
    for i, mag in enumerate([1e-6, 1e-9, 1e-12, 1e7, 1.0, 127.0]):
        x[0, 32 * i:32 * i + 32] = rng.uniform(-1, 1, size=32) * mag
    x[0, 32 * 5:32 * 6] = np.arange(-16, 16) * 7.0 + 0.5    # absmax 127 below: every value a tie
    x[0, 32 * 5 + 31] = 127.0
    got = run_q8(gd, x)
    assert np.array_equal(got, oracle.quantize_q8_0(x))


@pytest.mark.parametrize("K", [256, 4096])
def test_q8_0_codes_at_ties_and_tiny_blocks(gd, K):
    """Blocks whose scaled values sit exactly on half-integers and one f32
    ulp either side (the f32 decision must hand them to the f64 rule, ties
    toward +infinity), and blocks whose absmax is subnormal or near 1e-37
    (127/absmax beyond f32, every code in f64): bit for bit with the
    oracle."""
    rng = np.random.default_rng(K + 7)
    base = rng.integers(-126, 126, size=(3, K)).astype(np.float64) + 0.5
    x = base.astype(np.float32)
    x[1] = np.nextafter(x[1], np.float32(np.inf))     # just above the ties
    x[2] = np.nextafter(x[2], np.float32(-np.inf))    # just below
    x[0, ::32], x[1, ::32], x[2, ::32] = 127.0, 127.0, -127.0   # each block's absmax 127: reciprocal 1
    mags = np.array([1e-40, 3e-39, 1e-37, 3.6e-37, 1e-36, 1.0], dtype=np.float64)
    tiny = rng.uniform(-1, 1, size=(1, K)) * np.repeat(np.resize(mags, K // 32), 32)[None, :]
    tiny = tiny.astype(np.float32)
    for blk in range(K // 32):
        m = np.float32(mags[blk % len(mags)])
        tiny[0, 32 * blk] = m                          # the block's absmax
        tiny[0, 32 * blk + 1] = m / np.float32(2)      # half of it: code 64, not a clamped 127
    x = np.concatenate([x, tiny])
    got = run_q8(gd, x)
    want = oracle.quantize_q8_0(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


@pytest.mark.parametrize("count,K", [(1, 32), (1, 96), (1, 2560), (1, 6912), (4, 2560), (3, 160), (2, 2048),
                                     (2, 8192), (1, 8224), (2, 14336)])
def test_token_planes_and_scales(gd, count, K):
    x = acts(count, K, seed=count * 7 + K)
    planes, scale = run_act(gd, x)
    q, s = oracle.quantize_absmax_int8(x)
    assert np.array_equal(planes.cpu().numpy().view(np.uint32).reshape(count, 8, K // 32), planes_of(q))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("K", [256, 2560, 8192])
def test_token_codes_at_ties(gd, K):
    """Tokens whose scaled values sit exactly on half-integers, and one f32
    ulp either side of them: the f32 decision must hand these to the exact
    f64 rule (ties toward +infinity), bit for bit with the oracle."""
    rng = np.random.default_rng(K)
    base = rng.integers(-126, 126, size=(3, K)).astype(np.float64) + 0.5
    x = base.astype(np.float32)
    x[0, 0] = 127.0                                        # absmax 127: the reciprocal is exactly 1
    x[1] = np.nextafter(x[1], np.float32(np.inf))          # just above the ties
    x[1, 0] = 127.0
    x[2] = np.nextafter(x[2], np.float32(-np.inf))         # just below
    x[2, 0] = -127.0
    planes, scale = run_act(gd, x)
    q, s = oracle.quantize_absmax_int8(x)
    assert np.array_equal(planes.cpu().numpy().view(np.uint32).reshape(3, 8, K // 32), planes_of(q))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.array_equal(q[0, 1:], np.floor(base[0, 1:] + 0.5).astype(np.int8))   # ties went up


@pytest.mark.parametrize("K", [256, 2560, 8192, 8224])
def test_token_tiny_absmax(gd, K):
    """Tokens whose absmax lies in the f32 subnormal range or near 1e-37,
    where 127/absmax no longer fits in f32: codes and scales still follow the
    f64 rule bit for bit (x = absmax/2 must give 64, not a clamped 127)."""
    rng = np.random.default_rng(K + 1)
    mags = [1e-40, 3e-39, 1e-37, 3.6e-37, 1e-36]
    x = np.stack([rng.uniform(-1, 1, size=K) * m for m in mags]).astype(np.float32)
    for r in range(len(mags)):
        x[r, 0] = np.float32(mags[r])                  # the token's absmax
        x[r, 1] = np.float32(mags[r]) / np.float32(2)  # half of it
    planes, scale = run_act(gd, x)
    q, s = oracle.quantize_absmax_int8(x)
    assert np.array_equal(planes.cpu().numpy().view(np.uint32).reshape(len(mags), 8, K // 32), planes_of(q))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert all(q[r, 1] == 64 for r in range(len(mags)))


def test_zero_input(gd):
    x = np.zeros((2, 128), dtype=np.float32)
    assert not run_q8(gd, x).any()
    planes, scale = run_act(gd, x)
    assert not planes.cpu().numpy().any() and not scale.cpu().numpy().any()


@pytest.mark.parametrize("rows,K", [(2560, 2560), (6912, 2560), (2560, 6912)])
def test_ternary_pipeline_device_scale(gd, rows, K):
    """f32 activations -> ternary_quantize_act -> ternary_gemv_grouped with
    the scale read from device memory: y and the int32 dot bit-exact with
    the oracle's GEMV of the oracle's quantization (three tokens, one
    problem each)."""
    count = 3
    P, N, ws, _, _ = wl.ternary_inputs(rows, K, seed=rows + K)
    x = acts(count, K, seed=rows * 3 + K)
    planes, scale = run_act(gd, x)
    W = K // 32
    Pd, Nd = dev(P.view(np.int32)), dev(N.view(np.int32))
    ys = [torch.full((rows,), float("nan"), device="cuda") for _ in range(count)]
    ds = [torch.full((rows,), -7, dtype=torch.int32, device="cuda") for _ in range(count)]
    probs = gd.make_ternary_problems([(Pd, Nd, planes[c * 8 * W:(c + 1) * 8 * W], ys[c], ds[c], ws,
                                       scale[c:c + 1]) for c in range(count)])
    gd.ternary_gemv_grouped(probs, count, rows, K)
    torch.cuda.synchronize()
    q, s = oracle.quantize_absmax_int8(x)
    for c in range(count):
        want_y, want_d = oracle.ternary_gemv(P, N, ws, q[c], s[c], nthreads=oracle.max_threads())
        assert np.array_equal(ds[c].cpu().numpy(), want_d), c
        assert np.array_equal(ys[c].cpu().numpy().view(np.uint32), want_y.view(np.uint32)), c


@pytest.mark.parametrize("rows,K,n_act", [(256, 1024, 1), (4096, 4096, 1), (1000, 4224, 3), (14336, 4096, 4)])
def test_q1_pipeline(gd, rows, K, n_act):
    """f32 activations -> q8_0_quantize -> q1_q8_gemv: bit-exact with the
    oracle's GEMV of the oracle's q8_0 blocks."""
    W = wl.q1_weights_aos(rows, K, seed=rows + 5)
    x = acts(n_act, K, seed=rows + K + n_act)
    b, s = gd.q1_alloc_planes(rows, K)
    gd.q1_repack(dev(W.reshape(-1)), rows, K, b, s)
    a = torch.empty(n_act * (K // 32) * 34, dtype=torch.uint8, device="cuda")
    gd.q8_0_quantize(dev(x), a, n_act, K)
    y = torch.full((n_act * rows,), float("nan"), device="cuda")
    gd.q1_q8_gemv(b, s, a, y, rows, K, n_act)
    torch.cuda.synchronize()
    A = oracle.quantize_q8_0(x)
    assert np.array_equal(a.cpu().numpy(), A)
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n_act, nthreads=oracle.max_threads())
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.reshape(-1).view(np.uint32))
