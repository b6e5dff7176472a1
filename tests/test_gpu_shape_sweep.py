"""Seeded random-shape sweeps of every entry point against the oracle.

The other GPU test files pin each path at chosen shapes (decode and prefill
sizes, ragged tails, the edges of each dispatch rule). Here every path is
driven over shapes drawn from a fixed-seed generator instead: log-uniform row
and output counts, K anywhere in its legal range (multi-chunk and tail
blocks included), 1 to 12 activation columns, grouped launches of mixed row
counts, and split counts chosen by the caller or by the library. So a shape
that falls between the chosen ones, and a kernel that a dispatch rule picks
only there, is still compared with the oracle. Each case's parameters are
part of its test id, and each bar is the path's own: bit for bit for Q1_0,
ternary and the quantizers; 1e-5 of ||y||_inf for the f32 contractions;
1e-5 + 2^-22 * max|score| for attention.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = 1e-5
D = 128   # attention head dim (the only one the library takes)


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


def log_uniform(rng, lo, hi):
    return int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))


def assert_bits_equal(got, want, what):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32).reshape(-1)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32).reshape(-1)
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, f"{what}: {bad.size} of {g.size} outputs differ, first at {bad[0]}"


def draw(seed, n, fn):
    rng = np.random.default_rng(seed)
    return [fn(rng, i) for i in range(n)]


# ------------------------------------------------------------------ Q1_0

def _q1_case(rng, i):
    while True:
        rows = log_uniform(rng, 1, 6000)
        K = 128 * int(rng.integers(1, 73))
        n_act = 1 if rng.random() < 0.4 else int(rng.integers(2, 13))
        if rows * K * n_act <= 6e7:
            return rows, K, n_act, 7000 + i


Q1_CASES = draw(11, 40, _q1_case)


@pytest.mark.parametrize("rows,K,n_act,seed", Q1_CASES)
def test_q1_gemv_random_shapes(gd, rows, K, n_act, seed):
    if seed % 3 == 0:   # the page's randomCase: broad f16 exponents, -128 quants
        W, A1 = wl.random_case(rows, K, seed)
        A = np.concatenate([A1.reshape(1, -1)] +
                           [wl.q8_acts_aos(K, seed + c).reshape(1, -1) for c in range(1, n_act)])
    else:
        W = wl.q1_weights_aos(rows, K, seed)
        A = wl.q8_acts_aos(K, seed + 1, n_act)
    b, s = gd.q1_alloc_planes(rows, K)
    gd.q1_repack(dev(W.reshape(-1)), rows, K, b, s)
    y = torch.full((n_act * rows,), float("nan"), device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y, rows, K, n_act)
    torch.cuda.synchronize()
    want = oracle.q1_q8_gemv_aos(W, A.reshape(-1), rows, K, n_act=n_act, nthreads=8)
    assert_bits_equal(y.cpu().numpy(), want, f"rows={rows} K={K} n_act={n_act}")


def _q1_group_case(rng, i):
    while True:
        R = log_uniform(rng, 1, 6000) if i % 2 else log_uniform(rng, 300, 6000)
        K = 128 * int(rng.integers(1, 41))
        count = int(rng.integers(1, 41))
        rows = [R if rng.random() < 0.3 else int(rng.integers(1, R + 1)) for _ in range(count)]
        rows[int(rng.integers(0, count))] = R   # the launch's rows: the largest problem's
        shared = bool(rng.random() < 0.5)
        if sum(rows) * K <= 8e7:
            return R, K, tuple(rows), shared, 7100 + i


def _q1_group_case_at(K):
    def f(rng, i):
        while True:
            R = log_uniform(rng, 300, 6000)
            count = int(rng.integers(2, 41))
            rows = [R if rng.random() < 0.3 else int(rng.integers(1, R + 1)) for _ in range(count)]
            rows[int(rng.integers(0, count))] = R
            shared = bool(rng.random() < 0.5)
            if sum(rows) * K <= 8e7:
                return R, K, tuple(rows), shared, 7150 + i + K
    return f


# random problem sets, plus one at each K whose rows run several 256- or
# 128-row units per workgroup (whole groups of eight blocks in one table chunk)
Q1_GROUP_CASES = draw(12, 10, _q1_group_case) + [draw(20 + K // 1024, 1, _q1_group_case_at(K))[0]
                                                  for K in (1024, 2048, 3072, 4096)]


@pytest.mark.parametrize("R,K,rows,shared,seed", Q1_GROUP_CASES,
                         ids=[f"R{c[0]}-K{c[1]}-n{len(c[2])}-{'shared' if c[3] else 'own'}"
                              for c in Q1_GROUP_CASES])
def test_q1_grouped_random_problem_sets(gd, R, K, rows, shared, seed):
    """Problems of mixed row counts in one launch (rows R = the largest),
    each activation either shared by all or the problem's own; guard
    elements after each output must stay untouched."""
    acts = [wl.q8_acts_aos(K, seed + (0 if shared else j)).reshape(-1) for j in range(len(rows))]
    entries, wants = [], []
    for j, r in enumerate(rows):
        W = wl.q1_weights_aos(r, K, seed * 100 + j)
        b, s = gd.q1_alloc_planes(r, K)
        gd.q1_repack(dev(W.reshape(-1)), r, K, b, s)
        a = dev(acts[j])
        y = torch.full((r + 64,), float("nan"), device="cuda")
        entries.append((b, s, a, y, r))
        wants.append(oracle.q1_q8_gemv_aos(W, acts[j], r, K, n_act=1, nthreads=8))
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, len(rows), R, K)
    torch.cuda.synchronize()
    for j, ((_, _, _, y, r), want) in enumerate(zip(entries, wants)):
        got = y.cpu().numpy()
        assert_bits_equal(got[:r], want, f"problem {j} (rows {r}) of R={R} K={K}")
        assert np.all(np.isnan(got[r:])), f"problem {j}: write past its {r} rows"


# ---------------------------------------------------------------- sign-bit

def _sign_case(rng, i):
    while True:
        M = log_uniform(rng, 1, 400)
        N = log_uniform(rng, 1, 1500)
        K = 32 * int(rng.integers(1, 261))
        if M * N * K <= 1.5e8:
            return M, N, K, 7200 + i


SIGN_CASES = draw(13, 16, _sign_case)


@pytest.mark.parametrize("M,N,K,seed", SIGN_CASES)
def test_sign_gemm_random_shapes(gd, M, N, K, seed):
    """The matrix-core GEMM on the caller's words and on packed weights."""
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed)
    want = oracle.sign_gemm_f64(x, bits, scales, nthreads=8)
    xd = dev(x)
    y = torch.full((M * N,), float("nan"), device="cuda")
    gd.q1_sign_gemm(xd, dev(bits.view(np.int32)), dev(scales), y, M, N, K)
    wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gd.q1_sign_pack(dev(bits.view(np.int32)), dev(scales), N, K, wp)
    yp = torch.full((M * N,), float("nan"), device="cuda")
    gd.q1_sign_gemm_packed(xd, wp, yp, M, N, K)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(M, N)
    assert rel_err(got, want) <= TOL, f"M={M} N={N} K={K}: {rel_err(got, want):.3e}"
    assert_bits_equal(yp.cpu().numpy(), got, f"packed vs caller's words, M={M} N={N} K={K}")


def _sign_gemv_case(rng, i):
    while True:
        M = int(rng.integers(1, 5))
        N = log_uniform(rng, 1, 20000)
        K = 32 * int(rng.integers(1, 401))
        if M * N * K <= 1.5e8:
            return M, N, K, 7300 + i


SIGN_GEMV_CASES = draw(14, 16, _sign_gemv_case)


@pytest.mark.parametrize("M,N,K,seed", SIGN_GEMV_CASES)
def test_sign_gemv_random_shapes(gd, M, N, K, seed):
    """The decode GEMV on packed weights (the narrow kernel up to 8192
    outputs, the wide one above), against the f64 definition."""
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed)
    wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gd.q1_sign_pack(dev(bits.view(np.int32)), dev(scales), N, K, wp)
    y = torch.full((M * N,), float("nan"), device="cuda")
    gd.q1_sign_gemv(dev(x), wp, y, M, N, K)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(M, N)
    want = oracle.sign_gemm_f64(x, bits, scales, nthreads=8)
    assert rel_err(got, want) <= TOL, f"M={M} N={N} K={K}: {rel_err(got, want):.3e}"


def _lut4_case(rng, i):
    while True:
        M = log_uniform(rng, 1, 100)
        N = log_uniform(rng, 1, 1200)
        K = 32 * int(rng.integers(1, 131))
        if M * N * K <= 1e8:
            return M, N, K, 7400 + i


LUT4_CASES = draw(15, 8, _lut4_case)


@pytest.mark.parametrize("M,N,K,seed", LUT4_CASES)
def test_sign_lut4_random_shapes(gd, M, N, K, seed):
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, seed)
    wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gd.q1_sign_pack(dev(bits.view(np.int32)), dev(scales), N, K, wp)
    y = torch.full((M * N,), float("nan"), device="cuda")
    gd.q1_sign_gemm_lut4(dev(x), wp, y, M, N, K)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(M, N)
    want = oracle.sign_gemm_f64(x, bits, scales, nthreads=8)
    assert rel_err(got, want) <= TOL, f"M={M} N={N} K={K}: {rel_err(got, want):.3e}"


# ---------------------------------------------------------------- block-Q8

def _bq_case(rng, i):
    m = 1 if rng.random() < 0.3 else int(rng.integers(2, 17))
    k = 32 * int(rng.integers(1, min(16384 // m, 4096) // 32 + 1))
    n = log_uniform(rng, 1, 5000)
    return m, k, n, 7500 + i


BQ_CASES = draw(16, 24, _bq_case)


@pytest.mark.parametrize("m,k,n,seed", BQ_CASES)
def test_blockq8_random_shapes(gd, m, k, n, seed):
    """Every kernel the dispatch can pick (m = 1 GEMV, matrix cores for
    k <= 1024, the staged-x VALU kernel above), against the page's f32 order."""
    x, quants, scales = wl.blockq8_inputs(m, k, n, seed)
    y = torch.full((m * n,), float("nan"), device="cuda")
    gd.blockq8_matmul_nt(dev(x), dev(quants.view(np.int32)), dev(scales), y, m, k, n)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(m, n)
    want = oracle.blockq8_f32(x, quants, scales, nthreads=8)
    assert rel_err(got, want) <= TOL, f"m={m} k={k} n={n}: {rel_err(got, want):.3e}"


# ----------------------------------------------------------------- ternary

def _tern_case(rng, i):
    rows = log_uniform(rng, 1, 5000)
    K = 32 * int(rng.integers(1, 301))
    return rows, K, 7600 + i


TERN_CASES = draw(17, 20, _tern_case)


@pytest.mark.parametrize("rows,K,seed", TERN_CASES)
def test_ternary_random_shapes(gd, rows, K, seed):
    """Planes from the int8 codes, the GEMV (dot and y) bit for bit, and the
    same problem through the grouped entry point with the scale on the device."""
    P, N, ws, xq, xs = wl.ternary_inputs(rows, K, seed)
    W = K // 32
    xp = torch.empty(8 * W, dtype=torch.int32, device="cuda")
    gd.ternary_act_bitplanes(dev(xq), 1, K, xp)
    Pd, Nd = dev(P.view(np.int32)), dev(N.view(np.int32))
    y = torch.full((rows,), float("nan"), device="cuda")
    d = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    gd.ternary_gemv(Pd, Nd, ws, xp, xs, y, d, rows, K)
    xs_dev = torch.tensor([xs], dtype=torch.float32, device="cuda")
    y2 = torch.full((rows,), float("nan"), device="cuda")
    probs = gd.make_ternary_problems([(Pd, Nd, xp, y2, None, ws, xs_dev)])
    gd.ternary_gemv_grouped(probs, 1, rows, K)
    torch.cuda.synchronize()
    yo, do = oracle.ternary_gemv(P, N, ws, xq, xs, nthreads=8)
    assert np.array_equal(d.cpu().numpy(), do), f"rows={rows} K={K}: dot"
    assert_bits_equal(y.cpu().numpy(), yo, f"rows={rows} K={K}: y")
    assert_bits_equal(y2.cpu().numpy(), yo, f"rows={rows} K={K}: grouped y")


# ------------------------------------------------------------ quantizers

def _quant_case(rng, i):
    n = log_uniform(rng, 1, 40)
    K = 32 * int(rng.integers(1, 451))
    return n, K, 7700 + i


QUANT_CASES = draw(18, 16, _quant_case)


def _acts(n, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(n, K)) * (10.0 ** rng.uniform(-4, 4, size=(n, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("n,K,seed", QUANT_CASES)
def test_quantizers_random_shapes(gd, n, K, seed):
    """q8_0 bytes and per-token int8 planes + scales, bit for bit."""
    x = _acts(n, K, seed)
    a = torch.full((n * (K // 32) * 34,), 0xEE, dtype=torch.uint8, device="cuda")
    gd.q8_0_quantize(dev(x), a, n, K)
    planes = torch.full((n * 8 * (K // 32),), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((n,), float("nan"), device="cuda")
    gd.ternary_quantize_act(dev(x), n, K, planes, sc)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), oracle.quantize_q8_0(x)), f"q8_0 n={n} K={K}"
    codes, scales = oracle.quantize_absmax_int8(x)
    u = codes.view(np.uint8).astype(np.uint32).reshape(n, K // 32, 32)
    want = np.zeros((n, 8, K // 32), dtype=np.uint32)
    for b in range(8):
        want[:, b] = (((u >> b) & 1) << np.arange(32, dtype=np.uint32)).sum(axis=2).astype(np.uint32)
    got = planes.cpu().numpy().view(np.uint32).reshape(n, 8, K // 32)
    assert np.array_equal(got, want), f"int8 planes n={n} K={K}"
    assert_bits_equal(sc.cpu().numpy(), scales, f"token scales n={n} K={K}")


# --------------------------------------------------------------- attention

def _attn_case(rng, i):
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    L = log_uniform(rng, 1, 10000)
    stride = L + int(rng.integers(0, 6))
    splits = 0 if rng.random() < 0.5 else int(rng.integers(1, 81))
    return Hkv * G, Hkv, L, stride, splits, 7800 + i


ATTN_CASES = draw(19, 20, _attn_case)


@pytest.mark.parametrize("Hq,Hkv,L,stride,splits,seed", ATTN_CASES)
def test_attention_random_shapes(gd, Hq, Hkv, L, stride, splits, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    k = rng.standard_normal((Hkv, stride, D)).astype(np.float32)
    v = rng.standard_normal((Hkv, stride, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    out = torch.full((Hq * D,), float("nan"), device="cuda")
    gd.attn_decode_splitk(dev(q), dev(k), dev(v), out, Hq, Hkv, D, L, stride, scale, splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(Hq, D)
    want = oracle.attention_decode(q, k[:, :L], v[:, :L], scale)
    G = Hq // Hkv
    smax = max(float(np.max(np.abs(scale * (k[h // G, :L].astype(np.float64) @ q[h].astype(np.float64)))))
               for h in range(Hq))
    bound = TOL + smax * 2.0 ** -22
    err = rel_err(got, want)
    assert err <= bound, f"Hq={Hq} Hkv={Hkv} L={L} stride={stride} splits={splits}: {err:.3e} > {bound:.3e}"
