"""GPU parity for the Q1_0 . q8_0 path (repack + GEMV), through the C ABI.

Bar: bit-exact. The planes must equal the declared layout (written by the
test helper q1_layout) byte for byte; every output's f32 bits must equal the
oracle's (form F1, the page "browseml-gpu.js" arithmetic). Inputs are seeded and synthetic; -128 quants
and random f16 exponents come from the page's randomCase generator.
"""
import numpy as np
import pytest

import oracle
import q1_layout
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


def planes_on_gpu(gd, W, rows, K):
    b, s = gd.q1_alloc_planes(rows, K)
    b.fill_(0xA5)
    s.fill_(0x5A)   # the repack must overwrite every byte, padding included
    gd.q1_repack(dev(W.reshape(-1)), rows, K, b, s)
    return b, s


def run_gemv(gd, W, A, rows, K, n_act=1):
    b, s = planes_on_gpu(gd, W, rows, K)
    y = torch.full((n_act * rows,), float("nan"), dtype=torch.float32, device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y, rows, K, n_act)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(n_act, rows)


def assert_bits_equal(got, want, what=""):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32)
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, (f"{what}: {bad.size} outputs differ; first: "
                           + ", ".join(f"[{i}] gpu={g.reshape(-1)[i]:#010x} ref={w.reshape(-1)[i]:#010x}"
                                       for i in bad[:16]))


@pytest.mark.parametrize("rows,K", [(1, 128), (63, 256), (65, 1024), (256, 1024), (300, 1152), (1000, 4224)])
def test_repack_matches_oracle_planes(gd, rows, K):
    W = wl.q1_weights_aos(rows, K, seed=rows * 7 + K)
    b, s = planes_on_gpu(gd, W, rows, K)
    torch.cuda.synchronize()
    ob, os_ = q1_layout.q1_planes(W, rows, K)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), ob)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), os_)


def test_gemv_small_config_bit_exact(gd):
    """Q1_0.q8_0 GEMV, rows=256, K=1024, batch 1 (the correctness-sized case)."""
    cfg = wl.Q1_SMALL
    W = wl.q1_weights_aos(cfg.rows, cfg.K, cfg.weight_seed)
    A = wl.q8_acts_aos(cfg.K, cfg.act_seeds[0])
    y = run_gemv(gd, W, A, cfg.rows, cfg.K)
    assert_bits_equal(y, oracle.q1_q8_gemv_aos(W, A, cfg.rows, cfg.K), "rows=256 K=1024")


def test_page_exact_protocol(gd):
    """The page's exact() protocol: randomCase(256, 2048, seed 1) row by row,
    then five activations through the several-column entry point, each
    column against its own oracle result."""
    rows, n = 256, 2048
    W, A = wl.random_case(rows, n, 1)
    As = np.concatenate([A] + [wl.random_case(1, n, 100 + k)[1] for k in range(1, 5)])
    y1 = run_gemv(gd, W, A, rows, n)
    assert_bits_equal(y1, oracle.q1_q8_gemv_aos(W, A, rows, n), "randomCase single")
    y5 = run_gemv(gd, W, As, rows, n, n_act=5)
    assert_bits_equal(y5, oracle.q1_q8_gemv_aos(W, As, rows, n, n_act=5, nthreads=8), "randomCase x5")


@pytest.mark.parametrize("rows,K,seed", [(1, 128, 1), (63, 128, 2), (65, 384, 3), (257, 1024, 4),
                                         (1000, 4224, 5), (130, 8192, 6)])
def test_ragged_and_chunked_shapes(gd, rows, K, seed):
    """Rows off the 64/256 tiles, one-block rows (K=128), and K past one LDS
    table chunk of 32 blocks (K=4224, 8192)."""
    W, A = wl.random_case(rows, K, seed)
    y = run_gemv(gd, W, A, rows, K)
    assert_bits_equal(y, oracle.q1_q8_gemv_aos(W, A, rows, K, nthreads=8), f"rows={rows} K={K}")


@pytest.mark.parametrize("n_act", [2, 3, 4, 5, 7, 8, 9, 16])
@pytest.mark.parametrize("rows,K", [(65, 128), (300, 1152), (257, 4608), (64, 8192)])
def test_multi_column_bit_exact(gd, n_act, rows, K):
    """Several activation columns against one weight (the small-M product),
    each column its own GEMV in one launch; K covers one block, short last
    chunks and several chunks; every column must carry the bits of its own
    batch-1 GEMV."""
    W = wl.q1_weights_aos(rows, K, rows + K)
    A = np.concatenate([wl.q8_acts_aos(K, 7000 + 31 * c + K) for c in range(n_act)])
    got = run_gemv(gd, W, A, rows, K, n_act)
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n_act, nthreads=oracle.max_threads())
    assert_bits_equal(got.reshape(n_act, rows), want.reshape(n_act, rows), f"n_act={n_act} {rows}x{K}")


@pytest.mark.parametrize("rows,K,n_act", [
    (14329, 4096, 16),   # 56 row blocks x 16 columns: two workgroups per CU
    (14329, 4096, 29),   # more workgroups than fit on the CUs at once
    (12289, 1152, 16),   # 49 row blocks, 9 blocks per row (a short last group)
    (12289, 1152, 40),   # 40 grid rows of columns, short chunks
    (14336, 4096, 4),    # the decode weight, 224 workgroups
    (10000, 1152, 6),    # a ragged last row block
    (12545, 1152, 6),    # one row past a 256-row block
])
def test_multi_column_wide_groups(gd, rows, K, n_act):
    """Many columns over wide weights (the 256-row kernel, one grid row per
    column, up to several workgroups per CU); every column bit-exact with
    its own batch-1 GEMV."""
    W = wl.q1_weights_aos(rows, K, 11 + n_act)
    A = np.concatenate([wl.q8_acts_aos(K, 9000 + c) for c in range(n_act)])
    got = run_gemv(gd, W, A, rows, K, n_act)
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n_act, nthreads=oracle.max_threads())
    assert_bits_equal(got.reshape(n_act, rows), want.reshape(n_act, rows), f"n_act={n_act} {rows}x{K}")


@pytest.mark.parametrize("rows,K", [
    (4096, 4096),     # one chunk of 32 blocks, 16-row workgroups (128 x 32 rows fill half the CUs)
    (4097, 1024),     # 129 x 32 rows: 32-row workgroups
    (2000, 4224),     # two chunks: 32-row workgroups (16-row ones only for one chunk)
    (8191, 4224),     # a full chunk whose next chunk is one block long
    (8192, 8192),     # 64-row workgroups, two full chunks
    (14336, 4096),    # 64-row workgroups
    (16384, 1152),    # the largest row count on the one-chain-per-thread kernel
    (16385, 256),     # the first on the four-chain kernel (128-row workgroups)
    (20000, 4224),
    (32768, 256),     # 128 row blocks of 256: the last 128-row grid
    (32769, 256),     # the first 256-row grid
])
def test_single_gemv_paths(gd, rows, K):
    """Batch-1 GEMVs across the single-GEMV mappings (one chain per thread
    for up to 64 row blocks of 256, in 16-, 32- or 64-row workgroups; four
    per thread above: 128-row workgroups up to 128 row blocks, 256-row ones
    beyond), bit-exact, and nothing written past the last row."""
    W = wl.q1_weights_aos(rows, K, rows % 97 + K)
    A = wl.q8_acts_aos(K, 31 * rows + K)
    b, s = planes_on_gpu(gd, W, rows, K)
    y = torch.full((rows + 64,), float("nan"), dtype=torch.float32, device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y[:rows], rows, K, 1)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, nthreads=oracle.max_threads())
    assert_bits_equal(got[:rows], want.reshape(-1), f"{rows}x{K}")
    assert np.all(np.isnan(got[rows:])), "wrote past the last row"


@pytest.mark.parametrize("rows,K,n_act", [
    (4096, 4096, 4),     # n_act * rows = 16384: the one-chain-per-thread kernel per column
    (4096, 4096, 5),     # just past it: the 256-row kernel per column
    (8192, 8192, 2),     # at it with 64-row workgroups and two full chunks
    (2049, 1152, 8),     # just past it, short chunks
    (14336, 4096, 2),    # the decode weight, two columns: 128-row workgroups
    (300, 4224, 3),      # a chunk of one block
    (16384, 256, 2),     # 64 row blocks x 2 columns = 128: the last 128-row grid
    (16385, 256, 2),     # 65 x 2 = 130: the first 256-row grid
])
def test_columns_across_the_dispatch_boundary(gd, rows, K, n_act):
    """Several columns on either side of the switches between the
    one-chain-per-thread kernel, 128-row workgroups (while 256-row ones would
    fill at most half the CUs) and 256-row workgroups: every column
    bit-exact with its own batch-1 GEMV, nothing written past the last
    column."""
    W = wl.q1_weights_aos(rows, K, rows + 3 * n_act)
    A = np.concatenate([wl.q8_acts_aos(K, 500 + 17 * c + rows) for c in range(n_act)])
    b, s = planes_on_gpu(gd, W, rows, K)
    y = torch.full((n_act * rows + 64,), float("nan"), dtype=torch.float32, device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y[:n_act * rows], rows, K, n_act)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n_act, nthreads=oracle.max_threads())
    assert_bits_equal(got[:n_act * rows].reshape(n_act, rows), want.reshape(n_act, rows), f"{rows}x{K} n={n_act}")
    assert np.all(np.isnan(got[n_act * rows:])), "wrote past the last column"


def test_special_scales_and_bits(gd):
    """Subnormal, zero and large d0/d1, all-ones and all-zeros sign bits."""
    rows, K = 128, 1024
    W, A = wl.random_case(rows, K, 42)
    W = W.reshape(rows, K // 128, 18).copy()
    sub = np.array([0x0001, 0x03FF, 0x8001, 0x0000, 0x8000, 0x7BFF, 0x0400], dtype=np.uint16)
    W[:, :, 0:2] = sub[np.arange(rows * (K // 128)) % sub.size].reshape(rows, K // 128, 1).view(np.uint8)
    W[0, :, 2:] = 0xFF
    W[1, :, 2:] = 0x00
    A = A.reshape(K // 32, 34).copy()
    A[::3, 0:2] = np.array([0x0001], dtype=np.uint16).view(np.uint8)
    A[1::5, 0:2] = np.array([0x7800], dtype=np.uint16).view(np.uint8)
    y = run_gemv(gd, W, A, rows, K)
    assert_bits_equal(y, oracle.q1_q8_gemv_aos(W, A, rows, K), "special scales")


def _decode_set(rows, K, n_vec, seed_w, seeds_a):
    W = wl.q1_weights_aos(rows, K, seed_w)
    A = np.concatenate([wl.q8_acts_aos(K, s) for s in seeds_a[:n_vec]])
    return W, A


@pytest.mark.parametrize("idx", [0, 1])
def test_decode_shapes_grouped_full(gd, idx):
    """The decode shapes (4096x4096 and 14336x4096, 32 activation vectors),
    run as one grouped launch of 32 batch-1 problems over distinct plane
    copies, every output compared with the oracle."""
    cfg = wl.Q1_DECODE[idx]
    rows, K, n = cfg.rows, cfg.K, len(cfg.act_seeds)
    W, A = _decode_set(rows, K, n, cfg.weight_seed, cfg.act_seeds)
    b, s = planes_on_gpu(gd, W, rows, K)
    copies = [(b.clone(), s.clone()) for _ in range(n)]
    a_dev = [dev(A[c]) for c in range(n)]
    ys = [torch.full((rows,), float("nan"), device="cuda") for _ in range(n)]
    probs = gd.make_q1_problems([(copies[c][0], copies[c][1], a_dev[c], ys[c]) for c in range(n)])
    gd.q1_q8_gemv_grouped(probs, n, rows, K)
    torch.cuda.synchronize()
    got = np.stack([y.cpu().numpy() for y in ys])
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n, nthreads=oracle.max_threads())
    assert_bits_equal(got, want, f"decode {rows}x{K} grouped")
    # the multi-column entry point on the same inputs gives the same bits
    y = torch.empty(n * rows, device="cuda")
    gd.q1_q8_gemv(b, s, dev(A.reshape(-1)), y, rows, K, n)
    torch.cuda.synchronize()
    assert_bits_equal(y.cpu().numpy().reshape(n, rows), want, "n_act=32")


def test_decode_step_as_benchmarked(gd):
    """The decode step exactly as the benchmark builds and launches it: 32
    activation vectors against 4096x4096 and 14336x4096 (K = 4096), the 64
    problems in ONE grouped launch, each with its own copy of the planes and
    its own row count, the launch's rows 14336. Every output of all 64
    problems bit-exact with the oracle, and nothing written past a
    problem's rows."""
    import bench
    shapes = wl.Q1_DECODE
    K, n = shapes[0].K, len(shapes[0].act_seeds)
    Ws = [wl.q1_weights_aos(s.rows, s.K, s.weight_seed) for s in shapes]
    A = np.concatenate([wl.q8_acts_aos(K, sd) for sd in shapes[0].act_seeds])
    a_dev = [dev(A[c]) for c in range(n)]
    base = [planes_on_gpu(gd, W, s.rows, K) for s, W in zip(shapes, Ws)]
    copies = [[(b.clone(), sc.clone()) for _ in range(n)] for (b, sc) in base]
    guard = 64
    bufs = [[torch.full((s.rows + guard,), float("nan"), device="cuda") for _ in range(n)] for s in shapes]
    ys = [[bufs[si][c][:s.rows] for c in range(n)] for si, s in enumerate(shapes)]
    probs = bench.q1_step_problems(gd, shapes, copies, a_dev, ys)
    bench.q1_step_launch(gd, probs, shapes, n)
    torch.cuda.synchronize()
    for si, (s, W) in enumerate(zip(shapes, Ws)):
        got = np.stack([bufs[si][c].cpu().numpy() for c in range(n)])
        want = oracle.q1_q8_gemv_aos(W, A, s.rows, K, n_act=n, nthreads=oracle.max_threads())
        assert_bits_equal(got[:, :s.rows], want.reshape(n, s.rows), f"decode step {s.rows}x{K}")
        assert np.all(np.isnan(got[:, s.rows:])), f"{s.rows}x{K}: wrote past a problem's rows"


def test_deterministic_repeat(gd):
    rows, K = 4096, 4096
    W = wl.q1_weights_aos(rows, K, 1)
    A = wl.q8_acts_aos(K, 1000)
    b, s = planes_on_gpu(gd, W, rows, K)
    a = dev(A.reshape(-1))
    outs = []
    for _ in range(3):
        y = torch.empty(rows, device="cuda")
        gd.q1_q8_gemv(b, s, a, y, rows, K, 1)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert_bits_equal(outs[1], outs[0], "repeat 1")
    assert_bits_equal(outs[2], outs[0], "repeat 2")


@pytest.mark.parametrize("K", [128, 640, 1024, 1152])
def test_grouped_mixed_rows(gd, K):
    """One grouped launch over problems of different row counts (common K):
    each output bit-exact with the oracle for its own shape, nothing written
    past a problem's rows, and rows = 0 meaning the launch's rows. K up to
    1024 (one block, a partial and a full group of eight) takes the one-group
    kernel, 1152 the general one."""
    rows_max = 1000
    shapes = [(1000, 1000), (300, 300), (65, 65), (1000, 0), (1, 1), (257, 257)]   # (rows, field)
    entries, keep, wants = [], [], []
    for i, (rows, field) in enumerate(shapes):
        W = wl.q1_weights_aos(rows, K, 40 + i + K)
        A = wl.q8_acts_aos(K, 4000 + i + K)
        b, s = planes_on_gpu(gd, W, rows, K)
        a = dev(A.reshape(-1))
        y = torch.full((rows + 64,), float("nan"), device="cuda")      # 64 guard elements
        entries.append((b, s, a, y, field))
        keep.append((b, s, a, y, rows))
        wants.append(oracle.q1_q8_gemv_aos(W, A, rows, K, nthreads=oracle.max_threads()))
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, len(entries), rows_max, K)
    torch.cuda.synchronize()
    for (b, s, a, y, rows), want in zip(keep, wants):
        got = y.cpu().numpy()
        assert_bits_equal(got[:rows], want.reshape(-1), f"rows {rows}")
        assert np.all(np.isnan(got[rows:])), f"rows {rows}: wrote past its rows"


@pytest.mark.parametrize("K", [2048, 3072, 4096])
def test_grouped_units_per_workgroup(gd, K):
    """K of 16, 24 or 32 blocks (whole groups of eight, one table chunk)
    runs several consecutive 256-row units of a problem per workgroup, each
    unit's first groups loaded during the previous unit's last ones. Row
    counts of one unit, of a last unit that is partial or a single row, of
    unit counts that leave the last workgroup with one, two or all of its
    units, and of many units, plus rows = 0 (the launch's rows): every
    output bit-exact with the oracle for its own rows, nothing written past
    them."""
    rows_max = 1800
    shapes = [(256, 256), (257, 257), (300, 300), (512, 512), (700, 700), (1, 1), (1800, 0), (1537, 1537),
              (64, 64), (511, 511), (768, 768), (1025, 1025)]   # (rows, rows field)
    entries, keep, wants = [], [], []
    for i, (rows, field) in enumerate(shapes):
        W = wl.q1_weights_aos(rows, K, 90 + i + K)
        A = wl.q8_acts_aos(K, 9000 + i + K)
        b, s = planes_on_gpu(gd, W, rows, K)
        a = dev(A.reshape(-1))
        y = torch.full((rows + 64,), float("nan"), device="cuda")      # 64 guard elements
        entries.append((b, s, a, y, field))
        keep.append((b, s, a, y, rows))
        wants.append(oracle.q1_q8_gemv_aos(W, A, rows, K, nthreads=oracle.max_threads()))
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, len(entries), rows_max, K)
    torch.cuda.synchronize()
    for (b, s, a, y, rows), want in zip(keep, wants):
        got = y.cpu().numpy()
        assert_bits_equal(got[:rows], want.reshape(-1), f"K {K} rows {rows}")
        assert np.all(np.isnan(got[rows:])), f"K {K} rows {rows}: wrote past its rows"


@pytest.mark.parametrize("count", [72, 300])
def test_grouped_k4096_mixed_problems(gd, count):
    """A grouped launch at K = 4096 (one 32-block chunk per row) over many
    problems of mixed row counts (1 to the launch's rows, ragged tails,
    rows = 0 meaning the launch's rows), consecutive problems sharing one
    activation buffer in pairs, several problems reading prefixes of the
    same planes; 72 problems (more than one 64-wide pass over the problem
    list) and 300 problems of few rows each. Every output bit-exact with the
    oracle for its own rows, nothing written past them."""
    K, rows_max = 4096, 5000
    Ws = [wl.q1_weights_aos(5000, K, 71), wl.q1_weights_aos(4999, K, 72)]
    nacts = 8
    A = np.concatenate([wl.q8_acts_aos(K, 7100 + c) for c in range(nacts)])
    planes = [planes_on_gpu(gd, W, W.shape[0], K) for W in Ws]
    a_dev = [dev(A[c]) for c in range(nacts)]
    want_full = [oracle.q1_q8_gemv_aos(W, A, W.shape[0], K, n_act=nacts, nthreads=oracle.max_threads())
                 .reshape(nacts, W.shape[0]) for W in Ws]
    if count == 72:
        cycle = [(0, 5000, 5000), (1, 4999, 4999), (0, 1, 1), (1, 65, 65), (0, 300, 300), (1, 1000, 1000),
                 (0, 4096, 4096), (0, 5000, 0)]   # (weights, rows, rows field)
    else:
        cycle = [(0, 65, 65), (1, 1, 1), (0, 64, 64), (1, 129, 129), (0, 7, 7)]
    entries, checks = [], []
    for i in range(count):
        wi, rows, field = cycle[i % len(cycle)]
        act = (i // 2) % nacts   # pairs of consecutive problems share an activation buffer
        y = torch.full((rows + 64,), float("nan"), device="cuda")   # 64 guard elements
        entries.append((planes[wi][0], planes[wi][1], a_dev[act], y, field))
        checks.append((y, want_full[wi][act][:rows], rows, i))
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, count, rows_max, K)
    torch.cuda.synchronize()
    for y, want, rows, i in checks:
        got = y.cpu().numpy()
        assert_bits_equal(got[:rows], want, f"problem {i} rows {rows}")
        assert np.all(np.isnan(got[rows:])), f"problem {i} rows {rows}: wrote past its rows"


def test_grouped_graph_replay(gd):
    """The grouped launch captured in a HIP graph (as the benchmark replays
    it): four replays, with eager launches and host synchronisation between
    them, each bit-exact with the oracle."""
    rows, K, n = 1000, 4096, 6
    W = wl.q1_weights_aos(rows, K, 21)
    A = np.concatenate([wl.q8_acts_aos(K, 2100 + c) for c in range(n)])
    b, s = planes_on_gpu(gd, W, rows, K)
    a_dev = [dev(A[c]) for c in range(n)]
    ys = [torch.full((rows,), float("nan"), device="cuda") for _ in range(n)]
    probs = gd.make_q1_problems([(b, s, a_dev[c], ys[c]) for c in range(n)])
    want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=n, nthreads=oracle.max_threads())
    gd.q1_q8_gemv_grouped(probs, n, rows, K)      # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        gd.q1_q8_gemv_grouped(probs, n, rows, K)
    other = torch.empty(rows, device="cuda")
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        gd.q1_q8_gemv(b, s, a_dev[rep % n], other, rows, K, 1)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = np.stack([y.cpu().numpy() for y in ys])
        assert_bits_equal(got, want, f"replay {rep}")
        assert_bits_equal(other.cpu().numpy(), want[rep % n], f"eager between replays {rep}")


def test_validation_errors_raise(gd):
    b, s = gd.q1_alloc_planes(64, 128)
    y = torch.empty(64, device="cuda")
    a = torch.zeros(4 * 34, dtype=torch.uint8, device="cuda")
    with pytest.raises(gd.GemmDecodeError, match="GD_ESHAPE"):
        gd._check(gd.lib().q1_q8_gemv(b.data_ptr(), s.data_ptr(), a.data_ptr(), y.data_ptr(), 64, 100, 1, None))
    with pytest.raises(gd.GemmDecodeError, match="GD_EALIGN"):
        gd._check(gd.lib().q1_q8_gemv(b.data_ptr() + 4, s.data_ptr(), a.data_ptr(), y.data_ptr(), 64, 128, 1,
                                      None))


def test_small_config_grouped_as_benchmarked(gd):
    """The 256x1024 config in the launch the benchmark times: 7,646
    independent problems in one grouped launch (the one-group kernel).
    Problem p reads weight set p % 4 and activation (p // 4) % 3, so a
    problem mapped to the wrong planes, activation or output shows; every
    output bit-exact with the oracle."""
    cfg = wl.Q1_SMALL
    rows, K, count = cfg.rows, cfg.K, 7646
    Ws = [wl.q1_weights_aos(rows, K, cfg.weight_seed + w) for w in range(4)]
    As = [wl.q8_acts_aos(K, cfg.act_seeds[0] + a) for a in range(3)]
    planes = [planes_on_gpu(gd, W, rows, K) for W in Ws]
    acts = [dev(A.reshape(-1)) for A in As]
    y = torch.full((count * rows,), float("nan"), device="cuda")
    entries = [(planes[p % 4][0], planes[p % 4][1], acts[(p // 4) % 3], y[p * rows:(p + 1) * rows])
               for p in range(count)]
    probs = gd.make_q1_problems(entries)
    gd.q1_q8_gemv_grouped(probs, count, rows, K)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(count, rows)
    want = {(w, a): oracle.q1_q8_gemv_aos(Ws[w], As[a], rows, K).reshape(-1) for w in range(4) for a in range(3)}
    for p in range(count):
        assert_bits_equal(got[p], want[(p % 4, (p // 4) % 3)], f"problem {p}")
