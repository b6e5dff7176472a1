"""GPU parity for the ternary bitplane path, through the C ABI.

Bar: bit-exact for the bit planes, the int32 dot and the f32 output against
the oracle (popcount identity on offset-binary planes, itself pinned to the
direct int64 sum), on seeded inputs with the BitNet-2B-like decode shapes.
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


def i32(a):
    return np.ascontiguousarray(a).view(np.int32)


def planes_ref(xq):
    """Two's-complement bit planes, written from the header's definition."""
    K = xq.size
    u = xq.view(np.uint8).astype(np.uint32)
    out = np.zeros((8, K // 32), dtype=np.uint32)
    for b in range(8):
        bits = ((u >> b) & 1).reshape(K // 32, 32)
        out[b] = (bits << np.arange(32, dtype=np.uint32)).sum(axis=1).astype(np.uint32)
    return out


def run(gd, P, N, ws, xq, xs, with_dot=True):
    rows, W = P.shape
    K = W * 32
    xp = torch.empty(8 * W, dtype=torch.int32, device="cuda")
    gd.ternary_act_bitplanes(dev(xq), 1, K, xp)
    y = torch.full((rows,), float("nan"), device="cuda")
    d = torch.full((rows,), -7, dtype=torch.int32, device="cuda") if with_dot else None
    gd.ternary_gemv(dev(i32(P)), dev(i32(N)), ws, xp, xs, y, d, rows, K)
    torch.cuda.synchronize()
    return xp.cpu().numpy().view(np.uint32), y.cpu().numpy(), None if d is None else d.cpu().numpy()


@pytest.mark.parametrize("K", [32, 96, 2560, 6912])
def test_bitplanes_match_definition(gd, K):
    rng = np.random.default_rng(K)
    xq = rng.integers(-128, 128, size=K).astype(np.int8)
    xp = torch.empty(8 * (K // 32), dtype=torch.int32, device="cuda")
    gd.ternary_act_bitplanes(dev(xq), 1, K, xp)
    torch.cuda.synchronize()
    assert np.array_equal(xp.cpu().numpy().view(np.uint32).reshape(8, -1), planes_ref(xq))


@pytest.mark.parametrize("rows,K", [(2560, 2560), (6912, 2560), (2560, 6912), (1, 32), (37, 96), (200, 4000),
                                    (100, 128), (65, 1152), (64, 8192), (10, 8320)])
def test_gemv_bit_exact(gd, rows, K):
    P, N, ws, xq, xs = wl.ternary_inputs(rows, K, seed=rows + K)
    _, y, d = run(gd, P, N, ws, xq, xs)
    yo, do = oracle.ternary_gemv(P, N, ws, xq, xs, nthreads=8)
    assert np.array_equal(d, do)
    assert np.array_equal(y.view(np.uint32), yo.view(np.uint32))


def test_extremes_and_overlap(gd):
    """x = -128 / 127 extremes, all-(+1) and all-(-1) rows, and P&N overlap
    (counted as w = 0 on both sides)."""
    rows, K = 64, 512
    rng = np.random.default_rng(3)
    w = rng.integers(-1, 2, size=(rows, K))
    w[0] = 1
    w[1] = -1
    P = wl.pack_bits_lsb((w == 1).astype(np.uint8))
    N = wl.pack_bits_lsb((w == -1).astype(np.uint8))
    both = wl.pack_bits_lsb((rng.random((rows, K)) < 0.1).astype(np.uint8))
    P2, N2 = P | both, N | both
    xq = rng.integers(-128, 128, size=K).astype(np.int8)
    xq[::5] = -128
    xq[1::7] = 127
    _, y, d = run(gd, P2, N2, 0.5, xq, 0.25)
    _, do = oracle.ternary_gemv(P2, N2, 0.5, xq, 0.25)
    assert np.array_equal(d, do)
    assert np.array_equal(d.astype(np.int64), oracle.ternary_dot_direct(P2, N2, xq))


def test_dot_out_optional(gd):
    P, N, ws, xq, xs = wl.ternary_inputs(128, 2560, 7)
    _, y1, _ = run(gd, P, N, ws, xq, xs, with_dot=False)
    yo, _ = oracle.ternary_gemv(P, N, ws, xq, xs)
    assert np.array_equal(y1.view(np.uint32), yo.view(np.uint32))


def test_grouped_decode_step_shapes(gd):
    """One layer's seven GEMVs of the decode step, as three grouped launches
    (one per shape), each problem with its own activation, against the oracle."""
    shapes = wl.bitnet_step_shapes(1)
    by_shape = {}
    for j, (rows, K) in enumerate(shapes):
        by_shape.setdefault((rows, K), []).append(j)
    keep = []
    for (rows, K), idx in by_shape.items():
        entries, refs = [], []
        xs_all = []
        for j in idx:
            P, N, ws, xq, xs = wl.ternary_inputs(rows, K, wl.TERNARY_SEED_BASE + j)
            xs_all.append(xq)
            xp = torch.empty(8 * (K // 32), dtype=torch.int32, device="cuda")
            gd.ternary_act_bitplanes(dev(xq), 1, K, xp)
            y = torch.empty(rows, device="cuda")
            d = torch.empty(rows, dtype=torch.int32, device="cuda")
            Pd, Nd = dev(i32(P)), dev(i32(N))
            entries.append((Pd, Nd, xp, y, d, ws, xs))
            refs.append(oracle.ternary_gemv(P, N, ws, xq, xs, nthreads=8))
            keep.append((Pd, Nd, xp))
        probs = gd.make_ternary_problems(entries)
        gd.ternary_gemv_grouped(probs, len(idx), rows, K)
        torch.cuda.synchronize()
        for (P_, N_, xp, y, d, ws, xs), (yo, do) in zip(entries, refs):
            assert np.array_equal(d.cpu().numpy(), do)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))


def test_batched_bitplanes(gd):
    K, count = 2560, 5
    rng = np.random.default_rng(9)
    xq = rng.integers(-128, 128, size=(count, K)).astype(np.int8)
    xp = torch.empty(count * 8 * (K // 32), dtype=torch.int32, device="cuda")
    gd.ternary_act_bitplanes(dev(xq), count, K, xp)
    torch.cuda.synchronize()
    got = xp.cpu().numpy().view(np.uint32).reshape(count, 8, K // 32)
    for c in range(count):
        assert np.array_equal(got[c], planes_ref(xq[c]))


def test_full_decode_step_as_benchmarked(gd):
    """The whole 30-layer decode step (210 GEMVs) in the launch configuration
    the benchmark times: one weight per shape shared by its GEMVs, one
    activation per GEMV, the bit planes of every token of a K in one launch,
    then one grouped launch per shape (120, 60 and 30 problems). Every dot
    and output bit-exact with the oracle."""
    shapes = wl.bitnet_step_shapes()
    assert len(shapes) == 210
    groups = {}
    for j, sh in enumerate(shapes):
        groups.setdefault(sh, []).append(j)
    base = {sh: wl.ternary_inputs(sh[0], sh[1], wl.TERNARY_SEED_BASE + 1000 + sh[0] + sh[1])[:3] for sh in groups}
    xq, xsc = {}, {}
    for j, (rows, K) in enumerate(shapes):
        rng = np.random.default_rng(wl.TERNARY_SEED_BASE + j)
        xq[j], xsc[j] = wl.absmax_int8(rng.standard_normal(K))
    planes, where = {}, {}
    for K in sorted({sh[1] for sh in shapes}):
        js = [j for j, sh in enumerate(shapes) if sh[1] == K]
        xs_dev = dev(np.stack([xq[j] for j in js]))
        planes[K] = torch.empty(len(js) * 8 * (K // 32), dtype=torch.int32, device="cuda")
        gd.ternary_act_bitplanes(xs_dev, len(js), K, planes[K])
        for pos, j in enumerate(js):
            where[j] = (K, pos)
    wdev = {sh: (dev(i32(base[sh][0])), dev(i32(base[sh][1]))) for sh in groups}
    ys = {j: torch.full((shapes[j][0],), float("nan"), device="cuda") for j in range(len(shapes))}
    ds = {j: torch.full((shapes[j][0],), -7, dtype=torch.int32, device="cuda") for j in range(len(shapes))}
    probs = {}
    for sh, idx in groups.items():
        entries = []
        for j in idx:
            K, pos = where[j]
            W = K // 32
            entries.append((wdev[sh][0], wdev[sh][1], planes[K][pos * 8 * W:(pos + 1) * 8 * W], ys[j], ds[j],
                            base[sh][2], xsc[j]))
        probs[sh] = gd.make_ternary_problems(entries)
        gd.ternary_gemv_grouped(probs[sh], len(idx), sh[0], sh[1])
    torch.cuda.synchronize()
    for j, sh in enumerate(shapes):
        P, N, ws = base[sh]
        yo, do = oracle.ternary_gemv(P, N, ws, xq[j], xsc[j], nthreads=oracle.max_threads())
        assert np.array_equal(ds[j].cpu().numpy(), do), f"GEMV {j} {sh}: dot"
        assert np.array_equal(ys[j].cpu().numpy().view(np.uint32), yo.view(np.uint32)), f"GEMV {j} {sh}: y"
