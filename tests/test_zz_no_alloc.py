"""GPU test of the no-allocation entry point attn_decode_splitk_noalloc,
through the C ABI: it must give the results of attn_decode_splitk (same
kernels, same split plan: bit for bit) and meet the attention bar against the
oracle, on two calls in a row, the second with a smaller input (the scratch
keeps the first call's partials; nothing of them may show)."""
import ctypes

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def gd():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible HIP device")
    import gemm_decode_amd
    return gemm_decode_amd


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def case(Hq, Hkv, L, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    k = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    return q, k, v


def bar(q, k, scale, Hkv):
    G = q.shape[0] // Hkv
    smax = max(float(np.max(np.abs(scale * (k[h // G].astype(np.float64) @ q[h].astype(np.float64)))))
               for h in range(q.shape[0]))
    return 1e-5 + smax * 2.0 ** -22


def test_noalloc_matches_workspace_entry_point(gd):
    scale = 1.0 / np.sqrt(D)
    # first the decode shape (64 splits x 32 heads), then a smaller call
    for n, (Hq, Hkv, L, splits) in enumerate([(32, 8, 4096, 0), (8, 2, 777, 5)]):
        q, k, v = case(Hq, Hkv, L, 300 + n)
        qd, kd, vd = dev(q), dev(k), dev(v)
        ws = torch.full((gd.attn_decode_workspace_bytes(Hq, Hkv, D, L, splits),), 0x5A, dtype=torch.uint8,
                        device="cuda")
        o_ws = torch.full((Hq * D,), float("nan"), device="cuda")
        o_na = torch.full((Hq * D,), float("nan"), device="cuda")
        gd.attn_decode_splitk(qd, kd, vd, o_ws, Hq, Hkv, D, L, L, scale, splits, ws)
        gd.attn_decode_splitk_noalloc(qd, kd, vd, o_na, Hq, Hkv, D, L, L, scale, splits)
        torch.cuda.synchronize()
        a, b = o_ws.cpu().numpy(), o_na.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {n}: differs from attn_decode_splitk"
        want = oracle.attention_decode(q, k, v, scale)
        err = float(np.max(np.abs(b.reshape(Hq, D).astype(np.float64) - want)) / np.max(np.abs(want)))
        assert err <= bar(q, k, scale, Hkv), f"call {n}: {err:.3e}"


def test_noalloc_rejects_beyond_scratch(gd):
    """A shape whose partials exceed the scratch is refused before any launch."""
    q, k, v = case(64, 8, 2048, 1)
    out = torch.empty(64 * D, device="cuda")
    with pytest.raises(gd.GemmDecodeError, match="GD_ERANGE"):
        gd.attn_decode_splitk_noalloc(dev(q), dev(k), dev(v), out, 64, 8, D, 2048, 2048, 0.1, 1024)
