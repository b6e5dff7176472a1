"""The C ABI on a host without a GPU: the library loads, exports every
function include/gemm_decode.h declares, and rejects bad arguments with the
documented status before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)) - {"defined"})


@pytest.fixture(scope="module")
def gd():
    import gemm_decode_amd
    return gemm_decode_amd


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["q1_planes_bytes", "q1_repack", "q1_q8_gemv", "q1_q8_gemv_grouped", "q1_sign_gemm",
              "q1_sign_gemm_workspace_bytes",
              "blockq8_matmul_nt", "ternary_act_bitplanes", "ternary_gemv", "ternary_gemv_grouped",
              "q8_0_quantize", "ternary_quantize_act", "q1_sign_packed_bytes", "q1_sign_pack",
              "q1_sign_gemm_packed", "q1_sign_gemv", "q1_sign_gemm_lut4",
              "attn_decode_workspace_bytes", "attn_decode_splitk", "attn_decode_splitk_noalloc",
              "gemm_decode_status_string", "gemm_decode_last_error", "gemm_decode_abi_version",
              "gemm_decode_fill", "gemm_decode_stream_read"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(gd):
    lib = ctypes.CDLL(gd.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert lib.gemm_decode_abi_version() == gd.ABI_VERSION == 4


def test_status_strings(gd):
    L = gd.lib()
    for code, name in [(0, "GD_OK"), (-1, "GD_EINVAL"), (-2, "GD_ESHAPE"), (-3, "GD_EALIGN"),
                       (-4, "GD_EHIP"), (-5, "GD_ERANGE"), (7, "GD_UNKNOWN")]:
        assert L.gemm_decode_status_string(code).decode() == name


def test_plane_sizes(gd):
    assert gd.q1_planes_bytes(256, 1024) == (256 * 8 * 16, 256 * 8 * 2)
    assert gd.q1_planes_bytes(65, 128) == (128 * 16, 128 * 8 * 2)
    assert gd.q1_planes_bytes(14336, 4096) == (14336 * 32 * 16, 14336 * 32 * 2)
    with pytest.raises(gd.GemmDecodeError, match="GD_ESHAPE"):
        gd.q1_planes_bytes(4, 100)
    with pytest.raises(gd.GemmDecodeError, match="GD_EINVAL"):
        gd.q1_planes_bytes(0, 128)


FAKE = 0x100000   # an aligned address that is never dereferenced: validation fails first


def st(fn, *args):
    return fn(*args)


def test_validation_without_gpu(gd):
    L = gd.lib()
    E = dict(inval=-1, shape=-2, align=-3, range=-5)
    # Q1
    assert L.q1_repack(None, 4, 128, FAKE, FAKE, None) == E["inval"]
    assert L.q1_repack(FAKE + 1, 4, 128, FAKE, FAKE, None) == E["align"]
    assert L.q1_repack(FAKE, 4, 100, FAKE, FAKE, None) == E["shape"]
    assert L.q1_repack(FAKE, 4, 128, FAKE + 8, FAKE, None) == E["align"]
    assert "16-byte" in L.gemm_decode_last_error().decode()
    assert L.q1_q8_gemv(FAKE, FAKE, FAKE, FAKE, 0, 128, 1, None) == E["inval"]
    assert L.q1_q8_gemv(FAKE, FAKE, FAKE, FAKE, 4, 128, 0, None) == E["inval"]
    assert L.q1_q8_gemv(FAKE, FAKE, FAKE, FAKE, 4, 128, 70000, None) == E["range"]
    assert L.q1_q8_gemv(FAKE, FAKE, FAKE + 1, FAKE, 4, 128, 1, None) == E["align"]
    assert L.q1_q8_gemv(FAKE, FAKE, FAKE, FAKE + 2, 4, 128, 1, None) == E["align"]
    assert L.q1_q8_gemv_grouped(None, 1, 4, 128, None) == E["inval"]
    assert L.q1_q8_gemv_grouped(FAKE, 0, 4, 128, None) == E["inval"]
    assert L.q1_q8_gemv_grouped(FAKE, 65536, 4, 128, None) == E["range"]
    assert L.q1_q8_gemv_grouped(FAKE + 4, 1, 4, 128, None) == E["align"]
    # sign-bit GEMM
    WS = 1 << 20
    assert L.q1_sign_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, WS, None) == E["shape"]
    assert L.q1_sign_gemm(None, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, WS, None) == E["inval"]
    assert L.q1_sign_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 128, None, WS, None) == E["inval"]
    assert L.q1_sign_gemm(FAKE + 4, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, WS, None) == E["align"]
    assert L.q1_sign_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE + 8, WS, None) == E["align"]
    assert L.q1_sign_gemm(FAKE, FAKE, FAKE, FAKE, 0, 4, 128, FAKE, WS, None) == E["inval"]
    # workspace: 4*K bytes per token (padded to 16), 32 per padded token, 16 per output and group
    # pair, 4 per output
    ws = ctypes.c_size_t()
    assert L.q1_sign_gemm_workspace_bytes(17, 5, 128, ctypes.byref(ws)) == 0
    assert ws.value == 32 * 128 * 4 + 32 * 32 + 5 * 2 * 16 + 5 * 4
    assert L.q1_sign_gemm_workspace_bytes(17, 5, 96, ctypes.byref(ws)) == 0
    assert ws.value == 32 * 96 * 4 + 32 * 32 + 5 * 2 * 16 + 5 * 4
    assert L.q1_sign_gemm_workspace_bytes(17, 5, 100, ctypes.byref(ws)) == E["shape"]
    assert L.q1_sign_gemm(FAKE, FAKE, FAKE, FAKE, 17, 5, 128, FAKE, 32 * 128 * 4, None) == E["range"]
    # packed sign-bit weights: two sections of 16 bytes per output and group pair, 4 per output
    assert L.q1_sign_packed_bytes(5, 128, ctypes.byref(ws)) == 0 and ws.value == 2 * 5 * 2 * 16 + 5 * 4
    assert L.q1_sign_packed_bytes(5, 96, ctypes.byref(ws)) == 0 and ws.value == 2 * 5 * 2 * 16 + 5 * 4
    assert L.q1_sign_packed_bytes(5, 100, ctypes.byref(ws)) == E["shape"]
    assert L.q1_sign_pack(FAKE, FAKE, 4, 128, FAKE + 4, None) == E["align"]
    assert L.q1_sign_pack(FAKE, None, 4, 128, FAKE, None) == E["inval"]
    assert L.q1_sign_gemm_packed(FAKE, FAKE, FAKE, 17, 5, 128, FAKE, 32 * 128 * 4, None) == E["range"]
    assert L.q1_sign_gemm_packed(FAKE, FAKE + 8, FAKE, 17, 5, 128, FAKE, 1 << 20, None) == E["align"]
    for fn in (L.q1_sign_gemv, L.q1_sign_gemm_lut4):
        assert fn(FAKE, FAKE, FAKE, 1, 4, 100, None) == E["shape"]
        assert fn(FAKE, FAKE, FAKE, 0, 4, 128, None) == E["inval"]
        assert fn(FAKE + 4, FAKE, FAKE, 1, 4, 128, None) == E["align"]
        assert fn(FAKE, FAKE + 8, FAKE, 1, 4, 128, None) == E["align"]
    assert L.q1_sign_gemv(FAKE, FAKE, FAKE, 70000, 4, 128, None) == E["range"]
    # block-Q8
    assert L.blockq8_matmul_nt(FAKE, FAKE, FAKE, FAKE, 1, 100, 4, None) == E["shape"]
    assert L.blockq8_matmul_nt(FAKE, FAKE, FAKE, FAKE, 1, 960, 0, None) == E["inval"]
    assert L.blockq8_matmul_nt(FAKE, FAKE + 4, FAKE, FAKE, 1, 960, 4, None) == E["align"]
    assert L.blockq8_matmul_nt(FAKE + 4, FAKE, FAKE, FAKE, 1, 960, 4, None) == E["align"]
    assert L.blockq8_matmul_nt(FAKE, FAKE, FAKE, FAKE, 65, 960, 4, None) == E["range"]
    # ternary
    assert L.ternary_act_bitplanes(FAKE, 1, 100, FAKE, None) == E["shape"]
    assert L.ternary_act_bitplanes(FAKE, 1, 128, FAKE + 4, None) == E["align"]
    assert L.ternary_gemv(FAKE, FAKE, 1.0, FAKE, 1.0, FAKE, None, 4, 100, None) == E["shape"]
    assert L.ternary_gemv(FAKE, None, 1.0, FAKE, 1.0, FAKE, None, 4, 128, None) == E["inval"]
    assert L.ternary_gemv(FAKE, FAKE, 1.0, FAKE, 1.0, FAKE, None, 4, 1 << 20, None) == E["range"]
    assert L.ternary_gemv_grouped(FAKE, 0, 4, 128, None) == E["inval"]
    assert L.ternary_gemv_grouped(None, 1, 4, 128, None) == E["inval"]
    assert L.ternary_gemv_grouped(FAKE, 65536, 4, 128, None) == E["range"]
    assert L.ternary_gemv_grouped(FAKE, 1, 4, 100, None) == E["shape"]
    assert L.ternary_gemv_grouped(FAKE + 4, 1, 4, 128, None) == E["align"]
    assert L.ternary_gemv_grouped(FAKE, 1, 4, 1 << 17, None) == E["range"]
    # activation quantization
    assert L.q8_0_quantize(None, FAKE, 1, 128, None) == E["inval"]
    assert L.q8_0_quantize(FAKE, FAKE, 0, 128, None) == E["inval"]
    assert L.q8_0_quantize(FAKE, FAKE, 1, 100, None) == E["shape"]
    assert L.q8_0_quantize(FAKE + 4, FAKE, 1, 128, None) == E["align"]
    assert L.q8_0_quantize(FAKE, FAKE + 1, 1, 128, None) == E["align"]
    assert L.q8_0_quantize(FAKE, FAKE, 1 << 40, 1 << 20, None) == E["range"]
    assert L.ternary_quantize_act(FAKE, 1, 128, None, FAKE, None) == E["inval"]
    assert L.ternary_quantize_act(FAKE, 1, 96 + 4, FAKE, FAKE, None) == E["shape"]
    assert L.ternary_quantize_act(FAKE + 8, 1, 128, FAKE, FAKE, None) == E["align"]
    assert L.ternary_quantize_act(FAKE, 1, 128, FAKE + 2, FAKE, None) == E["align"]
    assert L.ternary_quantize_act(FAKE, 1 << 31, 128, FAKE, FAKE, None) == E["range"]
    # decode attention: workspace = splits * heads * (head_dim + 2) floats
    assert L.attn_decode_workspace_bytes(32, 8, 128, 4096, 0, ctypes.byref(ws)) == 0
    assert ws.value == 64 * 32 * 130 * 4                  # 512 workgroups over 8 KV heads
    assert L.attn_decode_workspace_bytes(32, 8, 128, 100, 0, ctypes.byref(ws)) == 0
    assert ws.value == 2 * 32 * 130 * 4                   # no more splits than 64-key tiles
    assert L.attn_decode_workspace_bytes(32, 8, 128, 4096, 3, ctypes.byref(ws)) == 0 and ws.value == 3 * 32 * 130 * 4
    assert L.attn_decode_workspace_bytes(32, 8, 64, 4096, 0, ctypes.byref(ws)) == E["shape"]
    assert L.attn_decode_workspace_bytes(24, 8, 128, 4096, 0, ctypes.byref(ws)) == E["shape"]
    assert L.attn_decode_workspace_bytes(48, 3, 128, 4096, 0, ctypes.byref(ws)) == E["shape"]   # 16 per KV head
    assert L.attn_decode_workspace_bytes(32, 8, 128, 0, 0, ctypes.byref(ws)) == E["inval"]
    att = (32, 8, 128, 4096, 4096, 0.1, 0)
    assert L.attn_decode_splitk(FAKE, FAKE, FAKE, FAKE, 32, 8, 128, 4096, 4000, 0.1, 0, FAKE, 1 << 30, None) == \
        E["inval"]
    assert L.attn_decode_splitk(FAKE + 4, FAKE, FAKE, FAKE, *att, FAKE, 1 << 30, None) == E["align"]
    assert L.attn_decode_splitk(FAKE, FAKE, FAKE, FAKE, *att, FAKE, 1024, None) == E["range"]
    assert L.attn_decode_splitk(FAKE, FAKE, FAKE, FAKE, 32, 8, 128, 4096, 4096, 0.1, 70000, FAKE, 1 << 30, None) == \
        E["range"]
    # measurement
    assert L.gemm_decode_fill(FAKE, 100, 1, None) == E["shape"]
    assert L.gemm_decode_stream_read(FAKE, 160, 0, FAKE, 1, None) == E["inval"]


def test_attention_noalloc_validation_before_any_hip_call(gd):
    """The no-allocation attention entry point rejects, without touching the
    device: null pointers, and shapes whose split partials would not fit its
    fixed scratch (GD_ATTN_NOALLOC_MAX_BYTES = 4 MiB)."""
    L = gd.lib()
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    p16 = p + (-p) % 16
    assert L.attn_decode_splitk_noalloc(None, p16, p16, p16, 32, 8, 128, 4096, 4096, 0.1, 0, None) == gd.GD_EINVAL
    # 64 heads x 1024 splits x 130 floats = 34 MB of partials > 4 MiB
    assert L.attn_decode_splitk_noalloc(p16, p16, p16, p16, 64, 8, 128, 1 << 20, 1 << 20, 0.1, 1024,
                                        None) == gd.GD_ERANGE
    assert "scratch" in L.gemm_decode_last_error().decode()
