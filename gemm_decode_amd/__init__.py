"""Thin Python binding of libgemm_decode.so (ctypes).

Argument marshalling only: each function checks that tensors live on a HIP
device with the expected dtype, size and contiguity, passes their
``data_ptr()`` and torch's current stream to the C entry point of the same
name (declared in include/gemm_decode.h), and raises on a non-zero status.
Every step of the computation runs in the library's HIP kernels; there is no
fallback. Importing this package fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_decode.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python gemm_decode_amd/build.py) first")

_lib = ctypes.CDLL(LIB_PATH)

GD_OK, GD_EINVAL, GD_ESHAPE, GD_EALIGN, GD_EHIP, GD_ERANGE = 0, -1, -2, -3, -4, -5

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F32 = ctypes.c_float


class GemmDecodeError(RuntimeError):
    def __init__(self, status: int, text: str):
        self.status = status
        name = _lib.gemm_decode_status_string(status).decode()
        super().__init__(f"{name}: {text}")


class Q1Problem(ctypes.Structure):
    """gd_q1_problem: one batch-1 problem of q1_q8_gemv_grouped."""
    _fields_ = [("bits_plane", _P), ("scale_plane", _P), ("a_q8", _P), ("y", _P), ("rows", _I64)]


class TernaryProblem(ctypes.Structure):
    """gd_ternary_problem: one problem of ternary_gemv_grouped."""
    _fields_ = [("w_pos", _P), ("w_neg", _P), ("x_planes", _P), ("y", _P),
                ("dot_out", _P), ("w_scale", _F32), ("x_scale", _F32), ("x_scale_dev", _P)]


def _declare():
    L = _lib
    L.gemm_decode_status_string.argtypes = [ctypes.c_int]
    L.gemm_decode_status_string.restype = ctypes.c_char_p
    L.gemm_decode_last_error.argtypes = []
    L.gemm_decode_last_error.restype = ctypes.c_char_p
    L.gemm_decode_abi_version.restype = ctypes.c_int
    sig = {
        "q1_planes_bytes": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)],
        "q1_repack": [_P, _I64, _I64, _P, _P, _P],
        "q1_q8_gemv": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
        "q1_q8_gemv_grouped": [_P, _I64, _I64, _I64, _P],
        "q1_sign_gemm": [_P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
        "q1_sign_gemm_workspace_bytes": [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
        "q1_sign_packed_bytes": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
        "q1_sign_pack": [_P, _P, _I64, _I64, _P, _P],
        "q1_sign_gemm_packed": [_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
        "q1_sign_gemv": [_P, _P, _P, _I64, _I64, _I64, _P],
        "q1_sign_gemm_lut4": [_P, _P, _P, _I64, _I64, _I64, _P],
        "blockq8_matmul_nt": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
        "ternary_act_bitplanes": [_P, _I64, _I64, _P, _P],
        "ternary_gemv": [_P, _P, _F32, _P, _F32, _P, _P, _I64, _I64, _P],
        "ternary_gemv_grouped": [_P, _I64, _I64, _I64, _P],
        "q8_0_quantize": [_P, _P, _I64, _I64, _P],
        "attn_decode_workspace_bytes": [_I64, _I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
        "attn_decode_splitk": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F32, _I64, _P, ctypes.c_size_t, _P],
        "attn_decode_splitk_noalloc": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F32, _I64, _P],
        "ternary_quantize_act": [_P, _I64, _I64, _P, _P, _P],
        "gemm_decode_fill": [_P, ctypes.c_size_t, ctypes.c_uint32, _P],
        "gemm_decode_stream_read": [_P, ctypes.c_size_t, ctypes.c_int32, _P, _I64, _P],
    }
    for name, args in sig.items():
        fn = getattr(L, name, None)
        if fn is None:
            continue
        fn.argtypes = args
        fn.restype = ctypes.c_int


_declare()

# The problem structs below mirror the header of this ABI version; a library
# built from other sources would read them with another layout.
ABI_VERSION = 4
if _lib.gemm_decode_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {_lib.gemm_decode_abi_version()}, this binding needs "
                      f"{ABI_VERSION}: rebuild it")


def lib():
    return _lib


def _check(status: int):
    if status != GD_OK:
        raise GemmDecodeError(status, _lib.gemm_decode_last_error().decode())


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dev(t, dtype, numel=None, name="tensor"):
    """data_ptr of a contiguous device tensor of the given dtype (and size)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


# --------------------------------------------------------------- Q1_0.q8_0

def q1_planes_bytes(rows: int, K: int):
    b, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.q1_planes_bytes(rows, K, ctypes.byref(b), ctypes.byref(s)))
    return b.value, s.value


def q1_repack(w_aos, rows: int, K: int, bits_plane, scale_plane):
    import torch
    bb, sb = q1_planes_bytes(rows, K)
    _check(_lib.q1_repack(_dev(w_aos, torch.uint8, rows * (K // 128) * 18, "w_aos"), rows, K,
                          _dev(bits_plane, torch.uint8, bb, "bits_plane"),
                          _dev(scale_plane, torch.uint8, sb, "scale_plane"), _stream()))


def q1_alloc_planes(rows: int, K: int, device="cuda"):
    """Allocates (bits_plane, scale_plane) uint8 device tensors of the right size."""
    import torch
    bb, sb = q1_planes_bytes(rows, K)
    return (torch.empty(bb, dtype=torch.uint8, device=device),
            torch.empty(sb, dtype=torch.uint8, device=device))


def q1_q8_gemv(bits_plane, scale_plane, a_q8, y, rows: int, K: int, n_act: int = 1):
    import torch
    bb, sb = q1_planes_bytes(rows, K)
    _check(_lib.q1_q8_gemv(_dev(bits_plane, torch.uint8, bb, "bits_plane"),
                           _dev(scale_plane, torch.uint8, sb, "scale_plane"),
                           _dev(a_q8, torch.uint8, n_act * (K // 32) * 34, "a_q8"),
                           _dev(y, torch.float32, n_act * rows, "y"), rows, K, n_act, _stream()))


def q1_q8_gemv_grouped(problems, count: int, rows: int, K: int):
    """problems: device uint8 tensor holding `count` gd_q1_problem structs
    (see make_q1_problems)."""
    import torch
    _check(_lib.q1_q8_gemv_grouped(_dev(problems, torch.uint8, count * ctypes.sizeof(Q1Problem), "problems"),
                                   count, rows, K, _stream()))


def make_q1_problems(entries, device="cuda"):
    """Device array of gd_q1_problem from [(bits_plane, scale_plane, a_q8, y[, rows]), ...]
    (rows 0 or absent: the launch's rows)."""
    import torch
    arr = (Q1Problem * len(entries))()
    for i, e in enumerate(entries):
        b, s, a, y = e[:4]
        arr[i] = Q1Problem(b.data_ptr(), s.data_ptr(), a.data_ptr(), y.data_ptr(), e[4] if len(e) > 4 else 0)
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device)


# --------------------------------------------------------- sign-bit GEMM

def q1_sign_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.q1_sign_gemm_workspace_bytes(M, N, K, ctypes.byref(out)))
    return out.value


_sign_ws = {}


def _sign_workspace(M: int, N: int, K: int, device=None):
    """The per-device cached sign-GEMM workspace, grown to the call's need."""
    import torch
    need = q1_sign_gemm_workspace_bytes(M, N, K) if K >= 32 and K % 32 == 0 else 16
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    ws = _sign_ws.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _sign_ws[dev] = ws
    return ws


def q1_sign_gemm(x, w_bits, w_scales, y, M: int, N: int, K: int, workspace=None):
    """y = x @ w^T for sign-bit weights. `workspace` (a uint8 CUDA tensor of
    at least q1_sign_gemm_workspace_bytes(M, N, K)) defaults to one cached per
    device, grown as needed and shared by every call on that device that
    passes none: pass your own to run calls on several streams at once."""
    import torch
    G = K // 32 if K % 32 == 0 else -1
    if workspace is None:
        workspace = _sign_workspace(M, N, K, x.device)
    _check(_lib.q1_sign_gemm(_dev(x, torch.float32, M * K, "x"),
                             _dev(w_bits, torch.int32, N * G if G > 0 else None, "w_bits"),
                             _dev(w_scales, torch.float32, N * G if G > 0 else None, "w_scales"),
                             _dev(y, torch.float32, M * N, "y"), M, N, K,
                             _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()))


def q1_sign_packed_bytes(N: int, K: int) -> int:
    b = ctypes.c_size_t()
    _check(_lib.q1_sign_packed_bytes(N, K, ctypes.byref(b)))
    return b.value


def q1_sign_pack(w_bits, w_scales, N: int, K: int, w_packed):
    """One-time repack of sign words + scales (uint8 [q1_sign_packed_bytes])."""
    import torch
    G = K // 32 if K % 32 == 0 else None
    _check(_lib.q1_sign_pack(_dev(w_bits, torch.int32, N * G if G else None, "w_bits"),
                             _dev(w_scales, torch.float32, N * G if G else None, "w_scales"), N, K,
                             _dev(w_packed, torch.uint8, q1_sign_packed_bytes(N, K) if G else None, "w_packed"),
                             _stream()))


def q1_sign_gemm_packed(x, w_packed, y, M: int, N: int, K: int, workspace=None):
    import torch
    if workspace is None:
        workspace = _sign_workspace(M, N, K, x.device)
    _check(_lib.q1_sign_gemm_packed(_dev(x, torch.float32, M * K, "x"),
                                    _dev(w_packed, torch.uint8, None, "w_packed"),
                                    _dev(y, torch.float32, M * N, "y"), M, N, K,
                                    _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()))


def q1_sign_gemv(x, w_packed, y, M: int, N: int, K: int):
    import torch
    _check(_lib.q1_sign_gemv(_dev(x, torch.float32, M * K, "x"), _dev(w_packed, torch.uint8, None, "w_packed"),
                             _dev(y, torch.float32, M * N, "y"), M, N, K, _stream()))


def q1_sign_gemm_lut4(x, w_packed, y, M: int, N: int, K: int):
    import torch
    _check(_lib.q1_sign_gemm_lut4(_dev(x, torch.float32, M * K, "x"), _dev(w_packed, torch.uint8, None, "w_packed"),
                                  _dev(y, torch.float32, M * N, "y"), M, N, K, _stream()))


# ------------------------------------------------------ block-Q8 matmul_nt

def blockq8_matmul_nt(x, quants, scales, y, m: int, k: int, n: int):
    import torch
    _check(_lib.blockq8_matmul_nt(_dev(x, torch.float32, m * k, "x"),
                                  _dev(quants, torch.int32, n * k // 4 if k % 4 == 0 else None, "quants"),
                                  _dev(scales, torch.float32, n * (k // 32) if k % 32 == 0 else None, "scales"),
                                  _dev(y, torch.float32, m * n, "y"), m, k, n, _stream()))


# ----------------------------------------------------------------- ternary

def ternary_act_bitplanes(x_q, count: int, K: int, planes):
    import torch
    _check(_lib.ternary_act_bitplanes(_dev(x_q, torch.int8, count * K, "x_q"), count, K,
                                      _dev(planes, torch.int32, count * 8 * (K // 32) if K % 32 == 0 else None,
                                           "planes"), _stream()))


def ternary_gemv(w_pos, w_neg, w_scale: float, x_planes, x_scale: float, y, dot_out, rows: int, K: int):
    import torch
    W = K // 32 if K % 32 == 0 else None
    dp = None if dot_out is None else _dev(dot_out, torch.int32, rows, "dot_out")
    _check(_lib.ternary_gemv(_dev(w_pos, torch.int32, rows * W if W else None, "w_pos"),
                             _dev(w_neg, torch.int32, rows * W if W else None, "w_neg"), float(w_scale),
                             _dev(x_planes, torch.int32, 8 * W if W else None, "x_planes"), float(x_scale),
                             _dev(y, torch.float32, rows, "y"), dp, rows, K, _stream()))


def make_ternary_problems(entries, device="cuda"):
    """Device array of gd_ternary_problem from
    [(w_pos, w_neg, x_planes, y, dot_out_or_None, w_scale, x_scale), ...];
    x_scale is a float, or a one-element device f32 tensor (x_scale_dev)."""
    import torch
    arr = (TernaryProblem * len(entries))()
    for i, (p, n, xp, y, d, ws, xs) in enumerate(entries):
        if isinstance(xs, torch.Tensor):
            xs_val, xs_dev = 0.0, _dev(xs, torch.float32, None, "x_scale")
        else:
            xs_val, xs_dev = float(xs), None
        arr[i] = TernaryProblem(p.data_ptr(), n.data_ptr(), xp.data_ptr(), y.data_ptr(),
                                None if d is None else d.data_ptr(), float(ws), xs_val, xs_dev)
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device)


def ternary_gemv_grouped(problems, count: int, rows: int, K: int):
    import torch
    _check(_lib.ternary_gemv_grouped(
        _dev(problems, torch.uint8, count * ctypes.sizeof(TernaryProblem), "problems"), count, rows, K, _stream()))


# ------------------------------------------------- activation quantization

def q8_0_quantize(x, a_q8, n: int, K: int):
    """f32 x [n, K] -> q8_0 blocks (uint8 [n * K/32 * 34]), on the device."""
    import torch
    _check(_lib.q8_0_quantize(_dev(x, torch.float32, n * K, "x"),
                              _dev(a_q8, torch.uint8, n * (K // 32) * 34 if K % 32 == 0 else None, "a_q8"),
                              n, K, _stream()))


def ternary_quantize_act(x, count: int, K: int, planes, x_scale):
    """f32 x [count, K] -> int8 bit planes (int32 [count * 8 * K/32]) and
    scales (f32 [count]), on the device."""
    import torch
    _check(_lib.ternary_quantize_act(_dev(x, torch.float32, count * K, "x"), count, K,
                                     _dev(planes, torch.int32, count * 8 * (K // 32) if K % 32 == 0 else None,
                                          "planes"),
                                     _dev(x_scale, torch.float32, count, "x_scale"), _stream()))


# ------------------------------------------------------ decode attention

def attn_decode_workspace_bytes(n_heads: int, n_kv_heads: int, head_dim: int, kv_len: int,
                                num_splits: int = 0) -> int:
    b = ctypes.c_size_t()
    _check(_lib.attn_decode_workspace_bytes(n_heads, n_kv_heads, head_dim, kv_len, num_splits, ctypes.byref(b)))
    return b.value


def attn_decode_splitk(q, k_cache, v_cache, out, n_heads: int, n_kv_heads: int, head_dim: int, kv_len: int,
                       kv_stride: int, scale: float, num_splits: int = 0, workspace=None):
    """Split-K decode attention for one token; the workspace (uint8) is
    allocated here when not given."""
    import torch
    need = attn_decode_workspace_bytes(n_heads, n_kv_heads, head_dim, kv_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cache_n = n_kv_heads * kv_stride * head_dim
    _check(_lib.attn_decode_splitk(_dev(q, torch.float32, n_heads * head_dim, "q"),
                                   _dev(k_cache, torch.float32, cache_n, "k_cache"),
                                   _dev(v_cache, torch.float32, cache_n, "v_cache"),
                                   _dev(out, torch.float32, n_heads * head_dim, "out"),
                                   n_heads, n_kv_heads, head_dim, kv_len, kv_stride, float(scale), num_splits,
                                   _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream()))


def attn_decode_splitk_noalloc(q, k_cache, v_cache, out, n_heads: int, n_kv_heads: int, head_dim: int,
                               kv_len: int, kv_stride: int, scale: float, num_splits: int = 0):
    """attn_decode_splitk with the split partials in the library's own
    scratch (no workspace, nothing allocated; calls that overlap on one
    device race)."""
    import torch
    cache_n = n_kv_heads * kv_stride * head_dim
    _check(_lib.attn_decode_splitk_noalloc(_dev(q, torch.float32, n_heads * head_dim, "q"),
                                           _dev(k_cache, torch.float32, cache_n, "k_cache"),
                                           _dev(v_cache, torch.float32, cache_n, "v_cache"),
                                           _dev(out, torch.float32, n_heads * head_dim, "out"),
                                           n_heads, n_kv_heads, head_dim, kv_len, kv_stride, float(scale),
                                           num_splits, _stream()))


# ------------------------------------------------------------ measurement

def gemm_decode_fill(buf, seed: int = 1):
    import torch
    _check(_lib.gemm_decode_fill(_dev(buf, torch.uint8, None, "buf"), buf.numel(), seed, _stream()))


def gemm_decode_stream_read(buf, passes: int, sink):
    import torch
    _check(_lib.gemm_decode_stream_read(_dev(buf, torch.uint8, None, "buf"), buf.numel(), passes,
                                        _dev(sink, torch.int32, None, "sink"), sink.numel(), _stream()))
