"""The CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. It wraps ``oracle.c`` (plain C, built with gcc
``-O2 -ffp-contract=off -fno-fast-math``) through ctypes and numpy; it shares
no code with the HIP library and never imports it.

Functions take and return numpy arrays in the pages' wire formats (see
``workloads``). Parity pins: ``tests/test_oracle_*.py``. The C header comment
of ``oracle.c`` cites the passage each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra"]


SANITIZE_CFLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc; CPU only). With sanitize, an
    ASan + UBSan build into liboracle_san.so, which lib() loads when
    GD_ORACLE_SANITIZED=1 (in a process that preloads gcc's libasan)."""
    out = _LIB_SAN if sanitize else _LIB
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SANITIZE_CFLAGS if sanitize else []), _SRC, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if os.environ.get("GD_ORACLE_SANITIZED") == "1":
            if not os.path.exists(_LIB_SAN):
                build(sanitize=True)
            _lib = ctypes.CDLL(_LIB_SAN)
        else:
            if not os.path.exists(_LIB):
                build()
            _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F32 = ctypes.c_float


def _declare(L):
    L.gdo_max_threads.restype = _INT
    L.gdo_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.gdo_f16_to_f32.restype = _F32
    L.gdo_q1_q8_gemv_aos.argtypes = [_P, _P, _P, _I64, _I64, _I64, _INT]
    L.gdo_pack_q1_p1.argtypes = [_P, _I64, _I64, _P, _P]
    L.gdo_pack_q8_p1.argtypes = [_P, _I64, _I64, _P, _P]
    L.gdo_q1_q8_gemv_p1packed.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT]
    L.gdo_sign_gemm_f64.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _INT]
    L.gdo_sign_gemm_f32.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _INT]
    L.gdo_blockq8_f32.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _INT]
    L.gdo_ternary_dot_direct.argtypes = [_P, _P, _P, _P, _I64, _I64]
    L.gdo_ternary_gemv.argtypes = [_P, _P, _F32, _P, _F32, _P, _P, _I64, _I64, _INT]
    L.gdo_quantize_absmax_int8.argtypes = [_P, _I64, _I64, _P, _P]
    L.gdo_f32_to_f16.argtypes = [_F32]
    L.gdo_f32_to_f16.restype = ctypes.c_uint16
    L.gdo_quantize_q8_0.argtypes = [_P, _I64, _I64, _P]
    for name in ("gdo_q1_q8_gemv_aos", "gdo_pack_q1_p1", "gdo_pack_q8_p1",
                 "gdo_q1_q8_gemv_p1packed", "gdo_sign_gemm_f64",
                 "gdo_sign_gemm_f32", "gdo_blockq8_f32", "gdo_ternary_dot_direct",
                 "gdo_ternary_gemv", "gdo_quantize_absmax_int8", "gdo_quantize_q8_0"):
        getattr(L, name).restype = None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def max_threads() -> int:
    return int(lib().gdo_max_threads())


def f16_to_f32(h: int) -> np.float32:
    return np.float32(lib().gdo_f16_to_f32(int(h) & 0xFFFF))


# ----------------------------------------------------------------- Q1_0.q8_0

def q1_q8_gemv_aos(w_aos, a_aos, rows: int, K: int, n_act: int = 1, nthreads: int = 1):
    """F1: y f32 [n_act, rows] from AoS weight bytes and AoS activation bytes."""
    w, wp = _c(w_aos, np.uint8)
    a, ap = _c(a_aos, np.uint8)
    _check_q1(w, a, rows, K, n_act)
    y = np.empty((n_act, rows), dtype=np.float32)
    lib().gdo_q1_q8_gemv_aos(wp, ap, y.ctypes.data, rows, K, n_act, nthreads)
    return y


def pack_q1_p1(w_aos, rows: int, K: int):
    w, wp = _c(w_aos, np.uint8)
    nb = K // 128
    d = np.empty(rows * nb, dtype=np.float32)
    b = np.empty(rows * nb * 4, dtype=np.uint32)
    lib().gdo_pack_q1_p1(wp, rows, K, d.ctypes.data, b.ctypes.data)
    return d, b


def pack_q8_p1(a_aos, n_act: int, K: int):
    a, ap = _c(a_aos, np.uint8)
    nb8 = K // 32
    d = np.empty(n_act * nb8, dtype=np.float32)
    q = np.empty(n_act * nb8 * 8, dtype=np.uint32)
    lib().gdo_pack_q8_p1(ap, n_act, K, d.ctypes.data, q.ctypes.data)
    return d, q


def q1_q8_gemv_p1packed(w_aos, a_aos, rows: int, K: int, n_act: int = 1, nthreads: int = 1):
    """F2: P1's packQ1/packQ8 layouts, one chain per (row, lane)."""
    wd, wb = pack_q1_p1(w_aos, rows, K)
    ad, aq = pack_q8_p1(a_aos, n_act, K)
    y = np.empty((n_act, rows), dtype=np.float32)
    lib().gdo_q1_q8_gemv_p1packed(wd.ctypes.data, wb.ctypes.data, ad.ctypes.data,
                                  aq.ctypes.data, y.ctypes.data, rows, K, n_act, nthreads)
    return y


def _check_q1(w, a, rows, K, n_act):
    if K % 128 or rows < 0 or n_act < 1:
        raise ValueError("bad Q1 shape")
    if w.size != rows * (K // 128) * 18:
        raise ValueError("weight bytes do not match rows x K")
    if a.size != n_act * (K // 32) * 34:
        raise ValueError("activation bytes do not match n_act x K")


# ------------------------------------------------------------ sign-bit GEMM

def sign_gemm_f64(x, bits, scales, nthreads: int = 1):
    x, xp = _c(x, np.float32)
    bits, bp = _c(bits, np.uint32)
    scales, sp = _c(scales, np.float32)
    M, K = x.shape
    N = bits.shape[0]
    if bits.shape != (N, K // 32) or scales.shape != (N, K // 32) or K % 32:
        raise ValueError("bad sign GEMM shapes")
    y = np.empty((M, N), dtype=np.float32)
    lib().gdo_sign_gemm_f64(xp, bp, sp, y.ctypes.data, M, N, K, nthreads)
    return y


def sign_gemm_f32(x, bits, scales, nthreads: int = 1):
    x, xp = _c(x, np.float32)
    bits, bp = _c(bits, np.uint32)
    scales, sp = _c(scales, np.float32)
    M, K = x.shape
    N = bits.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    lib().gdo_sign_gemm_f32(xp, bp, sp, y.ctypes.data, M, N, K, nthreads)
    return y


# ----------------------------------------------------------- block-Q8 nt

def blockq8_f32(x, quants, scales, nthreads: int = 1):
    x, xp = _c(x, np.float32)
    quants, qp = _c(quants, np.uint32)
    scales, sp = _c(scales, np.float32)
    m, k = x.shape
    n = quants.shape[0]
    if quants.shape != (n, k // 4) or scales.shape != (n, k // 32) or k % 32:
        raise ValueError("bad block-Q8 shapes")
    y = np.empty((m, n), dtype=np.float32)
    lib().gdo_blockq8_f32(xp, qp, sp, y.ctypes.data, m, k, n, nthreads)
    return y


# ------------------------------------------------------------------ ternary

def ternary_dot_direct(P, N, x_q):
    P, pp = _c(P, np.uint32)
    N, np_ = _c(N, np.uint32)
    x, xp = _c(x_q, np.int8)
    rows, W = P.shape
    K = W * 32
    dot = np.empty(rows, dtype=np.int64)
    lib().gdo_ternary_dot_direct(pp, np_, xp, dot.ctypes.data, rows, K)
    return dot


def ternary_gemv(P, N, w_scale, x_q, x_scale, nthreads: int = 1):
    """T2 (popcount identity): returns (y f32 [rows], dot int32 [rows])."""
    P, pp = _c(P, np.uint32)
    N, np_ = _c(N, np.uint32)
    x, xp = _c(x_q, np.int8)
    rows, W = P.shape
    K = W * 32
    if N.shape != P.shape or x.size != K:
        raise ValueError("bad ternary shapes")
    y = np.empty(rows, dtype=np.float32)
    dot = np.empty(rows, dtype=np.int32)
    lib().gdo_ternary_gemv(pp, np_, float(w_scale), xp, float(x_scale), y.ctypes.data,
                           dot.ctypes.data, rows, K, nthreads)
    return y, dot


# -------------------------------------------------------- activation quantization

def quantize_absmax_int8(x):
    """Per-row absmax int8 codes (Math.round of x * 127/absmax in f64, ties
    toward +inf, clamped to [-127, 127]) and f32 scales absmax/127.
    x f32 [M, K] (or [K]); returns (codes int8 same shape, scales f32 [M])."""
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    x2, xp = _c(x.reshape(-1, shape[-1]) if x.ndim else x.reshape(1, 1), np.float32)
    M, K = x2.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().gdo_quantize_absmax_int8(xp, M, K, q.ctypes.data, s.ctypes.data)
    return q.reshape(shape), s


def f32_to_f16_bits(v) -> int:
    """IEEE binary16 bits of f32 v, rounded to nearest even."""
    return int(lib().gdo_f32_to_f16(float(np.float32(v))))


def quantize_q8_0(x):
    """q8_0 AoS bytes [n * K/32 * 34] from f32 x [n, K] (or [K]): per block of
    32, codes as quantize_absmax_int8 does per row, d = f16(f32(absmax/127))."""
    x = np.asarray(x, dtype=np.float32)
    x2, xp = _c(x.reshape(-1, x.shape[-1]), np.float32)
    n, K = x2.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    out = np.empty(n * (K // 32) * 34, dtype=np.uint8)
    lib().gdo_quantize_q8_0(xp, n, K, out.ctypes.data)
    return out


# ------------------------------------------------------------ decode attention

def attention_decode(q, k, v, scale: float):
    """One decode token's attention, the plain f64 definition the split-K
    kernels reach up to rounding ("BonsaiのWebGPUカーネルを読み解く", section on
    split-K flash decode attention): for query head h, with KV head
    kv = h // (Hq / Hkv), s_j = scale * q[h] . k[kv, j], and
    out[h] = sum_j exp(s_j - max s) v[kv, j] / sum_j exp(s_j - max s).
    q [Hq, D]; k, v [Hkv, L, D] (f32 or f64); returns f64 [Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, D = q.shape
    Hkv, L, Dk = k.shape
    if Dk != D or v.shape != k.shape or Hq % Hkv or L < 1:
        raise ValueError("bad attention shapes")
    G = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // G
        s = float(scale) * (k[kv] @ q[h])
        p = np.exp(s - np.max(s))
        out[h] = (p @ v[kv]) / np.sum(p)
    return out
