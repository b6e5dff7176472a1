"""Seeded synthetic inputs for the block-quantized GEMV/GEMM paths.

This module is shared by the tests, the oracle-side checks and the benchmark.
It only *draws and lays out* inputs (bytes in the pages' wire formats); it
holds none of the arithmetic of the products themselves, and it imports
neither the oracle nor the HIP package.

Wire formats produced here (as the pages define them):

* Q1_0 weight block, 18 bytes: f16 scale d0 (little-endian) then 128 sign
  bits, element j in byte 2 + j//8, bit j%8; bit 1 means +d0, bit 0 means -d0
  ("browseml-gpu.js", header comment and ``Q1_DOT_WGSL``).
* q8_0 activation block, 34 bytes: f16 scale d1 then 32 int8 quants; four
  q8_0 blocks cover one Q1_0 block ("browseml-gpu.js", header comment).
* Packed sign bits: one u32 holds the sign bits of 32 consecutive weights,
  LSB first, bit 1 -> +1, bit 0 -> -1, with one scale per 32 weights
  ("BonsaiのWebGPUカーネルを読み解く", figure on the decode/prefill kernels).
* Block-scaled int8: quants packed four per u32, element t in byte t%4 of
  word t//4, scales [n, k/32] f32 ("block_q8_matmul_nt.wgsl", PACKING).
* Ternary P/N bitplanes: P bit set where w=+1, N bit set where w=-1
  ("BonsaiのWebGPUカーネルを読み解く", section on Bonsai), stored here as
  u32 [rows, K/32] with element 32m+j at bit j of word m.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q1_0_BYTES = 18
Q8_0_BYTES = 34
QK1_0 = 128
QK8_0 = 32


# ---------------------------------------------------------------------------
# The page's reproducible test case ("browseml-gpu.js": its small generator,
# a finite-f16 helper and randomCase), regenerated draw for draw so that the
# page's own shapes and seeds give the page's bytes.
# ---------------------------------------------------------------------------

_M32 = 0xFFFFFFFF


class Mulberry32:
    """Tommy Ettinger's mulberry32: a 32-bit state advanced by the Weyl
    constant 0x6D2B79F5 at every draw; the output is the new state put
    through two rounds of xor-shift-and-multiply (shift 15 with multiplier
    state|1, then shift 7 with multiplier |61, added back) and a final
    xor-shift by 14, read as a fraction of 2^32 in [0, 1)."""

    WEYL = 0x6D2B79F5

    def __init__(self, seed: int):
        self.state = seed & _M32

    def next_u32(self) -> int:
        self.state = (self.state + self.WEYL) & _M32
        z = self.state
        z = ((z ^ (z >> 15)) * (z | 1)) & _M32
        z = (z ^ ((z + ((z ^ (z >> 7)) * (z | 61))) & _M32)) & _M32
        return z ^ (z >> 14)

    def __call__(self) -> float:
        return self.next_u32() / 4294967296.0


def f16bits(r: Mulberry32, lo: int = 3, hi: int = 17) -> int:
    """A finite f16 bit pattern with a random sign, an exponent field drawn
    in [lo, hi) and a random 10-bit mantissa, drawn in that order."""
    negative = r() < 0.5
    exponent = lo + int(r() * (hi - lo))
    mantissa = int(r() * 1024)
    return (0x8000 if negative else 0) | (exponent << 10) | mantissa


def _q1_block(r: Mulberry32) -> bytes:
    """An 18-byte Q1_0 block: a random f16 scale, then 16 random bytes of
    sign bits."""
    scale = f16bits(r)
    return scale.to_bytes(2, "little") + bytes(int(r() * 256) for _ in range(16))


def _q8_block(r: Mulberry32) -> bytes:
    """A 34-byte q8_0 block: a random f16 scale, then 32 quant bytes, each
    0x80 (int8 -128) with probability 0.02 and otherwise a random byte (one
    draw decides, a second draw gives the byte)."""
    scale = f16bits(r)
    quants = bytes(0x80 if r() < 0.02 else int(r() * 256) for _ in range(32))
    return scale.to_bytes(2, "little") + quants


def random_case(rows: int, n: int, seed: int = 1):
    """P1's ``randomCase``: Q1_0 weights of rows x n and one q8_0 vector of
    n, drawn from one generator seeded with `seed`: every weight block in
    row-major order, then every activation block. About 2% of the quant
    bytes are -128. Returns (W bytes [rows*nb*18], A bytes [n/32*34])."""
    if n % QK1_0:
        raise ValueError("n must be a multiple of 128")
    r = Mulberry32(seed)
    W = b"".join(_q1_block(r) for _ in range(rows * (n // QK1_0)))
    A = b"".join(_q8_block(r) for _ in range(n // QK8_0))
    return np.frombuffer(W, dtype=np.uint8).copy(), np.frombuffer(A, dtype=np.uint8).copy()


# ---------------------------------------------------------------------------
# Config-shaped generators (numpy PCG64, ``default_rng(seed)``).
# ---------------------------------------------------------------------------

def q1_weights_aos(rows: int, K: int, seed: int, scale_sigma: float = 0.02) -> np.ndarray:
    """Q1_0 weights as AoS bytes [rows, K/128, 18].

    Draw order: d0 = f16(|N(0, sigma)|) for all blocks (row-major), then 16
    uniform random bytes of sign bits per block."""
    if K % QK1_0 or rows < 0:
        raise ValueError("K must be a multiple of 128")
    nb = K // QK1_0
    rng = np.random.default_rng(seed)
    d0 = np.abs(rng.normal(0.0, scale_sigma, size=(rows, nb))).astype(np.float16)
    bits = rng.integers(0, 256, size=(rows, nb, 16), dtype=np.uint8)
    out = np.empty((rows, nb, Q1_0_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d0.view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = bits
    return out


def q8_acts_aos(K: int, seed: int, n_act: int = 1,
                d_lo: float = 0.001, d_hi: float = 0.05) -> np.ndarray:
    """q8_0 activations as AoS bytes [n_act, K/32, 34].

    Draw order: d1 = f16(U(d_lo, d_hi)) for all blocks, then int8 quants
    uniform on [-127, 127]."""
    if K % QK8_0:
        raise ValueError("K must be a multiple of 32")
    nb32 = K // QK8_0
    rng = np.random.default_rng(seed)
    d1 = rng.uniform(d_lo, d_hi, size=(n_act, nb32)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n_act, nb32, 32), dtype=np.int64).astype(np.int8)
    out = np.empty((n_act, nb32, Q8_0_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d1.view(np.uint8).reshape(n_act, nb32, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out


def pack_bits_lsb(bits01: np.ndarray) -> np.ndarray:
    """Pack a [..., 32*m] array of 0/1 into u32 [..., m], element 32w+j at bit j."""
    b = np.asarray(bits01, dtype=np.uint8)
    if b.shape[-1] % 32:
        raise ValueError("last axis must be a multiple of 32")
    by = np.packbits(b, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4")


def sign_gemm_inputs(M: int, N: int, K: int, seed: int):
    """Sign-bit prefill GEMM inputs: x f32 N(0,1) [M,K]; bits u32 uniform
    [N,K/32]; scales f32 |N(0,0.02)| [N,K/32]. Draw order: x, bits, scales."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(M, K), dtype=np.float64).astype(np.float32)
    bits = rng.integers(0, 2**32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    scales = np.abs(rng.normal(0.0, 0.02, size=(N, K // 32))).astype(np.float32)
    return x, bits, scales


def blockq8_inputs(m: int, k: int, n: int, seed: int):
    """Block-Q8 matmul_nt inputs: x f32 N(0,1) [m,k]; quants int8 uniform on
    [-128,127] packed four per u32 LE as [n, k/4]; scales f32 U(1e-3,1e-2)
    [n, k/32]. Draw order: quants, scales, x."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    rng = np.random.default_rng(seed)
    q = rng.integers(-128, 128, size=(n, k), dtype=np.int64).astype(np.int8)
    scales = rng.uniform(1e-3, 1e-2, size=(n, k // 32)).astype(np.float32)
    x = rng.standard_normal(size=(m, k), dtype=np.float64).astype(np.float32)
    quants = np.ascontiguousarray(q).view("<u4").reshape(n, k // 4)
    return x, quants, scales


def absmax_int8(x: np.ndarray):
    """Input recipe for the int8 activation vector of the ternary path: one
    scale per token, codes clamp(round(x * (127/absmax)), -127, 127) with the
    reciprocal 127/absmax formed in f64 and ties rounded toward +infinity
    (the conventions "web-xpu-ops" states for its quantize op and q4 format).
    Returns (codes int8, scale f32 = absmax/127)."""
    x64 = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x64))) if x64.size else 0.0
    if amax == 0.0:
        return np.zeros(x64.shape, dtype=np.int8), np.float32(0.0)
    inv = 127.0 / amax
    v = x64 * inv
    q = np.floor(v) + ((v - np.floor(v)) >= 0.5)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, np.float32(amax / 127.0)


def ternary_inputs(rows: int, K: int, seed: int):
    """Ternary GEMV inputs: w uniform on {-1,0,+1} (p=1/3 each) stored as P/N
    bitplanes u32 [rows, K/32]; w_scale f32 U(0.01, 0.1); x f32 N(0,1) [K]
    turned into int8 codes + one f32 scale by ``absmax_int8``.
    Draw order: w, w_scale, x. Returns (P, N, w_scale, x_q, x_scale)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    w = rng.integers(-1, 2, size=(rows, K), dtype=np.int64)
    w_scale = np.float32(rng.uniform(0.01, 0.1))
    x = rng.standard_normal(size=K, dtype=np.float64)
    P = pack_bits_lsb((w == 1).astype(np.uint8))
    N = pack_bits_lsb((w == -1).astype(np.uint8))
    x_q, x_scale = absmax_int8(x)
    return P, N, w_scale, x_q, x_scale


# ---------------------------------------------------------------------------
# The five workloads (shapes, seeds) the library is exercised and timed on.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Q1Workload:
    rows: int
    K: int
    weight_seed: int
    act_seeds: tuple


#: Q1_0.q8_0 GEMV, rows=256, K=1024, batch 1 (correctness-sized).
Q1_SMALL = Q1Workload(rows=256, K=1024, weight_seed=0, act_seeds=(100,))
#: Q1_0.q8_0 GEMV at 8B-class decode shapes, 32 activation vectors each.
Q1_DECODE = (
    Q1Workload(rows=4096, K=4096, weight_seed=1, act_seeds=tuple(range(1000, 1032))),
    Q1Workload(rows=14336, K=4096, weight_seed=2, act_seeds=tuple(range(1000, 1032))),
)
#: Sign-bit prefill GEMM y = x @ w^T, M=512 tokens, N=4096, K=4096.
SIGN_PREFILL = dict(M=512, N=4096, K=4096, seed=2)
#: Block-Q8 matmul_nt, k=960, n=49152, m in {1, 16}.
BLOCKQ8_LMHEAD = dict(k=960, n=49152, ms=(1, 16), seed=3)


def bitnet_step_shapes(layers: int = 30):
    """(rows, K) of the 210 ternary GEMVs of one BitNet-2B-like decode step:
    per layer four 2560x2560, two 6912x2560 and one 2560x6912."""
    per_layer = [(2560, 2560)] * 4 + [(6912, 2560)] * 2 + [(2560, 6912)]
    return [s for _ in range(layers) for s in per_layer]


TERNARY_SEED_BASE = 4000
