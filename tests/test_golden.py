"""The oracle and the input generators against the values the pages print
(tests/golden/page_constants.txt, each line cited there)."""
import os

import numpy as np

import oracle
import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    out = {}
    with open(os.path.join(HERE, "golden", "page_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                name, value = line.split()
                out[name] = float(value) if ("." in value or "e-" in value) else int(value, 0)
    return out


G = golden()


def test_block_sizes_of_the_generated_wire_formats():
    """An AoS weight row of K elements is K/QK1_0 blocks of Q1_0_BYTES; an
    activation vector K/QK8_0 blocks of Q8_0_BYTES."""
    rows, K = 3, 512
    W = wl.q1_weights_aos(rows, K, seed=0)
    A = wl.q8_acts_aos(K, 1)
    assert W.size == rows * (K // G["QK1_0"]) * G["Q1_0_BYTES"]
    assert A.size == (K // G["QK8_0"]) * G["Q8_0_BYTES"]


def test_f16_subnormal_decode():
    """The oracle's f16 decode gives m x 2^-24 for a subnormal, the factor the
    page writes out, with the sign bit honoured."""
    unit = np.float32(G["F16_SUBNORMAL_UNIT"])
    assert unit == np.float32(2.0 ** -24)
    for m in (1, 2, 3, 0x155, 0x3FF):
        assert oracle.f16_to_f32(m) == np.float32(m) * unit
        assert oracle.f16_to_f32(0x8000 | m) == -(np.float32(m) * unit)


def test_mulberry32_state_step():
    """The generator's state advances by the page's increment: two generators
    whose seeds differ by it produce sequences offset by one draw."""
    inc = G["MULBERRY32_INCREMENT"]
    a = wl.Mulberry32(12345)
    b = wl.Mulberry32((12345 + inc) & 0xFFFFFFFF)
    xs = [a() for _ in range(6)]
    ys = [b() for _ in range(5)]
    assert xs[1:] == ys


def test_quantize_code_range():
    """Codes lie in the page's symmetric range, and each token's largest |x|
    reaches its end."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 256)) * np.array([[1e-3], [1.0], [7.0], [1e3], [1e6]])).astype(np.float32)
    q, s = oracle.quantize_absmax_int8(x)
    assert q.min() >= G["QUANT_CODE_MIN"] and q.max() <= G["QUANT_CODE_MAX"]
    for r in range(5):
        i = int(np.argmax(np.abs(x[r])))
        assert abs(int(q[r, i])) == G["QUANT_CODE_MAX"]
