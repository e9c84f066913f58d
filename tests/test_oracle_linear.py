"""Pins for the bias oracle (oracle/linear.py).

add_bias_bf16 is checked against (a) the single nearest-even rounding of the exact rational sum,
computed with Python fractions, (b) torch's own CPU bf16 addition (an independent implementation
of the operation the pages call), and (c) hand-worked values in tests/golden/bias_bf16.txt.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import linear as L


def _bits_to_fraction(b: int) -> Fraction:
    return Fraction(float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0]))


def _fraction_to_bf16_bits(v: Fraction, a_bits: int, b_bits: int) -> int:
    if v == 0:   # IEEE: the sum of two zeros keeps a common sign; x + (-x) is +0 under nearest even
        both_neg = (a_bits & 0x8000) and (b_bits & 0x8000)
        return 0x8000 if both_neg else 0x0000
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = float(n * ulp)
    bits = int(np.array([r], dtype=np.float32).view(np.uint32)[0]) >> 16
    return sign | bits


def _edge_and_random_pairs(n_random=4000, seed=7):
    rng = np.random.default_rng(seed)
    vals = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x3F81, 0x3B80, 0x3B81,
            0x4E80, 0x7F7F >> 1, 0x4B00, 0xC700, 0x3400, 0x00FF]
    pairs = [(a, b) for a in vals for b in vals]
    # random finite bf16 with exponents kept away from overflow
    exp = rng.integers(1, 230, size=(n_random, 2))
    man = rng.integers(0, 128, size=(n_random, 2))
    sgn = rng.integers(0, 2, size=(n_random, 2))
    bits = (sgn << 15) | (exp << 7) | man
    # also pairs with close exponents (cancellation) and wide gaps
    bits[: n_random // 4, 1] = (bits[: n_random // 4, 0] ^ 0x8000) + rng.integers(-3, 4, size=n_random // 4)
    pairs += [(int(a) & 0xFFFF, int(b) & 0xFFFF) for a, b in bits]
    return [(a, b) for a, b in pairs if (a & 0x7F80) != 0x7F80 and (b & 0x7F80) != 0x7F80]


def test_add_bias_bf16_is_the_rounding_of_the_exact_sum():
    pairs = _edge_and_random_pairs()
    a = np.array([p[0] for p in pairs], dtype=np.uint16)
    b = np.array([p[1] for p in pairs], dtype=np.uint16)
    got = L.add_bias_bf16(a, b)
    for i, (x, y) in enumerate(pairs):
        want = _fraction_to_bf16_bits(_bits_to_fraction(x) + _bits_to_fraction(y), x, y)
        assert int(got[i]) == want, (hex(x), hex(y), hex(int(got[i])), hex(want))


def test_add_bias_bf16_matches_torch_cpu_bf16_add():
    pairs = _edge_and_random_pairs(n_random=50000, seed=11)
    a = np.array([p[0] for p in pairs], dtype=np.uint16)
    b = np.array([p[1] for p in pairs], dtype=np.uint16)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    want = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(L.add_bias_bf16(a, b), want)


def test_add_bias_bf16_broadcasts_over_rows_and_golden_values():
    # golden: tests/golden/bias_bf16.txt, "out bias -> sum" in bf16 hex, worked by hand
    rows = []
    with open("tests/golden/bias_bf16.txt") as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                o, bb, s = line.replace("->", " ").split()
                rows.append((int(o, 16), int(bb, 16), int(s, 16)))
    assert len(rows) >= 6
    for o, bb, s in rows:
        assert int(L.add_bias_bf16(np.array([o], np.uint16), np.array([bb], np.uint16))[0]) == s
    out = np.array([[0x3F80, 0x4000], [0xBF80, 0x0000]], dtype=np.uint16)
    bias = np.array([0x3F80, 0xC000], dtype=np.uint16)
    assert L.add_bias_bf16(out, bias).tolist() == [[0x4000, 0x0000], [0x0000, 0xC000]]


def test_gemm_plus_bias_adds_the_fp32_bias_per_column():
    c = np.array([[1.0, 2.5], [-3.0, 0.0]])
    bias = np.array([0.1, -2.5], dtype=np.float32)    # 0.1 as fp32, not as fp64
    got = L.gemm_plus_bias(c, bias)
    assert got[0, 0] == 1.0 + float(np.float32(0.1)) and got[0, 0] != 1.1
    assert got[0, 1] == 0.0 and got[1, 1] == -2.5 and got[1, 0] == -3.0 + float(np.float32(0.1))
