"""Pins for the oracle's codecs: hand-written tables, tie cases and library cross-checks."""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.conftest import golden_lines


def _f32(s):
    return np.float32(float(s))


def test_e2m1_grid_matches_definition_table():
    table = F.e2m1_decode_table()
    rows = [l.split() for l in golden_lines("e2m1_grid.txt")]
    assert len(rows) == 16
    for code, val in rows:
        got = table[int(code)]
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e2m1_rne_cases():
    for inp, code in (l.split() for l in golden_lines("e2m1_rne_cases.txt")):
        got = int(F.e2m1_encode(np.array([_f32(inp)]))[0])
        assert got == int(code), (inp, got, code)


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(codes).astype(np.float32)), codes)


def test_e2m1_encode_is_nearest_by_brute_force():
    # every fp32 value in a dense sweep maps to a grid point no farther than any other point
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-70, 71) / 10.0]).astype(np.float32)
    q = F.e2m1_encode(v)
    dec = F.e2m1_decode(q)
    grid = F.e2m1_decode_table()
    for x, d in zip(v.astype(np.float64), dec):
        if abs(x) >= 6:
            assert abs(d) == 6 and np.sign(d) == np.sign(x)
            continue
        best = np.min(np.abs(grid - x))
        assert abs(d - x) == best


def test_e4m3_decode_matches_torch_float8_view():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert got[0x7E] == F.E4M3_MAX == float(torch.finfo(torch.float8_e4m3fn).max)


def test_e4m3_cases():
    table = F.e4m3_decode_table()
    for parts in (l.split() for l in golden_lines("e4m3_cases.txt")):
        if parts[0] == "decode":
            code, val = int(parts[1], 16), parts[2]
            if val == "nan":
                assert np.isnan(table[code])
            else:
                assert table[code] == float(val)
                assert np.signbit(table[code]) == val.startswith("-")
        else:
            got = int(F.e4m3_encode(np.array([_f32(parts[1])]))[0])
            assert got == int(parts[2], 16), (parts, hex(got))


def test_e4m3_encode_matches_torch_cast_after_clamp():
    # torch's float8_e4m3fn cast rounds to nearest even but does not saturate; clamping to
    # +-448 first makes it a library special case of the saturating encoder.
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(50000) * 10.0 ** rng.uniform(-5, 3, 50000),
        (np.arange(-2000, 2000) / 7.3),
        [0.0, -0.0, 1e-12, -1e-12, 447.9, 448.0, 465.0, -479.0, 1e9],
    ]).astype(np.float32)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v)
    assert np.array_equal(got, ref)


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes).astype(np.float32)), codes)


def test_e8m0_decode_closed_form_and_torch_view():
    c = np.arange(256)
    got = F.e8m0_decode(c)
    assert np.isnan(got[255])
    for k in range(255):
        assert got[k] == 2.0 ** (k - 127)
    if hasattr(torch, "float8_e8m0fnu"):
        ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        assert np.array_equal(ref[:255], got[:255])
        assert np.isnan(ref[255])


@pytest.mark.parametrize("v", [0.0, -0.0])
def test_zero_sign_is_kept(v):
    assert int(F.e2m1_encode(np.array([v], np.float32))[0]) == (8 if math.copysign(1, v) < 0 else 0)
    assert int(F.e4m3_encode(np.array([v], np.float32))[0]) == (0x80 if math.copysign(1, v) < 0 else 0)
