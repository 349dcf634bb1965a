"""Pins for the oracle's FP8 E4M3 encode/decode.

Checked against: the format definition worked by hand (golden file), torch's
independent float8_e4m3fn conversion on the CPU, exact midpoints (ties to
even), the closed-form fact that every row's absmax element lands on +-240,
and the 3-bit-mantissa round-trip bound.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_known_codes.txt")


def _golden():
    rows = []
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, value = line.split()[:2]
        rows.append((int(code, 16), float(value)))
    return rows


def test_known_codes_from_format_definition():
    for code, value in _golden():
        got = orc.e4m3_to_float(code)
        if math.isnan(value):
            assert math.isnan(got), hex(code)
        else:
            assert got == value and math.copysign(1, got) == math.copysign(1, value), hex(code)


def test_table_matches_torch_float8_e4m3fn():
    table = orc.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    fin = ~np.isnan(table)
    assert np.array_equal(table[fin], ref[fin])
    assert np.array_equal(np.signbit(table[fin]), np.signbit(ref[fin]))


def test_table_is_monotone_and_symmetric():
    t = orc.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])
    assert pos.max() == orc.E4M3_MAX


def test_encode_round_trips_every_code():
    t = orc.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(orc.e4m3_encode(t[codes]), codes)


def test_midpoints_round_half_to_even():
    t = orc.e4m3_table()
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(np.array([mid]))[0] == even, hex(c)
        assert orc.e4m3_encode(np.array([-mid]))[0] == even | 0x80
        above = np.nextafter(np.float32(mid), np.float32(np.inf))
        below = np.nextafter(np.float32(mid), np.float32(0))
        assert orc.e4m3_encode(np.array([float(above)]))[0] == c + 1
        assert orc.e4m3_encode(np.array([float(below)]))[0] == c


def test_encode_matches_torch_on_random_in_range_values():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 30,
    ]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(y.astype(np.float64)), ref)


def test_saturation_and_signed_zero():
    vals = np.array([448.0, 449.0, 464.0, 480.0, 1e6, -1e6, -0.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -10])
    got = orc.e4m3_encode(vals)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x02]


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        orc.e4m3_encode(np.array([np.nan]))


def test_row_absmax_codes_to_240_and_scale_is_correctly_rounded():
    rng = np.random.default_rng(19)
    x = (rng.standard_normal((500, 512)) * rng.uniform(1e-3, 1e3, (500, 1))).astype(np.float32)
    codes, scales = orc.fp8_encode_rows(x)
    amax = np.abs(x).max(axis=1)
    # float32 division in numpy is IEEE correctly rounded: an independent route to the scale
    assert np.array_equal(scales, (amax / np.float32(240.0)).astype(np.float32))
    arg = np.abs(x).argmax(axis=1)
    picked = codes[np.arange(len(x)), arg]
    assert np.all((picked == 0x77) | (picked == 0xF7))


def test_zero_row_and_round_trip_bound():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1] = np.linspace(-3, 3, 64, dtype=np.float32)
    codes, scales = orc.fp8_encode_rows(x)
    assert scales[0] == 0 and np.all(codes[0] == 0)
    dec = orc.fp8_decode_rows(codes, scales)
    y = x[1].astype(np.float64) / float(scales[1])
    big = np.abs(y) >= 2.0 ** -6
    rel = np.abs(dec[1][big] - x[1][big]) / np.abs(x[1][big])
    assert rel.max() <= 2.0 ** -4 + 1e-12
    small = ~big
    assert np.all(np.abs(dec[1][small] - x[1][small]) <= 2.0 ** -10 * float(scales[1]) + 1e-15)


def test_decode_is_exact_product():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = np.where(np.isin(codes, [0x7F, 0xFF]), 0, codes).astype(np.uint8)
    s = np.array([np.float32(0.0123)], dtype=np.float32)
    dec = orc.fp8_decode_rows(codes, s)
    assert np.array_equal(dec[0], orc.e4m3_table()[codes[0]] * float(s[0]))


def _quotient_rows(seed, n_rows=400, row_len=256):
    """Rows whose elements sit one float32 ulp around values ``m * s`` where m
    is an E4M3 rounding midpoint and s the row's scale: there a quotient that
    is off by one ulp (a reciprocal multiply instead of a division) changes
    the code. Element 0 fixes the row's absmax (so s is known in advance)."""
    rng = np.random.default_rng(seed)
    t = orc.e4m3_table()[:0x77]
    mids = (t[:-1] + t[1:]) / 2                      # midpoints below 240
    rows = np.zeros((n_rows, row_len), dtype=np.float32)
    for r in range(n_rows):
        amax = np.float32(rng.uniform(0.5, 4.0) * 2.0 ** rng.integers(-20, 20))
        s = np.float32(amax / np.float32(240.0))
        m = rng.choice(mids, row_len - 1)
        x = (m * np.float64(s)).astype(np.float32)
        nudge = rng.integers(-2, 3, row_len - 1)
        for k in range(1, 3):
            up, dn = nudge >= k, nudge <= -k
            x[up] = np.nextafter(x[up], np.float32(np.inf))
            x[dn] = np.nextafter(x[dn], np.float32(0))
        x *= np.where(rng.random(row_len - 1) < 0.5, np.float32(-1), np.float32(1))
        rows[r, 0] = amax
        rows[r, 1:] = x
    return rows


def test_row_quotient_is_a_correctly_rounded_division():
    """Context Optimization, "FP8 KV Cache / How It Works": each value is
    divided by its position's scale before quantisation. The oracle's codes
    must equal torch's independent float8_e4m3fn cast of numpy's IEEE float32
    quotient x / s (a correctly rounded division), on random rows and on rows
    built so that a quotient one ulp off changes the code."""
    rng = np.random.default_rng(3)
    plain = (rng.standard_normal((300, 1024)) * rng.uniform(1e-4, 1e4, (300, 1))).astype(np.float32)
    for x in (plain, _quotient_rows(11)):
        codes, scales = orc.fp8_encode_rows(x)
        y = x / scales[:, None]                       # float32 / float32: IEEE division
        assert y.dtype == np.float32
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref)


def test_reciprocal_multiply_quotient_fails_the_pin():
    """Negative control for the pin above: a quotient taken as x * (1/s) in
    float32 gives other codes on the constructed rows, so the pin can tell the
    two apart."""
    x = _quotient_rows(11)
    codes, scales = orc.fp8_encode_rows(x)
    recip = (np.float32(1.0) / scales).astype(np.float32)
    y_bad = (x * recip[:, None]).astype(np.float32)
    bad = torch.from_numpy(y_bad).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(codes, bad)
