"""Pins for the oracle's scalar codecs (bf16 widening, OCP E4M3 decode/encode).

Each check compares the oracle with something other than itself: torch's
float8_e4m3fn / bfloat16 casts, hand-worked fixtures from the OCP format
definition, and an independent nearest-value search over the 254 finite codes.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def _torch_fp8_values(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = _torch_fp8_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan).tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros
    assert math.copysign(1.0, ours[0x80]) == -1.0 and ours[0x80] == 0.0


def test_fp8_decode_golden():
    for code, val in _read_fixture("ocp_e4m3_decode.txt"):
        got = oracle.fp8_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_fp8_encode_golden():
    for row in _read_fixture("ocp_e4m3_encode.txt"):
        x, code = float(row[0]), int(row[1], 16)
        got = int(oracle.fp8_quantise(np.array([x], dtype=np.float32))[0])
        assert got == code, (row, hex(got))


def _finite_table():
    """Positive finite E4M3 values and their codes, from torch's decode (not the oracle's)."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # 0x00..0x7E
    vals = _torch_fp8_values(codes)
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


def _nearest_code(y: np.ndarray) -> np.ndarray:
    """Independent encoder: nearest finite code by search, ties to even code, saturating."""
    vals, codes = _finite_table()
    with np.errstate(invalid="ignore"):
        y = y.astype(np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    nan = np.isnan(a)
    sat = ~nan & (a >= vals[-1])
    mid = ~nan & ~sat
    am = a[mid]
    hi = np.searchsorted(vals, am, side="left")
    hi = np.clip(hi, 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = am - vals[lo], vals[hi] - am
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    exact = vals[lo] == am
    idx = np.where(exact, lo, np.where(pick_hi, hi, lo))
    out[mid] = codes[idx]
    out[sat] = 0x7E
    out[nan] = 0x7F
    return out | sign


def _interesting_floats() -> np.ndarray:
    vals, _ = _finite_table()
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact ties (representable in fp32)
    pts = np.concatenate([vals, mids, [464.0, 480.0, 1e30, np.inf, 2.0 ** -10, 2.0 ** -12, 2.0 ** -149]])
    pts = pts.astype(np.float32)
    around = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    return np.concatenate([around, -around, np.array([np.nan, -np.nan, 0.0, -0.0], dtype=np.float32)])


def test_fp8_encode_matches_independent_search():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    rand = bits.view(np.float32)
    # concentrate half of the draws on the representable range
    dense = (rng.standard_normal(1_000_000) * 64).astype(np.float32)
    tiny = (rng.standard_normal(500_000) * 2.0 ** -8).astype(np.float32)
    for y in (_interesting_floats(), rand, dense, tiny):
        got = oracle.fp8_quantise(y)
        want = _nearest_code(y)
        nan = np.isnan(y)
        # NaN: both give a NaN code; the sign is kept
        assert np.all((got[nan] & 0x7F) == 0x7F)
        assert np.array_equal(got[~nan], want[~nan])


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    y = np.concatenate([(rng.standard_normal(1_000_000) * 100).astype(np.float32), _interesting_floats()])
    y = y[np.isfinite(y) & (np.abs(y) <= 448)]
    got = oracle.fp8_quantise(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_fp8_quantise_divides_in_fp32():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200_000).astype(np.float32) * 3
    for s in (1.0, 0.5, 3.0, 1.0 / 448, 0.0123456):
        s32 = np.float32(s)
        y = (x / s32).astype(np.float32)  # numpy float32 division: IEEE, correctly rounded
        assert np.array_equal(oracle.fp8_quantise(x, float(s32)), _nearest_code(y))


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 16, size=200_000, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_double(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
