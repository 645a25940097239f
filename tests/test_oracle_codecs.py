"""Pins for the oracle's scalar codecs (E2M1, E4M3, E8M0, bf16).

Each codec is checked against something other than itself: the published
grids and code points (tests/golden/formats.txt), hand-derived decision
boundaries (tests/golden/e2m1_thresholds.txt), torch's own fp8 / e8m0 / bf16
conversions, and exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden


def _golden_dict(name):
    d = {}
    for row in read_golden(name):
        d.setdefault(row[0], []).append(row[1:])
    return d


FORMATS = _golden_dict("formats.txt")


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f)
    return bits[keep], f[keep]


# ---------------------------------------------------------------- E2M1

def test_e2m1_grid_matches_published(oracle_mod):
    grid = np.array([float(v) for v in FORMATS["e2m1_grid"][0]])
    t = oracle_mod.e2m1_table()
    assert np.array_equal(t[:8], grid)
    assert np.array_equal(t[8:], -grid)
    assert np.signbit(t[8])  # code 8 is -0
    assert t.max() == 6.0


def test_e2m1_thresholds_handworked(oracle_mod):
    for b, below, at, above in read_golden("e2m1_thresholds.txt"):
        t = np.float32(b)
        lo = np.nextafter(t, np.float32(-np.inf))
        hi = np.nextafter(t, np.float32(np.inf))
        got = oracle_mod.e2m1_encode(np.array([lo, t, hi], np.float32))
        assert list(got) == [int(below), int(at), int(above)], b
        gotn = oracle_mod.e2m1_encode(-np.array([lo, t, hi], np.float32))
        assert list(gotn) == [int(below) | 8, int(at) | 8, int(above) | 8], b


def test_e2m1_encode_all_bf16_by_threshold_table(oracle_mod):
    """Every finite bf16 value, classified independently by the hand-derived
    boundary table (a searchsorted over the boundaries with the tie rule),
    must agree with the oracle's nearest-value search."""
    bits, f = all_finite_bf16()
    rows = read_golden("e2m1_thresholds.txt")[:-1]  # drop the saturation row
    bounds = np.array([float(r[0]) for r in rows])
    code_at = np.array([int(r[2]) for r in rows])
    a = np.abs(f.astype(np.float64))
    idx = np.searchsorted(bounds, a, side="left")       # number of bounds < a
    exact = np.isin(a, bounds)
    pos = np.searchsorted(bounds, a)
    code = idx.copy()
    code[exact] = code_at[pos[exact]]
    code = code | np.where(np.signbit(f), 8, 0)
    got = oracle_mod.e2m1_encode(f)
    assert np.array_equal(got, code.astype(np.uint8))


def test_e2m1_encode_roundtrip_and_monotone(oracle_mod):
    t = oracle_mod.e2m1_table()
    for c in range(16):
        assert oracle_mod.e2m1_encode(np.array([t[c]], np.float32))[0] == c
    v = np.linspace(0, 10, 20001, dtype=np.float32)
    mag = t[oracle_mod.e2m1_encode(v) & 7]
    assert np.all(np.diff(mag) >= 0)
    # error at most half the local grid gap below saturation
    inside = v <= 6
    grid = t[:8]
    gaps = np.diff(grid)
    seg = np.clip(np.searchsorted(grid, v[inside], side="right") - 1, 0, 6)
    assert np.all(np.abs(mag[inside] - v[inside]) <= gaps[seg] / 2 + 1e-7)
    assert oracle_mod.e2m1_encode(np.array([np.inf, -np.inf, 1e30], np.float32)).tolist() == [7, 15, 7]


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = oracle_mod.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    for code, val in FORMATS["e4m3_point"]:
        assert got[int(code)] == float(val)
    assert got[int(FORMATS["e4m3_max_code"][0][0])] == float(FORMATS["e4m3_max"][0][0])


def _e4m3_probe_values():
    t = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)
    probes = [t, mids,
              np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))]
    _, f = all_finite_bf16()
    probes.append(f[(f >= 0) & (f <= 448)])
    rng = np.random.default_rng(7)
    probes.append((rng.random(200000) * 448).astype(np.float32))
    probes.append(np.exp2(rng.uniform(-14, 8.8, 200000)).astype(np.float32))
    v = np.concatenate(probes)
    return v[(v >= 0) & (v <= 448) & ~np.signbit(v)]


def test_e4m3_encode_matches_torch_in_range(oracle_mod):
    """Within [0, 448] the encoder must equal torch's round-to-nearest-even
    float8_e4m3fn conversion (a library routine), including every tie."""
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle_mod.e4m3_encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates_above_max(oracle_mod):
    v = np.array([448.0, np.nextafter(np.float32(448), np.float32(1e9)), 464.0, 470.0, 1e6, np.inf],
                 np.float32)
    assert oracle_mod.e4m3_encode(v).tolist() == [0x7E] * 6


# ---------------------------------------------------------------- E8M0

def test_e8m0_decode_matches_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = oracle_mod.e8m0_table()
    assert np.array_equal(got[:255], ref[:255])
    assert np.isnan(got[255])
    for code, val in FORMATS["e8m0_point"]:
        assert got[int(code)] == float(val)


# ---------------------------------------------------------------- bf16

def test_bf16_from_f32_matches_torch(oracle_mod):
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=400000, dtype=np.uint64).astype(np.uint32)
    # force ties and near-ties in a third of the samples
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000
    u[1::3] = (u[1::3] & 0xFFFF0000) | rng.choice([0x7FFF, 0x8001, 0x0000, 0xFFFF], size=u[1::3].size)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle_mod.bf16_from_f32(f)
    # values that overflow to inf are outside the contract
    ok = np.isfinite(oracle_mod.bf16_to_f32(ref))
    assert np.array_equal(got[ok], ref[ok])


def _nearest_bf16_exact(d):
    """Nearest bf16 to double d by exact rational comparison (tie: even)."""
    f = np.float32(d)
    base = int(np.array([f], np.float32).view(np.uint32)[0] >> 16) & 0x7FFF
    sign = 0x8000 if d < 0 else 0
    best, bd = None, None
    for m in (base - 1, base, base + 1):
        if m < 0 or m >= 0x7F80:
            continue
        v = float(np.array([(sign | m) << 16], np.uint32).view(np.float32)[0])
        dist = abs(Fraction(d) - Fraction(v))
        if best is None or dist < bd or (dist == bd and m % 2 == 0):
            best, bd = m, dist
    return sign | best


def test_bf16_from_f64_single_rounding(oracle_mod):
    rng = np.random.default_rng(12)
    d = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    # exact midpoints between neighbouring bf16 values, and one ulp either side
    b = rng.integers(0x0080, 0x7F00, 1000).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    d = np.concatenate([d, mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    got = oracle_mod.bf16_from_f64(d)
    ref = np.array([_nearest_bf16_exact(v) for v in d], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- constants

def test_constants(oracle_mod):
    e4m3_max = float(FORMATS["e4m3_max"][0][0])
    e2m1_max = float(FORMATS["e2m1_grid"][0][-1])
    assert e4m3_max * e2m1_max == float(FORMATS["nvfp4_max_product"][0][0])
    assert (e4m3_max * e2m1_max) ** 2 == float(FORMATS["alpha_denominator"][0][0])
    # g for amax = 2688 is exactly 1
    assert oracle_mod.global_scale(2688.0) == np.float32(1.0)
    assert oracle_mod.global_scale(0.0) == np.float32(0.0)
