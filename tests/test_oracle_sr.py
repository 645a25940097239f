"""Pins for the oracle's stochastic-rounding quantize (reading R15 of the
oracle: the USE_SR variant of the 4-bit quantizer, "perf(cuda): enable
hardware NVFP4/MXFP4 conversion on Blackwell builds", Current Behavior;
the pages give no rounding rule or random-bit contract).

- closed forms: r = 0 rounds every inexact magnitude up to the next grid
  value, r = 0xFFFFFFFF rounds it down (checked against the published E2M1
  grid with numpy, not the oracle's codec);
- grid values and saturation are unchanged;
- unbiasedness: over a uniform sweep of the random words, the mean of the
  rounded values equals the input to 1/4096 of the grid spacing;
- the scales are those of round-to-nearest quantize, and every code is one of
  the two grid neighbours of its scaled input.
"""
import numpy as np
import pytest

from conftest import read_golden

from synth_inputs import generic, random_words, to_bf16_bits

GRID = np.array([float(v) for v in read_golden("formats.txt")[0][1:]])  # 0 .. 6


def neighbours(a):
    """(lower, upper) grid magnitudes around |v| (equal on a grid point)."""
    i = np.searchsorted(GRID, a, side="right") - 1
    lo = GRID[np.clip(i, 0, 7)]
    hi = np.where(GRID[np.clip(i, 0, 7)] == a, lo, GRID[np.clip(i + 1, 0, 7)])
    return lo, hi


def magnitude(code):
    return GRID[code & 7]


def test_extreme_words_floor_and_ceil(oracle_mod):
    o = oracle_mod
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-6, 6, 4000), GRID, -GRID, [5.999, 0.0001, 3.5, -4.75]])
    v = v.astype(np.float32)
    a = np.abs(v.astype(np.float64))
    lo, hi = neighbours(a)
    up = np.array([magnitude(o.e2m1_encode_sr(x, 0)) for x in v])
    down = np.array([magnitude(o.e2m1_encode_sr(x, 0xFFFFFFFF)) for x in v])
    assert np.array_equal(up, hi)
    # u = 1 - 2^-24 exceeds every p except p within 2^-24 of 1; none here
    assert np.array_equal(down, lo)
    signs = np.array([o.e2m1_encode_sr(x, 12345) >> 3 for x in v])
    assert np.array_equal(signs, np.signbit(v).astype(int))


def test_grid_values_and_saturation(oracle_mod):
    o = oracle_mod
    words = random_words(64, seed=1)
    for c, g in enumerate(GRID):
        for r in words:
            assert o.e2m1_encode_sr(g, r) == c
            assert o.e2m1_encode_sr(-g, r) == c | 8
    for v in (6.0, 6.5, 100.0, 3e38):
        for r in words[:8]:
            assert o.e2m1_encode_sr(v, r) == 7 and o.e2m1_encode_sr(-v, r) == 15


@pytest.mark.parametrize("v", [0.1, 0.37, 0.8, 1.3, 1.75, 2.2, 3.99, 4.5, 5.3])
def test_unbiased_over_uniform_words(oracle_mod, v):
    """MXFP4 rows of 32-groups that each hold one 4.0 (so every group's
    exponent is 0 and the scaled value is v itself) and 31 copies of v.  The
    j-th copy of v gets the word j * 2^20 (j < 4096, u = j / 4096): the
    number rounded up is ceil(p * 4096), so the mean of the 4096 rounded
    values is v to 1/4096 of the grid spacing."""
    o = oracle_mod
    n_v, per = 4096, 31
    groups = -(-n_v // per)
    row = np.zeros((groups, 32), np.float32)
    row[:, 0] = 4.0
    words = np.zeros((groups, 32), np.uint32)
    flat_v = row[:, 1:].reshape(-1)
    flat_w = words[:, 1:].reshape(-1)
    flat_v[:n_v] = v
    flat_w[:n_v] = (np.arange(n_v, dtype=np.uint64) << 20).astype(np.uint32)
    row[:, 1:] = flat_v.reshape(groups, per)
    words[:, 1:] = flat_w.reshape(groups, per)
    x = to_bf16_bits(row.reshape(-1)).reshape(1, -1)
    q = o.quantize(1, x, rbits=words.reshape(1, -1))
    assert np.all(q.scales == 127)  # exponent 0 in every group
    deq = o.dequant_exact(q)[0].reshape(groups, 32)[:, 1:].reshape(-1)[:n_v]
    vb = o.bf16_to_f64(x).reshape(groups, 32)[0, 1]
    lo, hi = neighbours(np.array([vb]))
    spacing = float(hi[0] - lo[0])
    assert abs(deq.mean() - vb) <= spacing / 4096 + 1e-12
    assert set(np.unique(deq)) <= {float(lo[0]), float(hi[0])}


@pytest.mark.parametrize("mode", [1, 2])
def test_scales_match_rne_and_codes_are_neighbours(oracle_mod, mode):
    o = oracle_mod
    x = generic((6, 256), 1.0, seed=50 + mode)
    r = random_words((6, 256), seed=51 + mode)
    qs = o.quantize(mode, x, rbits=r)
    qn = o.quantize(mode, x)
    assert np.array_equal(qs.scales, qn.scales)
    if mode == 2:
        assert qs.g == qn.g
    # scaled inputs: x / (dequantized block scale) (exactly what was rounded)
    xs = o.bf16_to_f64(x)
    codes = ((qs.codes[:, :, None].astype(np.int64) >> (4 * np.arange(8))) & 0xF).reshape(6, 256)
    G = o.GROUP[mode]
    if mode == 1:
        scale = np.repeat(2.0 ** (qs.scales.astype(np.float64) - 127), G, axis=1)
    else:
        e4m3 = np.array([o.lib().bo_e4m3_decode(int(c)) for c in range(256)])
        scale = np.repeat(e4m3[qs.scales], G, axis=1) * float(qs.g)
    v = np.abs(xs) / np.where(scale == 0, 1, scale)
    lo, hi = neighbours(np.minimum(v, 6.0))
    mag = magnitude(codes)
    ok = (mag == lo) | (mag == hi) | (scale == 0)
    assert ok.all()
    # round-to-nearest and stochastic codes differ somewhere but never by more
    # than one grid step
    assert not np.array_equal(qs.codes, qn.codes)
