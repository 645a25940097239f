"""Pins for the oracle's quantizers and dequantizers.

- hand-worked examples (tests/golden/worked_examples.txt);
- exact reproduction of values built from representable parts;
- invariants: MXFP4 idempotence, per-element error bounds, zero rules;
- the global scale and alpha against their closed forms.
"""
import numpy as np
import pytest

from conftest import read_golden

from synth_inputs import generic, to_bf16_bits


def _worked():
    d = {}
    for row in read_golden("worked_examples.txt"):
        name, field = row[0].split(".")
        d.setdefault(name, {})[field] = row[1:]
    return d


WORKED = _worked()


def _bits(vals):
    # -0 must stay negative zero
    return to_bf16_bits(np.array([float(v) for v in vals], np.float32)).reshape(1, -1)


def _ints(vals):
    return [int(v, 0) for v in vals]


@pytest.mark.parametrize("name", ["nvfp4_a", "nvfp4_b", "nvfp4_c"])
def test_nvfp4_worked_examples(oracle_mod, name):
    ex = WORKED[name]
    x = _bits(ex["x"])
    g = ex["g"][0]
    if g == "none":
        q = oracle_mod.quantize(oracle_mod.NVFP4, x, use_global=False)
    else:
        q = oracle_mod.quantize(oracle_mod.NVFP4, x, use_global=True, g=float(g))
    assert q.scales.ravel().tolist() == _ints(ex["scales"])
    assert q.codes.ravel().tolist() == _ints(ex["words"])


@pytest.mark.parametrize("name", ["mxfp4_a", "mxfp4_b"])
def test_mxfp4_worked_examples(oracle_mod, name):
    ex = WORKED[name]
    q = oracle_mod.quantize(oracle_mod.MXFP4, _bits(ex["x"]))
    assert q.scales.ravel().tolist() == _ints(ex["scales"])
    assert q.codes.ravel().tolist() == _ints(ex["words"])


def test_affine_worked_example(oracle_mod):
    ex = WORKED["affine_a"]
    q = oracle_mod.quantize(oracle_mod.AFFINE, _bits(ex["x"]))
    assert q.scales.ravel().tolist() == _ints(ex["scales"])
    assert q.biases.ravel().tolist() == _ints(ex["biases"])
    assert q.codes.ravel().tolist() == _ints(ex["words"])


def test_packing_order(oracle_mod):
    """Codes 1..8 in elements 0..7 pack to 0x87654321 (low nibble first):
    values 0.5,1,1.5,2,3,4,6 and -0 with a unit scale (no global scale,
    bamax 6 -> S = 1)."""
    x = _bits([0.5, 1, 1.5, 2, 3, 4, 6, -0.0] + [0] * 8)
    q = oracle_mod.quantize(oracle_mod.NVFP4, x, use_global=False)
    assert q.codes[0, 0] == 0x87654321
    assert q.codes[0, 1] == 0


# ------------------------------------------------------------ exact reproduction

def _nvfp4_exact_tensor(rng, rows, cols, k):
    """x = v * S * 2^k with v on the E2M1 grid (max |v| = 6 per block), S an
    E4M3 value; one block holds 6 * 448 * 2^k so that amax/2688 = 2^k."""
    from oracle import oracle as o
    grid = o.e2m1_table()
    e4 = o.e4m3_table()
    nb = cols // 16
    codes = rng.integers(0, 16, size=(rows, nb, 16))
    codes[..., rng.integers(0, 16)] = rng.choice([7, 15], size=(rows, nb))  # |v| = 6 somewhere
    S = rng.integers(0x20, 0x70, size=(rows, nb))  # comfortably normal E4M3 values
    S[0, 0] = 0x7E
    v = grid[codes]
    x = v * e4[S][..., None] * 2.0 ** k
    return to_bf16_bits(x.reshape(rows, cols).astype(np.float32)), codes, S


@pytest.mark.parametrize("k", [0, -7, 5])
def test_nvfp4_exact_reproduction(oracle_mod, k):
    rng = np.random.default_rng(100 + k)
    x, codes, S = _nvfp4_exact_tensor(rng, 6, 160, k)
    # the bf16 inputs are exact (6 significant bits at most)
    assert np.array_equal(oracle_mod.bf16_to_f32(x).astype(np.float64),
                          (oracle_mod.e2m1_table()[codes] * oracle_mod.e4m3_table()[S][..., None]
                           * 2.0 ** k).reshape(6, 160))
    q = oracle_mod.quantize(oracle_mod.NVFP4, x)
    assert q.g == np.float32(2.0 ** k)
    assert q.amax == np.float32(2688 * 2.0 ** k)
    assert np.array_equal(q.scales, S.astype(np.uint8))
    got_codes = (q.codes[:, :, None] >> (4 * np.arange(8))) & 0xF
    assert np.array_equal(got_codes.reshape(6, 160), codes.reshape(6, 160))
    assert np.array_equal(oracle_mod.dequantize(q), x)


@pytest.mark.parametrize("maxv", [4.0, 6.0])
def test_mxfp4_exact_reproduction(oracle_mod, maxv):
    rng = np.random.default_rng(int(maxv))
    grid = oracle_mod.e2m1_table()
    rows, cols = 5, 256
    nb = cols // 32
    codes = rng.integers(0, 16, size=(rows, nb, 32))
    codes = np.where((codes & 7) > (6 if maxv == 4.0 else 7), codes - 1, codes)
    codes[..., 3] = 6 if maxv == 4.0 else 7
    e = rng.integers(-20, 20, size=(rows, nb))
    x = grid[codes] * 2.0 ** e[..., None]
    xb = to_bf16_bits(x.reshape(rows, cols).astype(np.float32))
    q = oracle_mod.quantize(oracle_mod.MXFP4, xb)
    assert np.array_equal(q.scales.astype(int), e + 127)
    got_codes = (q.codes[:, :, None] >> (4 * np.arange(8))) & 0xF
    assert np.array_equal(got_codes.reshape(rows, cols), codes.reshape(rows, cols))
    assert np.array_equal(oracle_mod.dequantize(q), xb)


@pytest.mark.parametrize("step_mant", [1, 3])
def test_affine_exact_reproduction(oracle_mod, step_mant):
    rng = np.random.default_rng(step_mant)
    rows, cols = 4, 256
    nb = cols // 64
    j = rng.integers(-12, -2, size=(rows, nb))
    sb = step_mant * 2.0 ** j
    c = rng.integers(-40, 40, size=(rows, nb))
    bb = c * 2.0 ** j
    q_true = rng.integers(0, 16, size=(rows, nb, 64))
    q_true[..., 0] = 0
    q_true[..., 1] = 15
    x = bb[..., None] + sb[..., None] * q_true
    xb = to_bf16_bits(x.reshape(rows, cols).astype(np.float32))
    assert np.array_equal(oracle_mod.bf16_to_f32(xb).astype(np.float64), x.reshape(rows, cols))
    q = oracle_mod.quantize(oracle_mod.AFFINE, xb)
    assert np.array_equal(oracle_mod.bf16_to_f32(q.scales).astype(np.float64), sb)
    assert np.array_equal(oracle_mod.bf16_to_f32(q.biases).astype(np.float64), bb)
    got = (q.codes[:, :, None] >> (4 * np.arange(8))) & 0xF
    assert np.array_equal(got.reshape(rows, cols), q_true.reshape(rows, cols))
    assert np.array_equal(oracle_mod.dequantize(q), xb)


# ------------------------------------------------------------ invariants

def test_mxfp4_idempotent(oracle_mod):
    x = generic((16, 512), 1.0, seed=3)
    q1 = oracle_mod.quantize(oracle_mod.MXFP4, x)
    q2 = oracle_mod.quantize(oracle_mod.MXFP4, oracle_mod.dequantize(q1))
    assert np.array_equal(q1.codes, q2.codes)
    assert np.array_equal(q1.scales, q2.scales)


def _unpack(codes, cols):
    return ((codes[:, :, None] >> (4 * np.arange(8))) & 0xF).reshape(codes.shape[0], cols)


def test_nvfp4_error_bound(oracle_mod):
    """|x - xhat| <= half the local E2M1 gap times d (plus fp32/bf16
    rounding) for unsaturated elements; saturated ones stay within the E4M3
    rounding of the block scale."""
    x = generic((32, 1024), 1.0, seed=4)
    q = oracle_mod.quantize(oracle_mod.NVFP4, x)
    xf = oracle_mod.bf16_to_f32(x).astype(np.float64)
    xh = oracle_mod.bf16_to_f32(oracle_mod.dequantize(q)).astype(np.float64)
    d = (oracle_mod.e4m3_table()[q.scales] * np.float64(q.g))
    d = np.repeat(d, 16, axis=1)
    grid = oracle_mod.e2m1_table()[:8]
    r = np.abs(xf) / d
    gaps = np.diff(grid)
    seg = np.clip(np.searchsorted(grid, np.minimum(r, 6), side="right") - 1, 0, 6)
    bound = np.where(r <= 6, gaps[seg] / 2 * d, np.abs(xf) - 6 * d) + 2 ** -8 * np.abs(xh) + 1e-12
    assert np.all(np.abs(xf - xh) <= bound * (1 + 1e-6))
    assert np.all(r <= 6 / (1 - 2 ** -4) * (1 + 1e-6))
    # dequantized values never exceed the block maximum by more than the scale rounding
    assert np.all(np.abs(xh) <= np.abs(xf).reshape(32, -1, 16).max(-1).repeat(16, 1) * (1 + 2 ** -3))


def test_mxfp4_error_bound(oracle_mod):
    x = generic((32, 1024), 1.0, seed=5)
    q = oracle_mod.quantize(oracle_mod.MXFP4, x)
    xf = oracle_mod.bf16_to_f32(x).astype(np.float64)
    xh = oracle_mod.bf16_to_f32(oracle_mod.dequantize(q)).astype(np.float64)
    s = np.repeat(oracle_mod.e8m0_table()[q.scales], 32, axis=1)
    r = np.abs(xf) / s
    grid = oracle_mod.e2m1_table()[:8]
    seg = np.clip(np.searchsorted(grid, np.minimum(r, 6), side="right") - 1, 0, 6)
    bound = np.where(r <= 6, np.diff(grid)[seg] / 2 * s, np.abs(xf) - 6 * s)
    assert np.all(np.abs(xf - xh) <= bound + 1e-30)
    assert np.all(r < 8)  # the floor rule keeps bamax/2^e in [4, 8)


def test_affine_error_bound(oracle_mod):
    x = generic((32, 1024), 0.02, seed=6)
    q = oracle_mod.quantize(oracle_mod.AFFINE, x)
    xf = oracle_mod.bf16_to_f32(x).astype(np.float64)
    xh = oracle_mod.bf16_to_f32(oracle_mod.dequantize(q)).astype(np.float64)
    s = np.repeat(oracle_mod.bf16_to_f32(q.scales).astype(np.float64), 64, axis=1)
    b = np.repeat(oracle_mod.bf16_to_f32(q.biases).astype(np.float64), 64, axis=1)
    mn = xf.reshape(32, -1, 64).min(-1).repeat(64, 1)
    mx = xf.reshape(32, -1, 64).max(-1).repeat(64, 1)
    s_true = (mx - mn) / 15
    assert np.array_equal(b, mn)                       # bias is the exact group min
    assert np.all(np.abs(s - s_true) <= 2 ** -8 * s_true + 1e-30)
    bound = 0.5 * s * (1 + 1e-6) + 15 * np.abs(s - s_true) + 2 ** -8 * np.abs(xh) + 1e-12
    assert np.all(np.abs(xf - xh) <= bound)


def test_zero_rules(oracle_mod):
    z = np.zeros((2, 64), np.uint16)
    q = oracle_mod.quantize(oracle_mod.NVFP4, z)
    assert q.g == 0 and q.amax == 0
    assert not q.codes.any() and not q.scales.any()
    assert not oracle_mod.dequantize(q).any()
    q = oracle_mod.quantize(oracle_mod.MXFP4, z)
    assert not q.codes.any() and not q.scales.any()
    # a zero block inside a non-zero tensor
    x = generic((1, 64), 1.0, seed=9)
    x[0, 16:32] = 0
    q = oracle_mod.quantize(oracle_mod.NVFP4, x)
    assert q.scales[0, 1] == 0 and q.codes[0, 2] == 0 and q.codes[0, 3] == 0
    x[0, 32:64] = 0
    q = oracle_mod.quantize(oracle_mod.MXFP4, x)
    assert q.scales[0, 1] == 0 and not q.codes[0, 4:].any()
    # affine constant group: scale 0, codes 0, bias = the constant
    c = to_bf16_bits(np.full((1, 64), -0.375, np.float32))
    q = oracle_mod.quantize(oracle_mod.AFFINE, c)
    assert q.scales[0, 0] == 0 and not q.codes.any()
    assert np.array_equal(oracle_mod.dequantize(q), c)


def test_nvfp4_given_global_scale_saturates(oracle_mod):
    """A caller-given g far too small saturates the block scale at 448 and
    then the codes at 6."""
    x = generic((1, 32), 1.0, seed=10)
    q = oracle_mod.quantize(oracle_mod.NVFP4, x, use_global=True, g=1e-6)
    assert np.all(q.scales == 0x7E)
    c = _unpack(q.codes, 32)
    xf = oracle_mod.bf16_to_f32(x)
    big = np.abs(xf[0]) > 6 * 448 * 1e-6 * 1.01
    assert np.all((c[0][big] & 7) == 7)


def test_global_scale_and_alpha_closed_form(oracle_mod):
    rng = np.random.default_rng(13)
    for _ in range(200):
        ax = np.float32(np.exp(rng.uniform(-8, 8)))
        aw = np.float32(np.exp(rng.uniform(-8, 8)))
        gx, gw = oracle_mod.global_scale(ax), oracle_mod.global_scale(aw)
        assert gx == np.float32(ax) / np.float32(2688)   # correctly rounded fp32 divide
        a = oracle_mod.alpha(gx, gw)
        closed = float(ax) * float(aw) / 7225344.0
        assert abs(float(a) - closed) <= 3 * np.spacing(np.float32(closed))
    assert oracle_mod.alpha(oracle_mod.global_scale(2688), oracle_mod.global_scale(2688)) == 1.0


def test_amax_matches_numpy(oracle_mod):
    x = generic((64, 320), 3.0, seed=14)
    assert oracle_mod.amax(x) == np.float32(np.abs(oracle_mod.bf16_to_f32(x)).max())
    q = oracle_mod.quantize(oracle_mod.NVFP4, x)
    assert q.amax == oracle_mod.amax(x)
    # the maximum at the first, a middle and the last position, either sign
    # (bf16 0x4200 = 32, 0xC200 = -32, above every N(0, 3^2) draw here)
    for pos in (0, x.size // 2, x.size - 1):
        for bits in (0x4200, 0xC200):
            y = x.copy().reshape(-1)
            y[pos] = bits
            assert oracle_mod.amax(y.reshape(x.shape)) == np.float32(32.0), (pos, bits)
