"""Pins for the oracle's format variants (readings R17, R18): MXFP8 (E4M3
elements, one E8M0 exponent per 32) and affine 4/8-bit with groups 32, 64
and 128 ("feat(quant): backend quantization capability table ...", Context:
the modes a ROCm backend runs and the group sizes its GEMV dispatches).

- the generic affine code path reproduces the pinned 4-bit / group-64
  quantizer bit for bit;
- exact reproduction of values built from representable parts (8-bit
  affine, MXFP8);
- error bounds (affine: half a step), MXFP8 exponent closed form,
  idempotence and saturation;
- dequantized values against torch's float8_e4m3fn / float8_e8m0fnu decoders.
"""
import numpy as np
import pytest
import torch

from synth_inputs import generic, to_bf16_bits

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def _p(a):
    import ctypes
    return a.ctypes.data_as(ctypes.c_void_p)


def unpack(q):
    per = 32 // q.bits
    c = (q.codes[:, :, None].astype(np.int64) >> (q.bits * np.arange(per))) & ((1 << q.bits) - 1)
    return c.reshape(q.rows, q.cols)


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_generic_affine_reproduces_4bit_group64(oracle_mod):
    o = oracle_mod
    x = generic((9, 640), 1.3, seed=60)
    q = o.quantize(0, x)
    codes = np.zeros_like(q.codes)
    scales = np.zeros_like(q.scales)
    biases = np.zeros_like(q.biases)
    o.lib().bo_quantize_affine_g(_p(x), 9, 640, 4, 64, _p(codes), _p(scales), _p(biases))
    assert np.array_equal(codes, q.codes) and np.array_equal(scales, q.scales)
    assert np.array_equal(biases, q.biases)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_affine8_exact_reproduction(oracle_mod, group):
    """x = -8 + q / 16 with q over 0..255 in every group (every value has at
    most 8 significant bits): scale 1/16, bias -8 and the codes come back."""
    o = oracle_mod
    rng = np.random.default_rng(group)
    n_groups = 6
    q = rng.integers(0, 256, (n_groups, group))
    q[:, 0], q[:, 1] = 0, 255
    x = to_bf16_bits((-8.0 + q / 16.0).astype(np.float32)).reshape(1, -1)
    qt = o.quantize(0, x, bits=8, group=group)
    assert np.array_equal(unpack(qt)[0], q.reshape(-1))
    assert np.all(bf16_f64(qt.scales) == 1 / 16) and np.all(bf16_f64(qt.biases) == -8.0)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_affine_variant_error_bound(oracle_mod, bits, group):
    o = oracle_mod
    x = generic((5, 512), 0.7, seed=61 + bits, stream=group)
    q = o.quantize(0, x, bits=bits, group=group)
    xs = bf16_f64(x)
    s = np.repeat(bf16_f64(q.scales), group, axis=1)
    b = np.repeat(bf16_f64(q.biases), group, axis=1)
    c = unpack(q)
    assert c.max() <= (1 << bits) - 1
    # the exact dequantized value is the independent s * c + b
    assert np.array_equal(o.dequant_exact(q), s * c + b)
    # within half a step plus the bf16 rounding of the bias and the step
    err = np.abs(s * c + b - xs)
    lim = s / 2 + (np.abs(b) + np.abs(xs) + s * ((1 << bits) - 1)) * 2.0 ** -8
    assert np.all(err <= lim)


def test_mxfp8_exponent_and_decoders(oracle_mod):
    o = oracle_mod
    x = generic((7, 256), 3.0, seed=62)
    x[0, :32] = 0  # an all-zero group
    q = o.quantize(3, x)
    xs = bf16_f64(x)
    am = np.abs(xs).reshape(7, 8, 32).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(am > 0, np.floor(np.log2(np.where(am > 0, am, 1))) - 8, -127)
    assert np.array_equal(q.scales.astype(np.int64) - 127, np.clip(e, -127, 127).astype(np.int64))
    c = unpack(q)
    v = E4M3[c] * np.repeat(E8M0[q.scales], 32, axis=1)
    assert np.array_equal(o.dequant_exact(q), v)
    # E4M3 keeps 4 significant bits: relative error at most 2^-4 of the value
    # (or half the subnormal step 2^-9 * 2^e); scaled magnitudes above 448
    # (a group max whose mantissa exceeds 1.75) saturate to +-448 * 2^e
    scale = np.repeat(2.0 ** (q.scales.astype(np.float64) - 127), 32, axis=1)
    sat = np.abs(xs) >= 448 * scale
    assert np.array_equal(v[sat], np.sign(xs[sat]) * 448 * scale[sat])
    ok = np.abs(v - xs) <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10 * scale)
    assert np.all(ok | sat)
    # the bf16 dequantization is the exact value rounded once
    assert np.array_equal(bf16_f64(o.dequantize(q)), bf16_f64(to_bf16_bits(v.astype(np.float32))))


def test_mxfp8_exact_reproduction_and_idempotence(oracle_mod):
    o = oracle_mod
    rng = np.random.default_rng(63)
    # E4M3 magnitudes times 2^e, group max forced to a value in [256, 448]
    codes = rng.integers(0, 0x7F, (4, 64))
    sign = rng.integers(0, 2, (4, 64)) * 0x80
    codes[:, 0], codes[:, 32] = 0x78, 0x7E  # 256 and 448 set the exponent
    e = np.array([[-3], [0], [5], [-20]])
    vals = E4M3[codes | sign] * np.repeat(2.0 ** e, 64, axis=1)
    x = to_bf16_bits(vals.astype(np.float32))
    q = o.quantize(3, x)
    assert np.array_equal(unpack(q), codes | sign)
    assert np.array_equal(q.scales.astype(np.int64) - 127, np.repeat(e, 2, axis=1))
    q2 = o.quantize(3, o.dequantize(q))
    assert np.array_equal(q2.codes, q.codes) and np.array_equal(q2.scales, q.scales)


def test_mxfp8_saturates(oracle_mod):
    o = oracle_mod
    # group max 1.99 * 2^8 scales to 509 > 448 at e = 0
    row = np.full(32, 1.0, np.float32)
    row[3], row[9] = 509.0, -500.0
    q = o.quantize(3, to_bf16_bits(row).reshape(1, 32))
    c = unpack(q)[0]
    assert q.scales[0, 0] == 127 and c[3] == 0x7E and c[9] == 0xFE


def _bf16_bits_of(v):
    """fp32 values -> bf16 bit patterns by torch's nearest-even conversion."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_affine_variant_dequantize_pinned(oracle_mod, bits, group):
    """bo_dequantize_g's affine branch against the rule R8 written out here
    with no oracle codec: codes unpacked by this test (element k at bit
    bits*(k % (32/bits)) of word k/(32/bits)), scale and bias decoded by
    torch, s*q + b formed in fp64 (s*q has at most 16 significant bits and
    the magnitudes below keep the sum exact), rounded once to fp32 (the
    single rounding of fma) and then to bf16 by torch.  Random codes over
    the whole range and random scales and biases of both signs, with groups
    whose fp32 rounding matters (|b| much larger than s*q), so a wrong group
    index, nibble order, a bias with the wrong sign or an early bf16
    rounding of s*q fails here."""
    o = oracle_mod
    rng = np.random.default_rng(1000 + 10 * bits + group)
    rows, cols = 7, 4 * group
    per = 32 // bits
    codes = rng.integers(0, 2 ** 32, (rows, cols // per), dtype=np.uint64).astype(np.uint32)
    ng = cols // group
    s = (rng.uniform(0.25, 1.0, (rows, ng)) * 2.0 ** rng.integers(-14, 2, (rows, ng)))
    b = rng.uniform(-1.0, 1.0, (rows, ng)) * 2.0 ** rng.integers(-6, 9, (rows, ng))
    s[0, 0] = 0.0   # a constant group: every value is the bias
    b[1, 1] = 0.0
    s[2, 0], b[2, 0] = 0.75 * 2.0 ** -20, 201.0  # s*q + b needs more than 24 bits
    s_bits = _bf16_bits_of(s.astype(np.float32))
    b_bits = _bf16_bits_of(b.astype(np.float32))
    q = o.QTensor(0, rows, cols, codes, s_bits, b_bits, bits=bits, group=group)
    got = o.dequantize(q)
    c = unpack(q).astype(np.float64)
    sv = np.repeat(bf16_f64(s_bits), group, axis=1)
    bv = np.repeat(bf16_f64(b_bits), group, axis=1)
    exact = sv * c + bv
    want = _bf16_bits_of(exact.astype(np.float32))
    assert np.array_equal(got, want)
    # the fp32 step matters for some elements (else the pin would not see
    # a skipped fp32 rounding)
    assert np.any(exact.astype(np.float32).astype(np.float64) != exact)
    # and the exact dequantized values are the same s*q + b
    assert np.array_equal(o.dequant_exact(q), exact)
