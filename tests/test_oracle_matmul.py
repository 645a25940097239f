"""Pins for the oracle's matmul references.

- tiny shapes against numpy's fp64 matmul over operands decoded here
  independently (torch's float8 / e8m0 decoders, the published E2M1 grid);
- one-hot activations (y = a column of the dequantized weights) and one-hot
  weights (y = selected activations), which pin nibble order, scale indexing
  and the row mapping;
- qq consistency: alpha * dq0(x) dq0(W)^T equals the product of the fully
  dequantized operands (the pages' alpha = amax_x amax_w / (448*6)^2);
- the dense path (W rounded to bf16 first): equal to the weight-only product
  where that rounding is exact, equal to a product over weights decoded and
  rounded independently here, and within 2^-8 of the weight-only product.
"""
import numpy as np
import pytest
import torch

from conftest import read_golden

from synth_inputs import generic, to_bf16_bits

GRID = np.array([float(v) for v in read_golden("formats.txt")[0][1:]])
E2M1 = np.concatenate([GRID, -GRID])
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def bf16_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def independent_dequant(o, q, with_g=True):
    """Decode codes, scales (and biases) without the oracle's codecs."""
    rows, cols = q.rows, q.cols
    c = ((q.codes[:, :, None].astype(np.int64) >> (4 * np.arange(8))) & 0xF).reshape(rows, cols)
    G = o.GROUP[q.mode]
    if q.mode == o.AFFINE:
        s = np.repeat(bf16_f64(q.scales), G, axis=1)
        b = np.repeat(bf16_f64(q.biases), G, axis=1)
        return s * c + b
    if q.mode == o.MXFP4:
        return E2M1[c] * np.repeat(E8M0[q.scales], G, axis=1)
    w = E2M1[c] * np.repeat(E4M3[q.scales], G, axis=1)
    if with_g and q.g is not None:
        w = w * float(q.g)
    return w


MODES = [0, 1, 2]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,groups", [(1, 17, 1), (3, 5, 4), (2, 16, 3)])
def test_matmul_bruteforce_tiny(oracle_mod, mode, M, N, groups):
    o = oracle_mod
    K = o.GROUP[mode] * groups
    x = generic((M, K), 1.0, seed=20 + mode, stream=M)
    w = generic((N, K), 0.02, seed=30 + mode, stream=N)
    q = o.quantize(mode, w)
    B = independent_dequant(o, q)
    assert np.array_equal(o.dequant_exact(q), B)
    A = bf16_f64(x)
    y, den = o.matmul_wonly(x, q)
    ref = A @ B.T
    assert y.shape == (M, N)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(den, np.abs(A) @ np.abs(B).T, rtol=1e-12)


@pytest.mark.parametrize("mode", MODES)
def test_onehot_activation_selects_weight_column(oracle_mod, mode):
    o = oracle_mod
    K = o.GROUP[mode] * 3
    N = 11
    w = generic((N, K), 0.02, seed=40 + mode)
    q = o.quantize(mode, w)
    B = independent_dequant(o, q)
    for j in (0, 1, 7, 8, K // 2 + 3, K - 1):
        x = np.zeros((1, K), np.uint16)
        x[0, j] = 0x3F80  # 1.0
        y, den = o.matmul_wonly(x, q)
        assert np.array_equal(y[0], B[:, j])
        # the bf16 output equals the rounded weight (zeros compare by value)
        assert np.array_equal(o.bf16_to_f32(o.bf16_from_f64(y[0])),
                              o.bf16_to_f32(o.bf16_from_f64(B[:, j])))


@pytest.mark.parametrize("mode", MODES)
def test_onehot_weights_select_activation(oracle_mod, mode):
    """Weights whose rows hold a single 1.0 at column j_n (unit scales, no
    global scale) give y[:, n] = x[:, j_n] exactly."""
    o = oracle_mod
    K = o.GROUP[mode] * 4
    N = 9
    rng = np.random.default_rng(50 + mode)
    j = rng.integers(0, K, N)
    x = generic((2, K), 1.0, seed=51 + mode)
    codes = np.zeros((N, K), np.int64)
    if mode == o.AFFINE:
        codes[np.arange(N), j] = 1
        scales = np.full((N, K // 64), 0x3F80, np.uint16)  # s = 1
        biases = np.zeros((N, K // 64), np.uint16)           # b = 0
    else:
        codes[np.arange(N), j] = 2                            # E2M1 1.0
        scales = np.full((N, K // o.GROUP[mode]), 127 if mode == o.MXFP4 else 0x38, np.uint8)
        biases = None
    words = np.zeros((N, K // 8), np.uint32)
    for k in range(8):
        words |= (codes[:, k::8].astype(np.uint32) << (4 * k))
    q = o.QTensor(mode, N, K, words, scales, biases, None)
    y, _ = o.matmul_wonly(x, q)
    assert np.array_equal(y, bf16_f64(x)[:, j])


def test_qq_alpha_consistency(oracle_mod):
    o = oracle_mod
    x = generic((3, 64), 0.02, seed=60)
    w = generic((7, 64), 0.02, seed=61)
    qw = o.quantize(o.NVFP4, w)
    y, den, qx, a = o.matmul_qq(x, qw)
    assert a == o.alpha(qx.g, qw.g)
    ref = independent_dequant(o, qx, with_g=True) @ independent_dequant(o, qw, with_g=True).T
    np.testing.assert_allclose(y, ref, rtol=4e-7)
    closed = float(qx.amax) * float(qw.amax) / 7225344.0
    assert abs(float(a) - closed) <= 3 * np.spacing(np.float32(closed))
    # qq for the other modes: alpha is 1 and x uses the weights' mode
    for mode in (o.MXFP4, o.AFFINE):
        qw2 = o.quantize(mode, w)
        y2, _, qx2, a2 = o.matmul_qq(x, qw2)
        assert a2 == 1.0 and qx2.mode == mode
        np.testing.assert_allclose(
            y2, independent_dequant(o, qx2) @ independent_dequant(o, qw2).T, rtol=1e-12)


def test_pairs_match_full(oracle_mod):
    o = oracle_mod
    A = bf16_f64(generic((5, 96), 1.0, seed=70))
    B = bf16_f64(generic((13, 96), 1.0, seed=71))
    y, d = o.matmul_f64(A, B, 0.5)
    ai = np.array([0, 4, 2, 3, 1]); bi = np.array([12, 0, 5, 7, 3])
    yp, dp = o.matmul_pairs(A, B, ai, bi, 0.5)
    assert np.array_equal(yp, y[ai, bi]) and np.array_equal(dp, d[ai, bi])


def test_norm_err(oracle_mod):
    o = oracle_mod
    yref = np.array([1.0, -2.0, 0.0, 0.0])
    den = np.array([4.0, 2.0, 0.0, 0.0])
    ybits = to_bf16_bits(np.array([1.0078125, -2.0, 0.0, 1.0], np.float32))
    e = o.norm_err(ybits, yref, den)
    assert e[0] == pytest.approx(0.0078125 / 4)
    assert e[1] == 0 and e[2] == 0 and np.isinf(e[3])


def independent_bf16_weights(o, q):
    """The dequantize rule without the oracle's codecs: the fp32 value
    (E2M1 * E4M3 exact, times g rounded to fp32; affine fma(s, q, b) in one
    fp32 rounding, exact in fp64 for these magnitudes), then fp32 -> bf16
    nearest even (torch's conversion)."""
    w = independent_dequant(o, q, with_g=False)
    if q.mode == o.NVFP4 and q.g is not None:
        w32 = w.astype(np.float32) * np.float32(q.g)
    else:
        w32 = w.astype(np.float32)
    return torch.from_numpy(w32).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("use_global", [True, False])
def test_dense_path_pins(oracle_mod, mode, use_global):
    o = oracle_mod
    if mode != o.NVFP4 and not use_global:
        pytest.skip("the global scale exists for NVFP4 only")
    M, N, K = 3, 40, 128
    x = generic((M, K), 1.0, seed=40 + mode, stream=int(use_global))
    w = generic((N, K), 0.02, seed=41 + mode)
    q = o.quantize(mode, w, use_global=use_global) if mode == o.NVFP4 else o.quantize(mode, w)
    yd, dd = o.matmul_dense(x, q)
    yw, dw = o.matmul_wonly(x, q)
    # independent decode and rounding
    yi, _ = o.matmul_f64(bf16_f64(x), independent_bf16_weights(o, q))
    assert np.array_equal(yd, yi)
    # bf16 rounding of W is exact for MXFP4 and for NVFP4 without g
    if mode == o.MXFP4 or (mode == o.NVFP4 and not use_global):
        assert np.array_equal(yd, yw) and np.array_equal(dd, dw)
    # within one bf16 rounding of the weights (relative 2^-8)
    assert np.all(np.abs(yd - yw) <= 2.0 ** -8 * dw + 1e-300)
    # the row selection returns the same weights
    rows = np.array([0, 7, N - 1])
    assert np.array_equal(o.matmul_dense(x, q, rows=rows), independent_bf16_weights(o, q)[rows])
