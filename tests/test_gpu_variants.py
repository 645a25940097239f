"""GPU parity of the format variants (MXFP8; affine 4-bit groups 32 / 128;
affine 8-bit groups 32 / 64 / 128) against the oracle (readings R17, R18):
quantize and dequantize bit-exact, the GEMV within the weight-only bar, the
dense prefill path within the qq bar ("feat(quant): backend quantization
capability table ...", Context / Gate impact)."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import from_dev, oracle_to_dev, to_dev, u8, words

pytestmark = pytest.mark.gpu

TOL = 3e-3
QQ_TOL = 2.2e-3
VARIANTS = [(3, 8, 32), (0, 4, 32), (0, 4, 128), (0, 8, 32), (0, 8, 64), (0, 8, 128)]
IDS = ["mxfp8", "aff4g32", "aff4g128", "aff8g32", "aff8g64", "aff8g128"]


def quant_both(o, b, x, fmt):
    mode, bits, group = fmt
    q = b.quantize(to_dev(x), mode, bits=bits, group=group)
    qo = o.quantize(mode, x, bits=bits, group=group)
    torch.cuda.synchronize()
    return q, qo


def assert_same(o, q, qo):
    assert np.array_equal(words(q.codes), qo.codes), "codes differ"
    if q.mode == o.AFFINE:
        assert np.array_equal(from_dev(q.scales), qo.scales), "scales differ"
        assert np.array_equal(from_dev(q.biases), qo.biases), "biases differ"
    else:
        assert np.array_equal(u8(q.scales), qo.scales), "scales differ"


@pytest.mark.parametrize("fmt", VARIANTS, ids=IDS)
@pytest.mark.parametrize("shape", [(1, 128), (37, 128 * 9), (3, 2944), (65, 5120)])
def test_variant_quantize_dequantize_exact(oracle_mod, bsfp, fmt, shape):
    o = oracle_mod
    x = S.generic(shape, 1.5, seed=400 + fmt[1] + fmt[2], stream=shape[0])
    q, qo = quant_both(o, bsfp, x, fmt)
    assert_same(o, q, qo)
    assert np.array_equal(from_dev(bsfp.dequantize(q)), o.dequantize(qo))


def _all_bf16_blocks():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < 1e36)
    bits = b[keep]
    n = (bits.size // 128) * 128
    return bits[:n].reshape(-1, 128)


@pytest.mark.parametrize("fmt", VARIANTS, ids=IDS)
def test_variant_every_bf16_value(oracle_mod, bsfp, fmt):
    o = oracle_mod
    x = _all_bf16_blocks()
    rng = np.random.default_rng(7)
    for xx in (x, rng.permutation(x.reshape(-1)).reshape(x.shape)):
        q, qo = quant_both(o, bsfp, xx, fmt)
        assert_same(o, q, qo)
        assert np.array_equal(from_dev(bsfp.dequantize(q)), o.dequantize(qo))


@pytest.mark.parametrize("fmt", VARIANTS, ids=IDS)
@pytest.mark.parametrize("M,N,K", [(1, 70, 128), (1, 333, 1024 * 3), (2, 129, 1152),
                                   (5, 300, 2048), (8, 77, 1408), (1, 4100, 5120)])
def test_variant_qmv(oracle_mod, bsfp, fmt, M, N, K):
    o = oracle_mod
    mode, bits, group = fmt
    x = S.generic((M, K), 1.0, seed=410 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=411 + bits + group, stream=N)
    qo = o.quantize(mode, w, bits=bits, group=group)
    qd = oracle_to_dev(bsfp, o, qo)
    y = from_dev(bsfp.qmv(to_dev(x), qd))
    yref, den = o.matmul_wonly(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= TOL, (e.max(), np.unravel_index(e.argmax(), e.shape))


@pytest.mark.parametrize("fmt", [(3, 8, 32), (0, 8, 64), (0, 4, 128)], ids=["mxfp8", "aff8g64", "aff4g128"])
@pytest.mark.parametrize("N,K", [(25600, 5120), (5120, 25600)])
def test_variant_qmv_decode_shapes(oracle_mod, bsfp, fmt, N, K):
    """The decode GEMV at the MLP projection shapes (M = 1)."""
    o = oracle_mod
    mode, bits, group = fmt
    x = S.generic((1, K), 1.0, seed=420, stream=K)
    w = S.generic((N, K), 0.02, seed=421, stream=N)
    qo = o.quantize(mode, w, bits=bits, group=group)
    y = from_dev(bsfp.qmv(to_dev(x), oracle_to_dev(bsfp, o, qo)))
    yref, den = o.matmul_wonly(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= TOL, e.max()


@pytest.mark.parametrize("fmt", VARIANTS, ids=IDS)
@pytest.mark.parametrize("M,N,K", [(37, 300, 320 * 4), (300, 513, 1280)])
def test_variant_dense_path(oracle_mod, bsfp, fmt, M, N, K):
    o = oracle_mod
    mode, bits, group = fmt
    x = S.generic((M, K), 1.0, seed=430 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=431 + bits, stream=group)
    qo = o.quantize(mode, w, bits=bits, group=group)
    y = from_dev(bsfp.qmm_dense(to_dev(x), oracle_to_dev(bsfp, o, qo)))
    yref, den = o.matmul_dense(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= QQ_TOL, (e.max(), np.unravel_index(e.argmax(), e.shape))


def test_variant_fused_qmm_points_to_dense(bsfp):
    x = to_dev(S.generic((16, 256), 1.0, seed=1))
    q = bsfp.quantize(to_dev(S.generic((64, 256), 0.02, seed=2)), 0, bits=8, group=32)
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm(x, q)
    assert ei.value.status == 2 and "bsfp_qmm_dense" in str(ei.value)


@pytest.mark.parametrize("M", [1, 3])
def test_variant_qmv_ragged_nan_codes_stay_in_their_row(oracle_mod, bsfp, M):
    """MXFP8 at K = 2880 (90 chunks of 32, not whole 32-chunk steps): the
    lanes past a row's last chunk load the next row's first codes.  With
    E4M3 NaN bytes (0x7F) planted in the first 6 chunks of every odd row,
    every even row must still match the oracle (a format's NaN code is data
    the contract accepts; it may only reach its own row)."""
    o = oracle_mod
    K, N = 2880, 64
    x = S.generic((M, K), 1.0, seed=440 + M)
    w = S.generic((N, K), 0.02, seed=441)
    qo = o.quantize(3, w)
    codes = qo.codes.copy()
    codes[1::2, :48] = 0x7F7F7F7F  # 192 code bytes = 6 chunks of 32 elements
    qo.codes = codes
    y = from_dev(bsfp.qmv(to_dev(x), oracle_to_dev(bsfp, o, qo)))
    yref, den = o.matmul_wonly(x, qo)
    ye, re, de = y[:, 0::2], yref[:, 0::2], den[:, 0::2]
    assert np.all(np.isfinite(re))
    e = o.norm_err(ye, re, de)
    assert e.max() <= TOL, (e.max(), np.unravel_index(e.argmax(), e.shape))
