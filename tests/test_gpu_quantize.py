"""GPU parity: amax, quantize and dequantize through the C ABI against the
oracle.  The bar is bit-exact codes, scales, global scale and dequantized
values (the pages' own test design: GPU quantize bit-identical to the CPU
quantizer at 4096x4096, "feat(quant): backend quantization capability table
...", the 2026-09-29 update)."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import from_dev, qt_to_oracle, to_dev, u8, words

pytestmark = pytest.mark.gpu

MODES = [0, 1, 2]


def check_quant_exact(o, b, x_bits, mode, gs="compute", g=None):
    xd = to_dev(x_bits)
    gd = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    q = b.quantize(xd, mode, global_scale=gs, g=gd)
    if mode == o.NVFP4:
        qo = o.quantize(mode, x_bits, use_global=(gs != "none"), g=g)
    else:
        qo = o.quantize(mode, x_bits)
    torch.cuda.synchronize()
    assert np.array_equal(words(q.codes), qo.codes), "codes differ"
    if mode == o.AFFINE:
        assert np.array_equal(from_dev(q.scales), qo.scales)
        assert np.array_equal(from_dev(q.biases), qo.biases)
    else:
        assert np.array_equal(u8(q.scales), qo.scales), "scales differ"
    if mode == o.NVFP4 and gs != "none":
        assert q.global_scale.item() == qo.g
        if gs == "compute":
            assert q.amax.item() == qo.amax
    # dequantize, bit-exact
    dq = from_dev(b.dequantize(q))
    assert np.array_equal(dq, o.dequantize(qo)), "dequantized values differ"
    return q, qo


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 64), (37, 64 * 13), (3, 2880), (129, 5120)])
def test_quantize_ragged_shapes(oracle_mod, bsfp, mode, shape):
    x = S.generic(shape, 1.5, seed=200 + mode, stream=shape[0])
    check_quant_exact(oracle_mod, bsfp, x, mode)


def test_nvfp4_activation_config_bit_exact(oracle_mod, bsfp):
    """X[4096,5120] ~ N(0,1) with 1 % outliers at +-20: codes, scales, g and
    amax bit-exact; the dequantization round trip bit-exact too."""
    x = S.nvfp4_activations()
    q, qo = check_quant_exact(oracle_mod, bsfp, x, oracle_mod.NVFP4)
    assert qo.amax == np.float32(20.0)


def _nvfp4_compute(b, xd, ws, rbits=None):
    """NVFP4 quantize with the global scale computed: through bsfp_quantize_ws
    when ws is a workspace tensor, through bsfp_quantize(_sr) when ws is None."""
    q = b.empty_quantized(b.NVFP4, xd.shape[0], xd.shape[1], xd.device)
    q.scratch = ws
    return b.quantize(xd, b.NVFP4, out=q, rbits=rbits)


@pytest.mark.parametrize("shape", [(1, 16), (37, 64 * 13), (4096, 5120)])
def test_nvfp4_compute_with_and_without_workspace(oracle_mod, bsfp, shape):
    """The two-launch path (partial maxima in a caller workspace, whose stale
    contents must not matter) and the three-launch path (zeroed atomic
    accumulator) give the oracle's codes, scales, g and amax, bit for bit, with
    nearest and with stochastic rounding."""
    o = oracle_mod
    x = S.nvfp4_activations(*shape, seed=220) if shape[0] > 1 else S.generic(shape, 1.0, seed=220)
    r = S.random_words(shape, seed=221)
    xd = to_dev(x)
    rd = torch.from_numpy(np.ascontiguousarray(r).view(np.int32)).to("cuda")
    ws = torch.full((bsfp.QUANTIZE_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")  # NaNs
    for rbits, words_r in ((None, None), (rd, r)):
        qo = o.quantize(o.NVFP4, x, use_global=True, rbits=words_r)
        for w in (ws, None):
            q = _nvfp4_compute(bsfp, xd, w, rbits)
            torch.cuda.synchronize()
            tag = ("workspace" if w is not None else "atomic") + (" sr" if rbits is not None else "")
            assert np.array_equal(words(q.codes), qo.codes), tag
            assert np.array_equal(u8(q.scales), qo.scales), tag
            assert q.amax.item() == qo.amax and q.global_scale.item() == qo.g, tag
            ws.fill_(0xFF)


@pytest.mark.parametrize("shape", [(3, 48), (512, 5120), (1134, 5120), (2048, 5120),
                                   (4096, 8192), (4112, 8192)])
def test_nvfp4_compute_workspace_shapes(oracle_mod, bsfp, shape):
    """More shapes for the workspace path (partial maxima from one workgroup
    per CU, then the quantize over a capped grid): a single 48-element row,
    1 to 16 packed words per amax lane on 256 CUs, and a tensor of 33.7 M
    elements.  Codes, scales, g and amax are bit-exact against the oracle,
    and so is the atomic path."""
    o = oracle_mod
    x = S.nvfp4_activations(*shape, seed=230 + shape[0])
    xd = to_dev(x)
    ws = torch.full((bsfp.QUANTIZE_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")  # NaNs
    qo = o.quantize(o.NVFP4, x, use_global=True)
    for w in (ws, None):
        q = _nvfp4_compute(bsfp, xd, w, None)
        torch.cuda.synchronize()
        tag = "workspace" if w is not None else "atomic"
        assert np.array_equal(words(q.codes), qo.codes), tag
        assert np.array_equal(u8(q.scales), qo.scales), tag
        assert q.amax.item() == qo.amax and q.global_scale.item() == qo.g, tag


def test_nvfp4_workspace_amax_planted_anywhere(bsfp):
    """One element of magnitude 7.5 among values of magnitude <= 3.5, at the
    first element, the middle, in the last workgroup's share and at the last
    element: the workspace path's amax is exactly 7.5 and g = 7.5/2688."""
    rows, cols = 4096, 5120
    n = rows * cols
    base = S.generic((n,), 1.0, seed=78)
    base = (base & 0x8000) | np.minimum(base & 0x7FFF, 0x4060)
    ws = torch.empty(bsfp.QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    for pos in (0, n // 2 + 3, n - 4099, n - 1):
        x = base.copy()
        x[pos] = 0xC0F0  # bf16 -7.5
        q = _nvfp4_compute(bsfp, to_dev(x.reshape(rows, cols)), ws)
        assert q.amax.item() == 7.5, pos
        assert q.global_scale.item() == np.float32(np.float32(7.5) / np.float32(2688.0)), pos


def test_nvfp4_given_and_no_global_scale(oracle_mod, bsfp):
    x = S.generic((64, 1024), 0.02, seed=210)
    check_quant_exact(oracle_mod, bsfp, x, oracle_mod.NVFP4, gs="given", g=3.7e-5)
    check_quant_exact(oracle_mod, bsfp, x, oracle_mod.NVFP4, gs="given", g=1e-9)  # saturating
    check_quant_exact(oracle_mod, bsfp, x, oracle_mod.NVFP4, gs="none")


def test_mxfp4_weight_config_bit_exact(oracle_mod, bsfp):
    check_quant_exact(oracle_mod, bsfp, S.mxfp4_weights(), oracle_mod.MXFP4)


def test_affine_weight_configs_bit_exact(oracle_mod, bsfp):
    _, w = S.affine_small()
    check_quant_exact(oracle_mod, bsfp, w, oracle_mod.AFFINE)
    _, w = S.affine_decode("up")
    check_quant_exact(oracle_mod, bsfp, w, oracle_mod.AFFINE)


def _all_bf16_blocks():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(f) & (np.abs(f) < 1e36)]
    n = (bits.size // 64) * 64
    return bits[:n].reshape(-1, 64)


@pytest.mark.parametrize("mode", MODES)
def test_every_bf16_value(oracle_mod, bsfp, mode):
    """All finite bf16 values (|x| < 1e36, so affine ranges stay finite), in
    order and shuffled, through each quantizer."""
    x = _all_bf16_blocks()
    check_quant_exact(oracle_mod, bsfp, x, mode, gs="none" if mode == 2 else "compute")
    rng = np.random.default_rng(5)
    xs = rng.permutation(x.reshape(-1)).reshape(x.shape)
    check_quant_exact(oracle_mod, bsfp, xs, mode)


@pytest.mark.parametrize("mode", MODES)
def test_threshold_neighbourhoods(oracle_mod, bsfp, mode):
    """Blocks whose scaled values sit on and next to every E2M1 decision
    boundary (NVFP4 with g = 1 and MXFP4: the block max fixes the scale)."""
    o = oracle_mod
    rng = np.random.default_rng(77 + mode)
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rows = []
    G = o.GROUP[mode]
    for _ in range(64):
        scale = float(2.0 ** rng.integers(-6, 6))
        v = rng.choice(bounds, G) * scale
        v *= rng.choice([1 - 2 ** -7, 1.0, 1 + 2 ** -7], G)
        v *= rng.choice([-1.0, 1.0], G)
        v[0] = 6.0 * scale  # block max: NVFP4 scale 1*scale... exact E4M3
        rows.append(v)
    x = S.to_bf16_bits(np.array(rows, np.float32).reshape(-1, 64))
    check_quant_exact(o, bsfp, x, mode, gs="none" if mode == 2 else "compute")


def test_zero_and_tiny_tensors(oracle_mod, bsfp):
    o = oracle_mod
    for mode in MODES:
        z = np.zeros((3, o.GROUP[mode] * 2), np.uint16)
        check_quant_exact(o, bsfp, z, mode)
    z = np.zeros((2, 64), np.uint16)
    z[0, 5] = 0x8000  # -0
    check_quant_exact(o, bsfp, z, o.NVFP4)
    # a tensor so small that it is one group
    check_quant_exact(o, bsfp, S.generic((1, 16), 1.0, seed=3), o.NVFP4)
    check_quant_exact(o, bsfp, S.generic((1, 32), 1.0, seed=3), o.MXFP4)


def test_empty_tensor(bsfp):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    for mode in MODES:
        q = bsfp.quantize(x, mode)
        assert q.codes.numel() == 0
        assert bsfp.dequantize(q).numel() == 0


def test_amax_matches_oracle(oracle_mod, bsfp):
    for n in (1, 7, 8, 9, 1000, 4096 * 5120 + 5):
        x = S.generic((n,), 2.0, seed=n % 1000)
        got = bsfp.amax(to_dev(x)).item()
        assert got == oracle_mod.amax(x), n
    assert bsfp.amax(torch.zeros(0, dtype=torch.bfloat16, device="cuda")).item() == 0.0


@pytest.mark.gpu
def test_amax_planted_maximum_anywhere(oracle_mod, bsfp):
    """One element of magnitude 7.5 (negative) among N(0,1) values, planted at
    the start, the middle, the last whole 8-element word, the n % 8 tail and
    the end; amax must be exactly 7.5 wherever it sits, also on repeated calls
    into a buffer that already holds a larger stale value."""
    n = 4096 * 5120 + 5
    base = S.generic((n,), 1.0, seed=77)
    base = (base & 0x8000) | np.minimum(base & 0x7FFF, 0x4060)  # |x| <= 3.5 (bf16 bits)
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    for pos in (0, n // 2 + 3, (n // 8) * 8 - 1, n - 3, n - 1):
        x = base.copy()
        x[pos] = 0xC0F0  # bf16 -7.5
        out.fill_(1000.0)
        got = bsfp.amax(to_dev(x), out=out).item()
        assert got == 7.5 == oracle_mod.amax(x), pos


def test_quantize_is_deterministic(bsfp):
    x = to_dev(S.nvfp4_activations(512, 5120, seed=9))
    a = bsfp.quantize(x, 2)
    b2 = bsfp.quantize(x, 2)
    assert torch.equal(a.codes, b2.codes) and torch.equal(a.scales, b2.scales)


# ------------------------------------------------- stochastic rounding (SR)
# The random words are inputs, drawn by the seeded input module and handed
# to both sides, so codes and scales must be bit-exact.

def check_sr_exact(o, b, x_bits, mode, r, gs="compute", g=None):
    xd = to_dev(x_bits)
    rd = torch.from_numpy(np.ascontiguousarray(r).view(np.int32)).to("cuda")
    gd = None if g is None else torch.tensor([g], dtype=torch.float32, device="cuda")
    q = b.quantize(xd, mode, global_scale=gs, g=gd, rbits=rd)
    if mode == o.NVFP4:
        qo = o.quantize(mode, x_bits, use_global=(gs != "none"), g=g, rbits=r)
    else:
        qo = o.quantize(mode, x_bits, rbits=r)
    torch.cuda.synchronize()
    assert np.array_equal(words(q.codes), qo.codes), "codes differ"
    assert np.array_equal(u8(q.scales), qo.scales), "scales differ"
    if mode == o.NVFP4 and gs != "none":
        assert q.global_scale.item() == qo.g
    return q, qo


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("shape", [(1, 64), (37, 64 * 13), (3, 2880), (129, 5120)])
def test_sr_ragged_shapes(oracle_mod, bsfp, mode, shape):
    x = S.generic(shape, 1.5, seed=300 + mode, stream=shape[0])
    r = S.random_words(shape, seed=301 + mode, stream=shape[0])
    check_sr_exact(oracle_mod, bsfp, x, mode, r)


def test_sr_nvfp4_global_scale_variants(oracle_mod, bsfp):
    o = oracle_mod
    x = S.generic((64, 1024), 0.02, seed=310)
    r = S.random_words((64, 1024), seed=311)
    check_sr_exact(o, bsfp, x, o.NVFP4, r, gs="given", g=3.7e-5)
    check_sr_exact(o, bsfp, x, o.NVFP4, r, gs="none")


@pytest.mark.parametrize("mode", [1, 2])
def test_sr_every_bf16_value_and_extreme_words(oracle_mod, bsfp, mode):
    """All finite bf16 values through the SR quantizer with random words, with
    all-zero words (round up) and with all-one words (round down)."""
    o = oracle_mod
    x = _all_bf16_blocks()
    gs = "none" if mode == 2 else "compute"
    for r in (S.random_words(x.shape, seed=320 + mode),
              np.zeros(x.shape, np.uint32), np.full(x.shape, 0xFFFFFFFF, np.uint32)):
        check_sr_exact(o, bsfp, x, mode, r, gs=gs)


@pytest.mark.parametrize("mode", [1, 2])
def test_sr_threshold_neighbourhoods(oracle_mod, bsfp, mode):
    """Scaled values on, just below and just above every E2M1 grid value and
    midpoint, with words near the decision u = p."""
    o = oracle_mod
    rng = np.random.default_rng(330 + mode)
    pts = np.array([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0])
    rows = []
    G = o.GROUP[mode]
    for _ in range(64):
        scale = float(2.0 ** rng.integers(-6, 6))
        v = rng.choice(pts, G) * scale
        v *= rng.choice([1 - 2 ** -7, 1.0, 1 + 2 ** -7], G)
        v *= rng.choice([-1.0, 1.0], G)
        v[0] = 6.0 * scale
        rows.append(v)
    x = S.to_bf16_bits(np.array(rows, np.float32).reshape(-1, 64))
    r = (rng.integers(0, 1 << 24, x.shape, dtype=np.uint64) << 8).astype(np.uint32)
    r[:, ::3] = 0x80000000  # u = 1/2 exactly: the midpoints decide on u < p
    check_sr_exact(o, bsfp, x, mode, r, gs="none" if mode == 2 else "compute")


def test_sr_nvfp4_activation_config(oracle_mod, bsfp):
    """X[4096,5120] with 1 % outliers: SR codes bit-exact at full size."""
    x = S.nvfp4_activations()
    r = S.random_words(x.shape, seed=340)
    check_sr_exact(oracle_mod, bsfp, x, oracle_mod.NVFP4, r)


def test_sr_rejects_affine_and_bad_words(bsfp):
    x = to_dev(S.generic((4, 128), 1.0, seed=1))
    r = torch.zeros(4 * 128, dtype=torch.int32, device="cuda")
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.quantize(x, 0, rbits=r)
    assert ei.value.status == 2
    with pytest.raises(ValueError):
        bsfp.quantize(x, 2, rbits=r[:100])
