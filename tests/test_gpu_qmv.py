"""GPU parity: decode GEMV (bsfp_qmv) against the oracle's fp64 product.

Bar: normalized error |y - y_ref| / sum_k |x_k w_k| <= 3e-3 (the pages'
~3e-3 relative bf16 tolerance against a dequantized f32 reference,
"feat(quant): backend quantization capability table ...", 2026-09-29
update).  Derivation for this path: bf16 output rounding contributes at most
2^-9 (1.95e-3) and fp32 accumulation over K <= 25600 well under 1e-3.
One-hot cases pin indexing exactly."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import from_dev, oracle_to_dev, to_dev

pytestmark = pytest.mark.gpu
TOL = 3e-3


def run_qmv(o, b, x_bits, qo):
    qd = oracle_to_dev(b, o, qo)
    y = b.qmv(to_dev(x_bits), qd)
    torch.cuda.synchronize()
    return from_dev(y)


def check(o, b, x_bits, qo, tol=TOL):
    y = run_qmv(o, b, x_bits, qo)
    yref, den = o.matmul_wonly(x_bits, qo)
    e = o.norm_err(y, yref, den)
    assert np.isfinite(e).all()
    assert e.max() <= tol, (e.max(), np.unravel_index(e.argmax(), e.shape))
    return e


def test_affine_small_config(oracle_mod, bsfp):
    x, w = S.affine_small()
    e = check(oracle_mod, bsfp, x, oracle_mod.quantize(0, w))
    assert e.max() <= 2 ** -8


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("N,K", [(37, 64 * 5), (300, 2880), (129, 5120), (17, 64 * 201)])
def test_qmv_ragged(oracle_mod, bsfp, mode, M, N, K):
    if mode == 1 and K % 32:
        pytest.skip("K must be a multiple of 32")
    x = S.generic((M, K), 1.0, seed=300 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=301 + mode, stream=N)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M", [4, 8])
@pytest.mark.parametrize("N,K", [(4200, 320), (4096, 1024), (8200, 448)])
def test_mma_gemv_launch_shapes(oracle_mod, bsfp, mode, M, N, K):
    """Several rows of x on the MFMA GEMV, on the launch shapes its rule
    picks for small matrices (256 CUs): N = 4200 (32-row workgroups, one per
    CU, the last with 8 rows), N = 4096 (one 16-row workgroup per CU) and
    N = 8200 (16-row workgroups, up to three per CU, the last with 8 rows);
    K with a partial last 128-element block (320, 448) and without (1024)."""
    if mode == 0 and K % 64:
        pytest.skip("affine K must be a multiple of 64")
    x = S.generic((M, K), 1.0, seed=420 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=421 + mode, stream=N)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_qmv_many_blocks_per_wave(oracle_mod, bsfp, mode):
    """A tall matrix (N = 40001, K = 2048): with two rows per team every wave
    walks three or more row blocks, so the staged block scales cycle through
    both of a wave's LDS buffers more than once; the last block is one row."""
    x = S.generic((1, 2048), 1.0, seed=410)
    w = S.generic((40001, 2048), 0.02, seed=411 + mode)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


def test_nvfp4_k_not_multiple_of_32(oracle_mod, bsfp):
    for M in (1, 4, 6):
        for K in (16, 48, 16 * 33):
            x = S.generic((M, K), 1.0, seed=K)
            w = S.generic((70, K), 0.02, seed=K + 1)
            check(oracle_mod, bsfp, x, oracle_mod.quantize(2, w))


def test_nvfp4_without_global_scale(oracle_mod, bsfp):
    x = S.generic((2, 1024), 1.0, seed=5)
    w = S.generic((100, 1024), 0.02, seed=6)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(2, w, use_global=False))


@pytest.mark.parametrize("which", ["up", "down"])
def test_affine_decode_full_size(oracle_mod, bsfp, which):
    x, w = S.affine_decode(which)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(0, w))


@pytest.mark.parametrize("M", [1, 8])
def test_mxfp4_config_full_size(oracle_mod, bsfp, M):
    w = S.mxfp4_weights()
    x = S.mxfp4_activations(M)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(1, w))


def test_nvfp4_prefill_weight_decode(oracle_mod, bsfp):
    x = S.generic((1, 5120), 1.0, seed=8)
    _, w = S.nvfp4_prefill(M=1, N=4096)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(2, w))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_onehot_activations_select_columns(oracle_mod, bsfp, mode):
    """x = e_j: y[n] = bf16(w_hat[n, j]) (bit-exact for MXFP4 and for NVFP4
    with a power-of-two global scale; at most one bf16 step otherwise)."""
    o = oracle_mod
    K, N = 64 * 9, 77
    w = S.generic((N, K), 0.02, seed=400 + mode)
    qo = o.quantize(mode, w, use_global=False) if mode == 2 else o.quantize(mode, w)
    B = o.dequant_exact(qo)
    for j in (0, 1, 5, 8, 31, 32, 100, K - 1):
        x = np.zeros((1, K), np.uint16)
        x[0, j] = 0x3F80
        y = o.bf16_to_f32(run_qmv(o, bsfp, x, qo)[0]).astype(np.float64)
        ref = o.bf16_to_f32(o.bf16_from_f64(B[:, j])).astype(np.float64)
        if mode == 0:
            assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -7 + 1e-30), j
        else:
            assert np.array_equal(y, ref), j


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_onehot_weights_select_activations(oracle_mod, bsfp, mode):
    """Each weight row holds one 1.0 (unit scales): y[m, n] = x[m, j_n]."""
    o = oracle_mod
    K, N, M = 64 * 6, 50, 3
    rng = np.random.default_rng(60 + mode)
    j = rng.integers(0, K, N)
    x = S.generic((M, K), 1.0, seed=61 + mode)
    codes = np.zeros((N, K), np.int64)
    if mode == 0:
        codes[np.arange(N), j] = 1
        scales = np.full((N, K // 64), 0x3F80, np.uint16)
        biases = np.zeros((N, K // 64), np.uint16)
    else:
        codes[np.arange(N), j] = 2
        scales = np.full((N, K // o.GROUP[mode]), 127 if mode == 1 else 0x38, np.uint8)
        biases = None
    wd = np.zeros((N, K // 8), np.uint32)
    for k in range(8):
        wd |= codes[:, k::8].astype(np.uint32) << (4 * k)
    qo = o.QTensor(mode, N, K, wd, scales, biases, None)
    y = run_qmv(o, bsfp, x, qo)
    assert np.array_equal(o.bf16_to_f32(y), o.bf16_to_f32(x[:, j]))


def test_qmv_deterministic(bsfp):
    x = to_dev(S.generic((1, 5120), 1.0, seed=1))
    w = to_dev(S.generic((4096, 5120), 0.02, seed=2))
    for mode in (0, 1, 2):
        q = bsfp.quantize(w, mode)
        a = bsfp.qmv(x, q)
        b2 = bsfp.qmv(x, q)
        assert torch.equal(a, b2)


def test_launch_event_hook_times_the_gemv(bsfp):
    """bsfp_time_next_launch: the events bracket the GEMV kernel of the next
    call only, and the result is the same as without the hook."""
    import ctypes as C
    rt = C.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    rt.hipEventDestroy.argtypes = [C.c_void_p]
    ev = [C.c_void_p(), C.c_void_p()]
    for e in ev:
        assert rt.hipEventCreate(C.byref(e)) == 0
    x = to_dev(S.generic((1, 5120), 1.0, seed=3))
    q = bsfp.quantize(to_dev(S.generic((8192, 5120), 0.02, seed=4)), 0)
    ref = bsfp.qmv(x, q)
    bsfp.time_next_launch(ev[0].value, ev[1].value)
    y = bsfp.qmv(x, q)
    y2 = bsfp.qmv(x, q)  # one-shot: this launch is not timed
    torch.cuda.synchronize()
    ms = C.c_float()
    assert rt.hipEventElapsedTime(C.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 100.0
    assert torch.equal(y, ref) and torch.equal(y2, ref)
    bsfp.time_next_launch(None, None)
    for e in ev:
        rt.hipEventDestroy(e)


# One row of x against matrices with few, long rows (16 or 25 steps of 32
# chunks per row), and the full [5120, 25600] down projection in every base
# format.
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,K", [(1000, 16384), (700, 25600), (5120, 25600)])
def test_qmv_long_rows(oracle_mod, bsfp, mode, N, K):
    x = S.generic((1, K), 1.0, seed=470, stream=K)
    w = S.generic((N, K), 0.02, seed=471 + mode, stream=N)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("mode", [1, 2])
def test_onehot_activations_long_rows(oracle_mod, bsfp, mode):
    """x = e_j with K = 8192 (8 steps per row), N = 77: y[n] = bf16(w_hat[n, j])
    exactly, for j at both ends of several steps."""
    o = oracle_mod
    K, N = 8192, 77
    w = S.generic((N, K), 0.02, seed=480 + mode)
    qo = o.quantize(mode, w, use_global=False) if mode == 2 else o.quantize(mode, w)
    B = o.dequant_exact(qo)
    for j in (0, 31, 1023, 1024, 2047, 2048, 3100, K - 1025, K - 1):
        x = np.zeros((1, K), np.uint16)
        x[0, j] = 0x3F80
        y = o.bf16_to_f32(run_qmv(o, bsfp, x, qo)[0]).astype(np.float64)
        ref = o.bf16_to_f32(o.bf16_from_f64(B[:, j])).astype(np.float64)
        assert np.array_equal(y, ref), j


@pytest.mark.parametrize("mode", [1, 2])
def test_qq_decode_long_rows(oracle_mod, bsfp, mode):
    """The qq decode GEMV (x quantized while staged) with 25 steps per row."""
    from test_gpu_qmm import check_qq
    x = S.generic((1, 25600), 1.0, seed=490, stream=mode)
    w = S.generic((700, 25600), 0.02, seed=491 + mode)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


# Where x exceeds the 64 KB LDS copy of the other kernels (from 4 rows of x),
# and from 5 rows on matrices under 2^26 weights, the GEMV runs on MFMA (x as
# the A operand, 16 weight rows dequantized in registers as the B operand).
# At hidden 5120 eight rows of x (80 KB) take the MFMA kernel and six stay
# with the LDS kernels; at K = 25600 all three counts take the MFMA kernel.
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M", [4, 6, 8])
def test_qmv_rows_decode_shapes(oracle_mod, bsfp, mode, M):
    for N, K, which in ((25600, 5120, 0), (5120, 25600, 1)):
        x = S.generic((M, K), 1.0, seed=495 + M, stream=K)
        w = S.generic((N, K), 0.02, seed=496 + mode, stream=which)
        check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_onehot_activations_rows(oracle_mod, bsfp, mode):
    """Eight rows of x, row m = e_{j_m}: y[m, n] = bf16(w_hat[n, j_m]) on the
    MFMA GEMV (exact for MXFP4 and NVFP4 without a global scale; one bf16 step
    for affine), for j at chunk and block edges and past 128-element blocks."""
    o = oracle_mod
    K, N, M = 64 * 13, 70, 8
    w = S.generic((N, K), 0.02, seed=497 + mode)
    qo = o.quantize(mode, w, use_global=False) if mode == 2 else o.quantize(mode, w)
    B = o.dequant_exact(qo)
    j = np.array([0, 7, 8, 31, 32, 127, 128, K - 1])
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), j] = 0x3F80
    y = o.bf16_to_f32(run_qmv(o, bsfp, x, qo)).astype(np.float64)
    ref = o.bf16_to_f32(o.bf16_from_f64(B[:, j].T)).astype(np.float64)
    if mode == 0:
        assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -7 + 1e-30)
    else:
        assert np.array_equal(y, ref)


# Several matrices that share x (bsfp_qmv_batch): one launch of the fast
# kernel with rows of every matrix dealt over the CUs together.  Each row is
# computed as bsfp_qmv computes it, so the outputs equal separate calls bit
# for bit, and meet the oracle bar.
def check_batch(o, b, x_bits, qos):
    qds = [oracle_to_dev(b, o, qo) for qo in qos]
    xd = to_dev(x_bits)
    ys = b.qmv_batch(xd, qds)
    singles = [b.qmv(xd, qd) for qd in qds]
    torch.cuda.synchronize()
    for y, y1, qo in zip(ys, singles, qos):
        assert torch.equal(y, y1)
        if y.numel() == 0:
            continue
        yref, den = o.matmul_wonly(x_bits, qo)
        e = o.norm_err(from_dev(y), yref, den)
        assert np.isfinite(e).all() and e.max() <= TOL, e.max()


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_qmv_batch_ragged_matrices(oracle_mod, bsfp, mode):
    """Row counts that end in partial blocks, 2 to 4 matrices; NVFP4 with a
    different global scale per matrix (weights of different spread)."""
    o = oracle_mod
    K = 4096
    x = S.generic((1, K), 1.0, seed=800, stream=mode)
    qos = [o.quantize(mode, S.generic((n, K), sd, seed=801 + i, stream=mode))
           for i, (n, sd) in enumerate([(96, 0.02), (37, 0.05), (200, 0.01), (3, 0.03)])]
    check_batch(o, bsfp, x, qos[:2])
    check_batch(o, bsfp, x, qos)


def test_qmv_batch_skips_empty_matrices(oracle_mod, bsfp):
    o = oracle_mod
    K = 4096
    x = S.generic((1, K), 1.0, seed=810)
    qos = [o.quantize(2, S.generic((n, K), 0.02, seed=811 + n)) for n in (64, 0, 130)]
    check_batch(o, bsfp, x, qos)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_qmv_batch_gate_up_full_size(oracle_mod, bsfp, mode):
    """The decode gate and up projections at hidden 5120: two [25600, 5120]
    matrices in one launch (51200 rows: four rows per team)."""
    o = oracle_mod
    x = S.generic((1, 5120), 1.0, seed=820)
    qos = [o.quantize(mode, S.generic((25600, 5120), 0.02, seed=821 + i)) for i in range(2)]
    check_batch(o, bsfp, x, qos)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_qmv_batch_four_rows_per_team_ragged(oracle_mod, bsfp, mode):
    """A batch of 33006 rows (four rows per team, blocks of 8 rows) whose
    three matrices all end in a partial block: 20001, 13000 and 5 rows."""
    o = oracle_mod
    K = 2048
    x = S.generic((1, K), 1.0, seed=840, stream=mode)
    qos = [o.quantize(mode, S.generic((n, K), 0.02, seed=841 + i, stream=mode))
           for i, n in enumerate((20001, 13000, 5))]
    check_batch(o, bsfp, x, qos)


@pytest.mark.parametrize("M", [2, 8])
def test_qmv_batch_several_rows_of_x(oracle_mod, bsfp, M):
    """With several rows of x the matrices run one launch each: same results
    as separate calls."""
    o = oracle_mod
    x = S.generic((M, 2048), 1.0, seed=830 + M)
    qos = [o.quantize(1, S.generic((n, 2048), 0.02, seed=831 + n)) for n in (70, 33)]
    check_batch(o, bsfp, x, qos)


@pytest.mark.parametrize("case", ["mxfp8", "affine8_g32", "nvfp4_k_odd"])
def test_qmv_batch_fallback_paths(oracle_mod, bsfp, case):
    """Formats and shapes the matrix list does not take run one launch per
    matrix: a format variant, and NVFP4 rows with K % 32 == 16."""
    o = oracle_mod
    K = 1040 if case == "nvfp4_k_odd" else 2048
    x = S.generic((1, K), 1.0, seed=840, stream=K)
    ws = [S.generic((n, K), 0.02, seed=841 + n) for n in (64, 45)]
    if case == "mxfp8":
        qos = [o.quantize(o.MXFP8, w) for w in ws]
    elif case == "affine8_g32":
        qos = [o.quantize(o.AFFINE, w, bits=8, group=32) for w in ws]
    else:
        qos = [o.quantize(2, w) for w in ws]
    check_batch(o, bsfp, x, qos)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,K", [(200, 6144), (129, 5120), (77, 7168)])
def test_qmv_step_counts(oracle_mod, bsfp, mode, N, K):
    """One row of x with staged scales, rows of 5, 6 and 7 steps of 1024
    elements on matrices with few rows per CU."""
    x = S.generic((1, K), 1.0, seed=850 + K, stream=mode)
    w = S.generic((N, K), 0.02, seed=851 + N, stream=mode)
    check(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))
