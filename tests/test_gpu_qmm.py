"""GPU parity: prefill GEMM (bsfp_qmm) against the oracle.

Bar: normalized error |y - y_ref| / sum_k |a_k b_k| <= 3e-3 with y_ref the
oracle's fp64 product (the pages' ~3e-3 relative bf16 tolerance against a
dequantized f32 reference, "feat(quant): backend quantization capability
table ...", 2026-09-29 update).  For the qq paths the dequantized operand
products are exact on the MFMA and only fp32 summation order and the final
bf16 rounding remain; the rounding is at most 2^-8 of |y|, and for the
independent x and w draws used here |y| stays far below sum_k |a_k b_k|, so
they are held to 2.2e-3.  (x and w from one random stream would make
|y| ~ sum_k |a_k b_k| on matching rows and the rounding alone could reach
3.9e-3 there.)  At the full prefill size the oracle computes sampled outputs
one by one."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import from_dev, oracle_to_dev, to_dev

pytestmark = pytest.mark.gpu
TOL = 3e-3
QQ_TOL = 2.2e-3


def qmm_dev(o, b, x_bits, qo, act):
    qd = oracle_to_dev(b, o, qo)
    y = b.qmm(to_dev(x_bits), qd, act=act)
    torch.cuda.synchronize()
    return from_dev(y)


def check_wonly(o, b, x, qo, tol=TOL):
    y = qmm_dev(o, b, x, qo, "bf16")
    yref, den = o.matmul_wonly(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= tol, (e.max(), np.unravel_index(e.argmax(), e.shape))
    return y


def check_qq(o, b, x, qo, tol=QQ_TOL):
    y = qmm_dev(o, b, x, qo, "same")
    yref, den, _, _ = o.matmul_qq(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= tol, (e.max(), np.unravel_index(e.argmax(), e.shape))
    return y


SHAPES = [(1, 70, 64), (37, 300, 320), (100, 385, 640), (130, 257, 1024), (300, 513, 5120 // 4)]


@pytest.mark.parametrize("M,K", [(9, 64), (130, 1024), (2048, 5120)])
def test_qq_nvfp4_workspace_amax_and_g(oracle_mod, bsfp, M, K):
    """The NVFP4 qq GEMM path leaves amax(x) and g_x = amax/2688 in the first
    two floats of its workspace (taken from per-workgroup partial maxima of
    |x|); both bit-exact against the oracle, also over a workspace that held
    garbage before the call."""
    x = S.generic((M, K), 1.0, seed=500 + M)
    x[M // 2, K // 3] = 0xC1A0  # bf16 -20: one outlier sets the maximum
    w = S.generic((96, K), 0.02, seed=501)
    qd = oracle_to_dev(bsfp, oracle_mod, oracle_mod.quantize(2, w))
    ws = torch.full((bsfp.qmm_workspace_bytes(2, M, K, "same"),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    bsfp.qmm(to_dev(x), qd, act="same", workspace=ws)
    torch.cuda.synchronize()
    head = ws[:8].cpu().numpy().view(np.float32)
    a = oracle_mod.amax(x)
    assert head[0] == a == np.float32(20.0)
    assert head[1] == oracle_mod.global_scale(a)


# Bytes before the fp16 activation operand in the NVFP4 qq workspace: amax
# and g_x (256 B), then 256 partial maxima.
NV_WS_HEAD = 256 + 256 * 4


@pytest.mark.parametrize("M", [9, 1134, 2048, 4096, 6553, 6600])
def test_qq_nvfp4_activation_operand_exact(oracle_mod, bsfp, M):
    """The NVFP4 qq GEMM's activation operand, E2M1(code) * E4M3(S) as fp16
    after the head of its workspace, equals the oracle's exact dequantization
    of q(x) without g, value for value, and the head holds the oracle's amax
    and g; from the smallest GEMM row count to 33.8 M elements."""
    o = oracle_mod
    K = 5120
    x = S.nvfp4_activations(M, K, seed=600 + M)
    w = S.generic((64, K), 0.02, seed=601)
    qd = oracle_to_dev(bsfp, o, o.quantize(2, w))
    ws = torch.full((bsfp.qmm_workspace_bytes(2, M, K, "same"),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    bsfp.qmm(to_dev(x), qd, act="same", workspace=ws)
    torch.cuda.synchronize()
    xhat = ws[NV_WS_HEAD:NV_WS_HEAD + M * K * 2].cpu().numpy().view(np.float16).reshape(M, K)
    qx = o.quantize(o.NVFP4, x, use_global=True)
    A = o.dequant_exact(qx, with_g=False)
    assert np.array_equal(xhat.astype(np.float64), A)
    head = ws[:8].cpu().numpy().view(np.float32)
    assert head[0] == qx.amax and head[1] == qx.g


def test_qq_nvfp4_graph_replay_matches_eager(oracle_mod, bsfp):
    """The NVFP4 qq call (activation amax partials, quantize, GEMM) captured
    in a HIP graph: three replays, with eager calls between them, each give
    the eager call's output bit for bit."""
    o = oracle_mod
    M, K, N = 1134, 5120, 512
    x = to_dev(S.nvfp4_activations(M, K, seed=610))
    qd = oracle_to_dev(bsfp, o, o.quantize(2, S.generic((N, K), 0.02, seed=611)))
    eager = bsfp.qmm(x, qd, act="same")
    ws = torch.empty(bsfp.qmm_workspace_bytes(2, M, K, "same"), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bsfp.qmm(x, qd, act="same", workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bsfp.qmm(x, qd, act="same", workspace=ws, out=out)
    for r in range(3):
        out.zero_()
        graph.replay()
        again = bsfp.qmm(x, qd, act="same")
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        assert torch.equal(again, eager), r


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_weight_only_ragged(oracle_mod, bsfp, mode, M, N, K):
    x = S.generic((M, K), 1.0, seed=500 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=501 + mode, stream=N)
    check_wonly(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_qq_ragged(oracle_mod, bsfp, mode, M, N, K):
    x = S.generic((M, K), 0.02, seed=600 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=601 + mode, stream=N)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


def test_qq_nvfp4_without_global_scale(oracle_mod, bsfp):
    x = S.generic((70, 512), 1.0, seed=9)
    w = S.generic((90, 512), 0.02, seed=10)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(2, w, use_global=False))


def test_qq_nvfp4_activation_outliers(oracle_mod, bsfp):
    """Activations with 1 % outliers at +-20 (the NVFP4 activation workload)."""
    x = S.nvfp4_activations(192, 5120, seed=11)
    _, w = S.nvfp4_prefill(M=1, N=384)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(2, w))


@pytest.mark.parametrize("M", [32, 200, 512, 2048])
def test_mxfp4_config_qq_full(oracle_mod, bsfp, M):
    w = S.mxfp4_weights()
    x = S.mxfp4_activations(M)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(1, w))


@pytest.mark.parametrize("M", [32, 512])
def test_mxfp4_config_weight_only_full(oracle_mod, bsfp, M):
    w = S.mxfp4_weights()
    x = S.mxfp4_activations(M)
    check_wonly(oracle_mod, bsfp, x, oracle_mod.quantize(1, w))


@pytest.mark.parametrize("M", [20, 100, 300])
@pytest.mark.parametrize("K", [384, 704, 768, 2880])
def test_mxfp4_qq_k_units(oracle_mod, bsfp, M, K):
    """MXFP4 x MXFP4 walks K in units of 256 plus one last unit of 64, 128
    or 192 (K % 256): every unit size, at the tile shapes of all three row
    ranges (up to 64, up to 256, beyond)."""
    x = S.generic((M, K), 0.02, seed=650 + M, stream=K)
    w = S.generic((300, K), 0.02, seed=651, stream=K)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(1, w))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_qq_decode_rows(oracle_mod, bsfp, mode, M):
    """M <= 8 runs the qq product as a GEMV on the exactly dequantized x (the
    qq decode path); same contract as the GEMM: alpha at every M."""
    x = S.generic((M, 2048), 1.0, seed=800 + M, stream=mode)
    w = S.generic((1000, 2048), 0.02, seed=801 + mode)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


def test_qq_decode_nvfp4_without_global_scale(oracle_mod, bsfp):
    """NVFP4 weights without a global scale: x is quantized with g = 1 too."""
    x = S.generic((3, 1024), 1.0, seed=810)
    w = S.generic((500, 1024), 0.02, seed=811)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(2, w, use_global=False))


@pytest.mark.parametrize("mode", [1, 2])
def test_qq_decode_x_beyond_gemv_lds(oracle_mod, bsfp, mode):
    """8 rows of K = 8192 (128 KB of x) exceed the GEMV's LDS copy of x: the
    quantize-dequantize runs as its own pass into the workspace first."""
    x = S.generic((8, 8192), 1.0, seed=820 + mode)
    w = S.generic((300, 8192), 0.02, seed=830)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("M", [1, 8])
def test_mxfp4_config_qq_decode(oracle_mod, bsfp, M):
    check_qq(oracle_mod, bsfp, S.mxfp4_activations(M), oracle_mod.quantize(1, S.mxfp4_weights()))


@pytest.mark.parametrize("mode", [1, 2])
def test_qq_decode_and_gemm_paths_agree(oracle_mod, bsfp, mode):
    """Rows 0..7 of a 9-row qq product (GEMM path) against the same 8 rows
    alone (decode path): both within tolerance of each other.  NVFP4's g_x
    comes from the whole x, so the 9th row is a copy of row 0 (same amax)."""
    o = oracle_mod
    x = S.generic((8, 1024), 1.0, seed=900, stream=mode)
    x9 = np.concatenate([x, x[:1]], axis=0)
    w = S.generic((600, 1024), 0.02, seed=901)
    qd = oracle_to_dev(bsfp, o, o.quantize(mode, w))
    a = o.bf16_to_f32(from_dev(bsfp.qmm(to_dev(x), qd, act="same"))).astype(np.float64)
    c = o.bf16_to_f32(from_dev(bsfp.qmm(to_dev(x9), qd, act="same"))[:8]).astype(np.float64)
    _, den, _, _ = o.matmul_qq(x, o.quantize(mode, w))
    assert np.max(np.abs(a - c) / den) <= 2 * QQ_TOL


# Full-size prefill checks sample 64 whole output rows plus 4096 random
# (m, n) outputs; the oracle computes each one on its own.
N_ROWS, N_PAIRS = 64, 4096


def _sample_pairs(M, N, seed, n_rows=N_ROWS, n_pairs=N_PAIRS):
    rng = np.random.default_rng(seed)
    rows = rng.choice(M, n_rows, replace=False)
    ai = np.concatenate([np.repeat(rows, N), rng.integers(0, M, n_pairs)])
    bi = np.concatenate([np.tile(np.arange(N), n_rows), rng.integers(0, N, n_pairs)])
    return ai, bi


def _sampled_qq(o, b, M, N, K, seed, x=None, w=None):
    if x is None:
        x, w = S.nvfp4_prefill(M=M, N=N, K=K, seed=seed)
    qo = o.quantize(2, w)
    y = qmm_dev(o, b, x, qo, "same")
    qx = o.quantize(2, x)  # alpha needs the full-tensor g_x
    alpha = o.alpha(qx.g, qo.g)
    a_rows, bi = _sample_pairs(M, N, seed)
    uniq_a, inv_a = np.unique(a_rows, return_inverse=True)
    uniq_b, inv_b = np.unique(bi, return_inverse=True)
    A = o.dequant_exact(qx, with_g=False, rows=uniq_a)
    B = o.dequant_exact(qo, with_g=False, rows=uniq_b)
    yref, den = o.matmul_pairs(A, B, inv_a, inv_b, float(alpha))
    got = y[a_rows, bi]
    e = o.norm_err(got, yref, den)
    return e


def _sampled_wonly(o, b, x, qo, seed):
    M, N = x.shape[0], qo.rows
    y = qmm_dev(o, b, x, qo, "bf16")
    ai, bi = _sample_pairs(M, N, seed)
    ua, ia = np.unique(ai, return_inverse=True)
    ub, ib = np.unique(bi, return_inverse=True)
    A = o.bf16_to_f64(x[ua])
    B = o.dequant_exact(qo, rows=ub)
    yref, den = o.matmul_pairs(A, B, ia, ib)
    return o.norm_err(y[ai, bi], yref, den)


@pytest.mark.parametrize("M", [100, 200, 1134, 2048, 4096])
def test_nvfp4_prefill_qq_sampled_full_size(oracle_mod, bsfp, M):
    """X[M,5120] x W[25600,5120]^T at full size: 64 full output rows plus
    4096 random outputs computed one by one by the oracle.  At M = 2048 and
    4096 the last 1024 output columns come from the second (small-tile)
    launch; the full rows cover them.  M = 100 and 200 run the tiles 128
    columns wide (128 x 128 and 256 x 128, partial in M)."""
    e = _sampled_qq(oracle_mod, bsfp, M, 25600, 5120, seed=5)
    assert e.max() <= QQ_TOL, e.max()


@pytest.mark.parametrize("M", [200, 1134, 2048, 4096])
def test_nvfp4_prefill_weight_only_sampled_full_size(oracle_mod, bsfp, M):
    """NVFP4 weight-only x[M,5120] . W[25600,5120]^T (bf16 x, W's global
    scale applied to the fp32 sums) at full size, sampled as above.  At
    M = 2048 and 4096 on 256 CUs the 256 x 256 tiles cover the first 24576
    output columns and the second launch (128 x 64 tiles) the last 1024;
    the 64 full rows span both."""
    o = oracle_mod
    x, w = S.nvfp4_prefill(M=M, N=25600, K=5120, seed=5)
    e = _sampled_wonly(o, bsfp, x, o.quantize(2, w), seed=55)
    assert e.max() <= TOL, e.max()


# 2048 rows x 8448 columns make 8 x 33 = 264 tiles of 256 x 256: on 256 CUs
# one whole round plus 8 tiles, so the first 8192 columns run on the big
# tiles and the last 256 on the second launch's 128 x 64 tiles.  A small K
# (2 and 3 steps of 64) keeps the full oracle product small.
TAIL_SPLIT = [(2048, 8448, 128), (2048, 8448, 192)]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M,N,K", TAIL_SPLIT)
def test_weight_only_tail_split_full(oracle_mod, bsfp, mode, M, N, K):
    x = S.generic((M, K), 1.0, seed=1700 + mode, stream=K)
    w = S.generic((N, K), 0.02, seed=1710 + mode, stream=K)
    check_wonly(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


@pytest.mark.parametrize("M,N,K", TAIL_SPLIT)
def test_qq_nvfp4_tail_split_full(oracle_mod, bsfp, M, N, K):
    x = S.generic((M, K), 0.02, seed=1720, stream=K)
    w = S.generic((N, K), 0.02, seed=1721, stream=K)
    check_qq(oracle_mod, bsfp, x, oracle_mod.quantize(2, w))


def test_affine_weight_only_extra_shape_sampled(oracle_mod, bsfp):
    """x[2048,5120] . W_up[25600,5120]^T, affine weight-only, sampled (the
    64 full rows span both the big-tile and the small-tile column ranges)."""
    o = oracle_mod
    x = S.generic((2048, 5120), 1.0, seed=6)
    _, w = S.affine_decode("up")
    e = _sampled_wonly(o, bsfp, x, o.quantize(0, w), seed=6)
    assert e.max() <= TOL, e.max()


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_onehot_rows_select_weight_columns(oracle_mod, bsfp, mode):
    """Row m of x is e_{j_m}: y[m, n] = bf16(w_hat[n, j_m]) (weight-only;
    exact for MXFP4 and NVFP4 without a global scale, one bf16 step for
    affine, whose weights are rounded to bf16 before the MFMA)."""
    o = oracle_mod
    M, N, K = 70, 300, 640
    w = S.generic((N, K), 0.02, seed=700 + mode)
    qo = o.quantize(mode, w, use_global=False) if mode == 2 else o.quantize(mode, w)
    B = o.dequant_exact(qo)
    rng = np.random.default_rng(mode)
    j = rng.integers(0, K, M)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), j] = 0x3F80
    y = o.bf16_to_f32(qmm_dev(o, bsfp, x, qo, "bf16")).astype(np.float64)
    ref = o.bf16_to_f32(o.bf16_from_f64(B[:, j].T)).astype(np.float64)
    if mode == 0:
        assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -7 + 1e-30)
    else:
        assert np.array_equal(y, ref)


def test_qmv_and_qmm_agree(oracle_mod, bsfp):
    o = oracle_mod
    x = S.generic((1, 2048), 1.0, seed=12)
    w = S.generic((512, 2048), 0.02, seed=13)
    for mode in (0, 1, 2):
        qd = oracle_to_dev(bsfp, o, o.quantize(mode, w))
        a = o.bf16_to_f32(from_dev(bsfp.qmv(to_dev(x), qd))).astype(np.float64)
        c = o.bf16_to_f32(from_dev(bsfp.qmm(to_dev(x), qd))).astype(np.float64)
        _, den = o.matmul_wonly(x, o.quantize(mode, w))
        assert np.max(np.abs(a - c) / den) <= 2 * TOL


def test_qmm_deterministic(bsfp):
    x = to_dev(S.generic((300, 1024), 0.02, seed=1))
    w = to_dev(S.generic((700, 1024), 0.02, seed=2))
    for mode, act in ((0, "bf16"), (1, "bf16"), (2, "bf16"), (1, "same"), (2, "same")):
        q = bsfp.quantize(w, mode)
        assert torch.equal(bsfp.qmm(x, q, act=act), bsfp.qmm(x, q, act=act))


def test_qmm_unsupported_cases(bsfp):
    x = to_dev(S.generic((4, 96), 1.0, seed=1))
    w = to_dev(S.generic((8, 96), 1.0, seed=2))
    q = bsfp.quantize(w, 2)
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm(x, q)
    assert ei.value.status == 2
    x = to_dev(S.generic((4, 128), 1.0, seed=1))
    qa = bsfp.quantize(to_dev(S.generic((8, 128), 1.0, seed=2)), 0)
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm(x, qa, act="same")
    assert ei.value.status == 2


# ---------------------------------------------------------------- dense path
# W dequantized to bf16 into a caller-owned scratch, then a dense bf16 GEMM
# ("mlx: opt-in dense GEMM for nvfp4 prefill").  Against the oracle's dense
# reference the operands are identical and exact, so only fp32 summation
# order and the output rounding remain: the qq bar.

def check_dense(o, b, x, qo, scratch=None, tol=QQ_TOL):
    qd = oracle_to_dev(b, o, qo)
    y = from_dev(b.qmm_dense(to_dev(x), qd, scratch=scratch))
    yref, den = o.matmul_dense(x, qo)
    e = o.norm_err(y, yref, den)
    assert e.max() <= tol, (e.max(), np.unravel_index(e.argmax(), e.shape))
    return y


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dense_ragged(oracle_mod, bsfp, mode, M, N, K):
    x = S.generic((M, K), 1.0, seed=1500 + M, stream=K)
    w = S.generic((N, K), 0.02, seed=1501 + mode, stream=N)
    check_dense(oracle_mod, bsfp, x, oracle_mod.quantize(mode, w))


# The dense path's column split.  From 768 rows the tiles are 256 x 256:
# 2048 rows x 8448 columns make 8 x 33 = 264 tiles, one whole round on 256
# CUs plus 8 tiles, so the first 8192 columns run on the big tiles and the
# last 256 on 128 x 64 tiles.  Below 768 rows the tiles are 256 x 128: 512 x
# 16896 make 2 x 132 = 264 (16384 columns, then 512).  K = 1024 and 1088 (16
# and 17 steps: both remainders of the three-stage loop): at K of a few
# hundred |y| can come close to sum_k |x_k w_k| for some of the outputs, and
# the bf16 rounding of the output alone (up to 2^-8 of |y|) then exceeds the
# 2.2e-3 bar.
DENSE_SPLIT = [(2048, 8448, 1024), (2048, 8448, 1088), (512, 16896, 1024)]


@pytest.mark.parametrize("M,N,K", DENSE_SPLIT)
def test_dense_tail_split_full(oracle_mod, bsfp, M, N, K):
    x = S.generic((M, K), 1.0, seed=1730, stream=K)
    w = S.generic((N, K), 0.02, seed=1731, stream=K)
    check_dense(oracle_mod, bsfp, x, oracle_mod.quantize(2, w))


def test_dense_scratch_reused_across_layers(oracle_mod, bsfp):
    """One scratch buffer serves two layers in a row (the bounded transient):
    each result is that layer's product."""
    o = oracle_mod
    N, K = 700, 1024
    scratch = torch.empty(bsfp.qmm_dense_scratch_bytes(N, K), dtype=torch.uint8, device="cuda")
    for layer in range(2):
        x = S.generic((300, K), 1.0, seed=1600 + layer)
        w = S.generic((N, K), 0.02, seed=1610 + layer)
        check_dense(o, bsfp, x, o.quantize(2, w), scratch=scratch)


def test_dense_policy_by_rows(oracle_mod, bsfp):
    """qmm(dense_rows=R): calls of at least R rows take the dense path (bit
    for bit the qmm_dense result), smaller ones the fused kernel."""
    o = oracle_mod
    w = S.generic((400, 512), 0.02, seed=1620)
    qd = oracle_to_dev(bsfp, o, o.quantize(2, w))
    big = to_dev(S.generic((64, 512), 1.0, seed=1621))
    small = to_dev(S.generic((16, 512), 1.0, seed=1622))
    assert torch.equal(bsfp.qmm(big, qd, dense_rows=64), bsfp.qmm_dense(big, qd))
    assert torch.equal(bsfp.qmm(small, qd, dense_rows=64), bsfp.qmm(small, qd))


def test_dense_errors(bsfp):
    x = to_dev(S.generic((4, 128), 1.0, seed=1))
    q = bsfp.quantize(to_dev(S.generic((8, 128), 1.0, seed=2)), 2)
    small = torch.empty(8 * 128 * 2 - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm_dense(x, q, scratch=small)
    assert ei.value.status == 1
    x96 = to_dev(S.generic((4, 96), 1.0, seed=1))
    q96 = bsfp.quantize(to_dev(S.generic((8, 96), 1.0, seed=2)), 2)
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm_dense(x96, q96)
    assert ei.value.status == 2


def test_dense_deterministic(bsfp):
    x = to_dev(S.generic((300, 1024), 1.0, seed=3))
    q = bsfp.quantize(to_dev(S.generic((700, 1024), 0.02, seed=4)), 2)
    assert torch.equal(bsfp.qmm_dense(x, q), bsfp.qmm_dense(x, q))


@pytest.mark.parametrize("M", [1134, 2048, 4096])
def test_dense_prefill_sampled_full_size(oracle_mod, bsfp, M):
    """X[M,5120] . W[25600,5120]^T (NVFP4, global scale) at full size: 64 full
    output rows plus 4096 random outputs against the oracle's dense
    reference, computed one by one.  All three run the 256 x 256 dense tile
    with two LDS stages; at M = 2048 and 4096 the last 1024 columns run on
    128 x 64 tiles (the full rows cover them)."""
    o = oracle_mod
    x, w = S.nvfp4_prefill(M=M, N=25600, K=5120, seed=7)
    qo = o.quantize(2, w)
    qd = oracle_to_dev(bsfp, o, qo)
    y = from_dev(bsfp.qmm_dense(to_dev(x), qd))
    ai, bi = _sample_pairs(M, 25600, seed=7)
    ua, ia = np.unique(ai, return_inverse=True)
    ub, ib = np.unique(bi, return_inverse=True)
    A = o.bf16_to_f64(x[ua])
    B = o.matmul_dense(None, qo, rows=ub)
    yref, den = o.matmul_pairs(A, B, ia, ib)
    e = o.norm_err(y[ai, bi], yref, den)
    assert e.max() <= QQ_TOL, e.max()
