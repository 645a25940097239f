"""bsfp_qmm_noalloc (the qq GEMM with the library's static device workspace,
for callers that cannot allocate) against bsfp_qmm with a caller workspace:
bit-identical outputs on two calls in a row, the second one smaller, for
every path that uses a workspace (NVFP4 and MXFP4 qq GEMM, the NVFP4 qq
decode path whose x exceeds the GEMV's LDS copy) and one that does not
(weight-only), plus the size limit."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _weights(b, mode, N, K, seed):
    return b.quantize(to_dev(S.generic((N, K), 0.02, seed=seed)), mode)


@pytest.mark.parametrize("mode,act,shapes", [
    (2, "same", [(2048, 5120), (300, 5120)]),   # NVFP4 qq GEMM: 21 MB, then 3 MB
    (1, "same", [(2048, 2880), (40, 2880)]),    # MXFP4 qq on the scaled MFMA
    (2, "same", [(8, 8192), (5, 8192)]),        # qq decode with x beyond the GEMV's LDS
    (1, "same", [(8, 8192), (3, 8192)]),
    (2, "bf16", [(512, 1024), (64, 1024)]),     # weight-only: no workspace
])
def test_noalloc_matches_qmm_twice(bsfp, mode, act, shapes):
    N = 1000
    K = shapes[0][1]
    w = _weights(bsfp, mode, N, K, seed=1800 + mode)
    for i, (M, _) in enumerate(shapes):
        x = to_dev(S.generic((M, K), 1.0, seed=1810 + i, stream=mode))
        want = bsfp.qmm(x, w, act=act)
        got = bsfp.qmm_noalloc(x, w, act=act)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (mode, act, M)


def test_noalloc_rejects_a_workspace_beyond_its_size(bsfp):
    K = 5120
    w = _weights(bsfp, 2, 64, K, seed=1820)
    M = bsfp.NOALLOC_WORKSPACE_BYTES // (2 * K) + 1  # fp16 x-hat alone exceeds it
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    assert bsfp.qmm_workspace_bytes(2, M, K, "same") > bsfp.NOALLOC_WORKSPACE_BYTES
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm_noalloc(x, w, act="same")
    assert ei.value.status == 2 and "static" in str(ei.value)
