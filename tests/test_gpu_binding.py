"""The binding's checks of caller buffers.  The C ABI takes plain pointers and
cannot know buffer sizes, so the binding checks every caller-supplied output,
workspace and scratch tensor (shape, dtype, layout, device) before a pointer
crosses it, and counts workspace bytes whatever the tensor's element type."""
import numpy as np
import pytest
import torch

import synth_inputs as S
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small(bsfp):
    x = to_dev(S.generic((2, 1024), 1.0, seed=700))
    x64 = to_dev(S.generic((64, 1024), 1.0, seed=701))
    w = to_dev(S.generic((96, 1024), 0.02, seed=702))
    return x, x64, w, bsfp.quantize(w, bsfp.NVFP4)


def test_qmv_rejects_bad_out(bsfp, small):
    x, _, _, q = small
    bad = [torch.empty((2, 95), dtype=torch.bfloat16, device="cuda"),      # shape
           torch.empty((2, 96), dtype=torch.float16, device="cuda"),       # dtype
           torch.empty((96, 2), dtype=torch.bfloat16, device="cuda").t(),  # layout
           torch.empty((2, 96), dtype=torch.bfloat16)]                     # host
    for out in bad:
        with pytest.raises(ValueError):
            bsfp.qmv(x, q, out=out)
    good = torch.empty((2, 96), dtype=torch.bfloat16, device="cuda")
    assert bsfp.qmv(x, q, out=good) is good


def test_qmm_dequantize_and_dense_reject_bad_out(bsfp, small):
    _, x64, _, q = small
    with pytest.raises(ValueError):
        bsfp.qmm(x64, q, out=torch.empty((64, 97), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        bsfp.dequantize(q, out=torch.empty((96, 1023), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        bsfp.qmm_dense(x64, q, out=torch.empty((64, 96), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        bsfp.qmm(x64, q, act="same",
                 workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda")[::2])


def test_quantize_rejects_out_of_another_format(bsfp, small):
    _, _, w, _ = small
    mx = bsfp.empty_quantized(bsfp.MXFP4, 96, 1024, w.device)
    with pytest.raises(ValueError):
        bsfp.quantize(w, bsfp.NVFP4, out=mx)
    other = bsfp.empty_quantized(bsfp.NVFP4, 96, 512, w.device)
    with pytest.raises(ValueError):
        bsfp.quantize(w, bsfp.NVFP4, out=other)


def test_workspace_counts_bytes_not_elements(bsfp, small):
    """A workspace of int32 words is as good as one of bytes: the binding
    passes numel * element_size, so the same call gives the same bits."""
    _, x64, _, q = small
    need = bsfp.qmm_workspace_bytes(bsfp.NVFP4, 64, 1024, "same")
    ws8 = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws32 = torch.empty((need + 3) // 4, dtype=torch.int32, device="cuda")
    y8 = bsfp.qmm(x64, q, act="same", workspace=ws8)
    y32 = bsfp.qmm(x64, q, act="same", workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(y8, y32)
    # a workspace one word short is refused by the library's size check
    with pytest.raises(bsfp.BsfpError) as ei:
        bsfp.qmm(x64, q, act="same", workspace=ws32[: need // 4 - 1])
    assert ei.value.status == 1
