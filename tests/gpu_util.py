"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""
import numpy as np
import torch


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bf16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    """bf16 / int16 GPU tensor -> uint16 bit patterns (numpy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def words(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint32)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint8)


def qt_to_oracle(o, q):
    """Copy a device QuantizedTensor into an oracle QTensor (host)."""
    scales = from_dev(q.scales) if q.mode == o.AFFINE else u8(q.scales)
    biases = from_dev(q.biases) if q.biases is not None else None
    g = None if q.global_scale is None else np.float32(q.global_scale.cpu().item())
    return o.QTensor(q.mode, q.rows, q.cols, words(q.codes), scales, biases, g,
                     bits=q.nbits, group=q.group_size)


def oracle_to_dev(b, o, qo):
    """Upload an oracle QTensor as a device QuantizedTensor."""
    codes = torch.from_numpy(qo.codes.view(np.int32)).cuda()
    if qo.mode == o.AFFINE:
        scales = to_dev(qo.scales)
        biases = to_dev(qo.biases)
    else:
        scales = torch.from_numpy(qo.scales).cuda()
        biases = None
    gs = None
    if qo.g is not None:
        gs = torch.tensor([float(qo.g)], dtype=torch.float32).cuda()
    return b.QuantizedTensor(qo.mode, qo.rows, qo.cols, codes, scales, biases, gs, None,
                             bits=qo.bits, group=qo.group_size)
