"""block_scaled_bit_fp_amd -- Python binding of libbsfp (MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
libbsfp.so (see include/bsfp.h for the contract).  PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing, every call raises.

    q = quantize(w_bf16, NVFP4)                 # QuantizedTensor on the GPU
    y = qmv(x_bf16, q)                          # [M<=8, N] bf16 decode GEMV
    y = qmm(x_bf16, q, act="same")              # [M, N] bf16 prefill GEMM
    w_hat = dequantize(q)
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsfp.so")

AFFINE, MXFP4, NVFP4, MXFP8 = 0, 1, 2, 3
GROUP = {AFFINE: 64, MXFP4: 32, NVFP4: 16, MXFP8: 32}
BITS = {AFFINE: 4, MXFP4: 4, NVFP4: 4, MXFP8: 8}
GS_NONE, GS_COMPUTE, GS_GIVEN = 0, 1, 2
ACT_BF16, ACT_SAME = 0, 1
STATUS = {0: "BSFP_OK", 1: "BSFP_ERR_ARG", 2: "BSFP_ERR_UNSUPPORTED", 3: "BSFP_ERR_DEVICE"}

EXPORTS = ("bsfp_amax", "bsfp_quantize", "bsfp_dequantize", "bsfp_qmv", "bsfp_qmv_batch",
           "bsfp_quantize_sr", "bsfp_quantize_ws", "bsfp_qmm_workspace_bytes", "bsfp_qmm",
           "bsfp_qmm_dense_scratch_bytes",
           "bsfp_qmm_dense", "bsfp_qmm_noalloc", "bsfp_time_next_launch", "bsfp_last_error",
           "bsfp_version")
# most matrices of one bsfp_qmv_batch call (BSFP_QMV_BATCH_MAX)
QMV_BATCH_MAX = 4
# bytes of bsfp_quantize_ws's workspace (BSFP_QUANTIZE_WS_BYTES)
QUANTIZE_WS_BYTES = 1024
# bytes of bsfp_qmm_noalloc's static device workspace (BSFP_NOALLOC_WORKSPACE_BYTES)
NOALLOC_WORKSPACE_BYTES = 32 << 20


class QTensorDesc(C.Structure):
    """Mirror of bsfp_qtensor."""
    _fields_ = [("mode", C.c_int32), ("bits", C.c_int32), ("group_size", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64),
                ("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("global_scale", C.c_void_p), ("amax", C.c_void_p)]


class BsfpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with block_scaled_bit_fp_amd/build.py "
                "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        P, I64, I32 = C.c_void_p, C.c_int64, C.c_int32
        QP = C.POINTER(QTensorDesc)
        sigs = {
            "bsfp_amax": (C.c_int, [P, I64, P, P]),
            "bsfp_quantize": (C.c_int, [P, QP, I32, P]),
            "bsfp_quantize_sr": (C.c_int, [P, QP, I32, P, P]),
            "bsfp_quantize_ws": (C.c_int, [P, QP, I32, P, P, I64, P]),
            "bsfp_dequantize": (C.c_int, [QP, P, P]),
            "bsfp_qmv": (C.c_int, [P, I64, QP, P, P]),
            "bsfp_qmv_batch": (C.c_int, [P, I64, C.POINTER(QP), I32, C.POINTER(P), P]),
            "bsfp_qmm_workspace_bytes": (C.c_size_t, [I32, I64, I64, I32]),
            "bsfp_qmm": (C.c_int, [P, I64, QP, I32, P, C.c_size_t, P, P]),
            "bsfp_qmm_dense_scratch_bytes": (C.c_size_t, [I64, I64]),
            "bsfp_qmm_dense": (C.c_int, [P, I64, QP, P, C.c_size_t, P, P]),
            "bsfp_qmm_noalloc": (C.c_int, [P, I64, QP, I32, P, P]),
            "bsfp_time_next_launch": (C.c_int, [P, P]),
            "bsfp_last_error": (C.c_char_p, []),
            "bsfp_version": (C.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise BsfpError(status, lib().bsfp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    """The current HIP stream of the current device, as a raw pointer."""
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def time_next_launch(start_event: Optional[int], stop_event: Optional[int]) -> None:
    """Attach two hipEvent_t handles (ints) to the main kernel of this thread's
    next qmv / qmm call: they record that kernel's own start and end."""
    _check(lib().bsfp_time_next_launch(start_event, stop_event))


def version() -> str:
    return lib().bsfp_version().decode()


@dataclass
class QuantizedTensor:
    """A quantized [rows, cols] tensor in device memory (see include/bsfp.h)."""
    mode: int
    rows: int
    cols: int
    codes: torch.Tensor                       # int32 [rows, cols*bits/32] (uint32 words)
    scales: torch.Tensor                      # uint8 [rows, cols/g] or bf16 (affine)
    biases: Optional[torch.Tensor] = None     # bf16 [rows, cols/g] (affine)
    global_scale: Optional[torch.Tensor] = None  # fp32 [1] (NVFP4 g)
    amax: Optional[torch.Tensor] = None          # fp32 [1] (NVFP4 tensor amax)
    bits: Optional[int] = None                   # None: the mode's (4; MXFP8 8)
    group: Optional[int] = None                  # None: the mode's group size
    # uint8 [QUANTIZE_WS_BYTES] (NVFP4): the bsfp_quantize_ws workspace used
    # when quantize() computes the global scale into this tensor
    scratch: Optional[torch.Tensor] = None

    @property
    def group_size(self) -> int:
        return self.group if self.group is not None else GROUP[self.mode]

    @property
    def nbits(self) -> int:
        return self.bits if self.bits is not None else BITS[self.mode]

    def desc(self) -> QTensorDesc:
        """The C descriptor; rebuilt whenever a field or a tensor's storage changed."""
        ts = (self.codes, self.scales, self.biases, self.global_scale, self.amax)
        key = (self.mode, self.nbits, self.group_size, self.rows, self.cols) + tuple(
            None if t is None else t.data_ptr() for t in ts)
        cached = self.__dict__.get("_desc")
        if cached is None or cached[0] != key:
            d = QTensorDesc(*key)
            self.__dict__["_desc"] = cached = (key, d)
        return cached[1]


def empty_quantized(mode: int, rows: int, cols: int, device="cuda",
                    global_scale: bool = True, bits: Optional[int] = None,
                    group: Optional[int] = None) -> QuantizedTensor:
    G = group if group is not None else GROUP[mode]
    nb = bits if bits is not None else BITS[mode]
    if cols % G:
        raise ValueError(f"cols={cols} is not a multiple of the group size {G}")
    codes = torch.empty((rows, cols * nb // 32), dtype=torch.int32, device=device)
    if mode == AFFINE:
        scales = torch.empty((rows, cols // G), dtype=torch.bfloat16, device=device)
        biases = torch.empty((rows, cols // G), dtype=torch.bfloat16, device=device)
        return QuantizedTensor(mode, rows, cols, codes, scales, biases, bits=bits, group=group)
    scales = torch.empty((rows, cols // G), dtype=torch.uint8, device=device)
    if mode == MXFP8:
        return QuantizedTensor(mode, rows, cols, codes, scales, bits=bits, group=group)
    gs = am = ws = None
    if mode == NVFP4 and global_scale:
        gs = torch.empty(1, dtype=torch.float32, device=device)
        am = torch.empty(1, dtype=torch.float32, device=device)
        ws = torch.empty(QUANTIZE_WS_BYTES, dtype=torch.uint8, device=device)
    return QuantizedTensor(mode, rows, cols, codes, scales, None, gs, am, scratch=ws)


def _as_2d_bf16(x: torch.Tensor) -> torch.Tensor:
    if x.dtype != torch.bfloat16:
        raise TypeError(f"expected bfloat16, got {x.dtype}")
    if not x.is_cuda:
        raise TypeError("expected a tensor on the GPU")
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return x.reshape(-1, x.shape[-1]) if x.dim() != 2 else x


def _out_bf16(out: Optional[torch.Tensor], shape, device) -> torch.Tensor:
    """A caller's output buffer: checked before any pointer crosses the C ABI
    (which cannot know buffer sizes), or a new one."""
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be bf16 of shape {tuple(shape)}, got {out.dtype} "
                         f"{tuple(out.shape)}")
    if not out.is_cuda or out.device != torch.device(device) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous tensor on {device}")
    return out


def _buffer(t: Optional[torch.Tensor], need: int, device, what: str) -> Optional[torch.Tensor]:
    """A caller's workspace or scratch of at least `need` bytes, or a new one."""
    if t is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need else None
    if not t.is_cuda or t.device != torch.device(device) or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous tensor on {device}")
    return t


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def amax(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |x| as a device fp32 [1] tensor."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("amax expects a contiguous bf16 GPU tensor")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().bsfp_amax(_ptr(x), x.numel(), _ptr(out), _stream()))
    return out


def quantize(x: torch.Tensor, mode: int, global_scale: str = "compute",
             g: Optional[torch.Tensor] = None,
             out: Optional[QuantizedTensor] = None,
             rbits: Optional[torch.Tensor] = None, bits: Optional[int] = None,
             group: Optional[int] = None,
             workspace: Optional[torch.Tensor] = None) -> QuantizedTensor:
    """Quantize a bf16 [rows, cols] GPU tensor.  For NVFP4, global_scale is
    'compute' (g = amax/2688), 'given' (use the fp32 [1] tensor g) or 'none'.
    rbits (uint32 words, one per element, NVFP4 / MXFP4): stochastic rounding
    of the codes with those random words (bsfp_quantize_sr).  NVFP4 with
    'compute' runs bsfp_quantize_ws on `workspace` (at least
    QUANTIZE_WS_BYTES bytes), else on out.scratch, when there is one."""
    x2 = _as_2d_bf16(x)
    rows, cols = x2.shape
    gs = {"none": GS_NONE, "compute": GS_COMPUTE, "given": GS_GIVEN}[global_scale]
    if out is None:
        out = empty_quantized(mode, rows, cols, x.device, global_scale=(gs != GS_NONE),
                              bits=bits, group=group)
        if mode == NVFP4 and gs == GS_GIVEN:
            if g is None:
                raise ValueError("global_scale='given' needs g")
            out.global_scale.copy_(g.reshape(1).to(torch.float32))
    else:
        if out.mode != mode or (out.rows, out.cols) != (rows, cols):
            raise ValueError(f"out holds mode {out.mode} [{out.rows}, {out.cols}], the call "
                             f"asks for mode {mode} [{rows}, {cols}]")
        if (bits is not None and bits != out.nbits) or (group is not None and
                                                         group != out.group_size):
            raise ValueError("out's bits or group size differ from the ones asked for")
    if mode == NVFP4 and gs == GS_NONE:
        out.global_scale = None
    d = out.desc()
    if rbits is not None:
        if rbits.numel() != rows * cols or rbits.element_size() != 4 or not rbits.is_contiguous():
            raise ValueError("rbits needs one contiguous 32-bit word per element")
    ws = workspace if workspace is not None else out.scratch
    if mode == NVFP4 and gs == GS_COMPUTE and ws is not None:
        ws = _buffer(ws, QUANTIZE_WS_BYTES, x.device, "workspace")
        _check(lib().bsfp_quantize_ws(_ptr(x2), C.byref(d), gs, _ptr(rbits), _ptr(ws),
                                      _nbytes(ws), _stream()))
        return out
    if rbits is not None:
        _check(lib().bsfp_quantize_sr(_ptr(x2), C.byref(d), gs if mode == NVFP4 else 0,
                                      _ptr(rbits), _stream()))
        return out
    _check(lib().bsfp_quantize(_ptr(x2), C.byref(d), gs if mode == NVFP4 else 0, _stream()))
    return out


def dequantize(q: QuantizedTensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    out = _out_bf16(out, (q.rows, q.cols), q.codes.device)
    d = q.desc()
    _check(lib().bsfp_dequantize(C.byref(d), _ptr(out), _stream()))
    return out


def qmv(x: torch.Tensor, w: QuantizedTensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[M, N] = x[M, K] . dq(W)^T for M <= 8 (decode GEMV)."""
    x2 = _as_2d_bf16(x)
    M = x2.shape[0]
    if x2.shape[1] != w.cols:
        raise ValueError(f"x has K={x2.shape[1]}, W has K={w.cols}")
    out = _out_bf16(out, (M, w.rows), x.device)
    d = w.desc()
    _check(lib().bsfp_qmv(_ptr(x2), M, C.byref(d), _ptr(out), _stream()))
    return out


def qmv_batch(x: torch.Tensor, ws, outs=None):
    """[x . dq(W_i)^T for W_i in ws]: the decode GEMV of several matrices that
    share x, K and the format (bsfp_qmv_batch: one launch where the kernels
    allow).  outs: optional list of bf16 [M, W_i.rows] outputs."""
    ws = list(ws)
    if not 1 <= len(ws) <= QMV_BATCH_MAX:
        raise ValueError(f"qmv_batch takes 1..{QMV_BATCH_MAX} matrices, got {len(ws)}")
    x2 = _as_2d_bf16(x)
    M = x2.shape[0]
    for w in ws:
        if x2.shape[1] != w.cols:
            raise ValueError(f"x has K={x2.shape[1]}, W has K={w.cols}")
    if outs is None:
        outs = [None] * len(ws)
    if len(outs) != len(ws):
        raise ValueError("qmv_batch needs one output per matrix")
    outs = [_out_bf16(o, (M, w.rows), x.device) for o, w in zip(outs, ws)]
    descs = [w.desc() for w in ws]
    darr = (C.POINTER(QTensorDesc) * len(ws))(*[C.pointer(d) for d in descs])
    yarr = (C.c_void_p * len(ws))(*[_ptr(o) for o in outs])
    _check(lib().bsfp_qmv_batch(_ptr(x2), M, darr, len(ws), yarr, _stream()))
    return outs


def qmm_workspace_bytes(mode: int, M: int, K: int, act: str = "bf16") -> int:
    return int(lib().bsfp_qmm_workspace_bytes(mode, M, K, ACT_SAME if act == "same" else ACT_BF16))


def qmm_dense_scratch_bytes(rows: int, cols: int) -> int:
    return int(lib().bsfp_qmm_dense_scratch_bytes(rows, cols))


def qmm_dense(x: torch.Tensor, w: QuantizedTensor, scratch: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense prefill path: W dequantized to bf16 into `scratch` (one layer's
    copy, caller-owned and reusable), then y = x . scratch^T."""
    x2 = _as_2d_bf16(x)
    M = x2.shape[0]
    if x2.shape[1] != w.cols:
        raise ValueError(f"x has K={x2.shape[1]}, W has K={w.cols}")
    need = qmm_dense_scratch_bytes(w.rows, w.cols)
    scratch = _buffer(scratch, need, x.device, "scratch")
    out = _out_bf16(out, (M, w.rows), x.device)
    d = w.desc()
    _check(lib().bsfp_qmm_dense(_ptr(x2), M, C.byref(d), _ptr(scratch), _nbytes(scratch),
                                _ptr(out), _stream()))
    return out


def qmm(x: torch.Tensor, w: QuantizedTensor, act: str = "bf16",
        workspace: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None, dense_rows: Optional[int] = None,
        scratch: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[M, N] = x . dq(W)^T ('bf16') or alpha * dq0(q(x)) . dq0(W)^T ('same').
    With dense_rows set, a 'bf16' call of at least that many rows takes the
    dense path (qmm_dense, dequantizing into `scratch`); off by default."""
    x2 = _as_2d_bf16(x)
    M = x2.shape[0]
    if x2.shape[1] != w.cols:
        raise ValueError(f"x has K={x2.shape[1]}, W has K={w.cols}")
    if act != "same" and dense_rows is not None and M >= dense_rows:
        return qmm_dense(x2, w, scratch=scratch, out=out)
    a = ACT_SAME if act == "same" else ACT_BF16
    need = int(lib().bsfp_qmm_workspace_bytes(w.mode, M, w.cols, a))
    workspace = _buffer(workspace, need, x.device, "workspace")
    out = _out_bf16(out, (M, w.rows), x.device)
    d = w.desc()
    _check(lib().bsfp_qmm(_ptr(x2), M, C.byref(d), a, _ptr(workspace), _nbytes(workspace),
                          _ptr(out), _stream()))
    return out


def qmm_noalloc(x: torch.Tensor, w: QuantizedTensor, act: str = "bf16",
                out: torch.Tensor = None) -> torch.Tensor:
    """qmm whose qq workspace is the library's static device array
    (bsfp_qmm_noalloc): the C call allocates nothing.  Pass `out` to keep
    the whole call free of allocations.  Calls that overlap on one GPU share
    that array and must be serialized by the caller."""
    x2 = _as_2d_bf16(x)
    M = x2.shape[0]
    if x2.shape[1] != w.cols:
        raise ValueError(f"x has K={x2.shape[1]}, W has K={w.cols}")
    out = _out_bf16(out, (M, w.rows), x.device)
    a = ACT_SAME if act == "same" else ACT_BF16
    d = w.desc()
    _check(lib().bsfp_qmm_noalloc(_ptr(x2), M, C.byref(d), a, _ptr(out), _stream()))
    return out
