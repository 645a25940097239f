"""Python face of the CPU oracle (ctypes over oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the CPU-baseline leg of bench.py, never by the
product package.  It does not import the product package and shares no code
with it.

All arrays are numpy, host side.  bf16 tensors are uint16 bit patterns.
Modes: 0 affine (4-bit group 64; format variants: 4 or 8 bits, groups 32,
64, 128), 1 MXFP4 (group 32), 2 NVFP4 (group 16), 3 MXFP8 (8-bit E4M3
elements, group 32).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# BSFP_ORACLE_LIB names another build of the same source (the mutation check
# in tests/ loads copies with one planted mistake each); default: this build.
LIB_PATH = os.environ.get("BSFP_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

AFFINE, MXFP4, NVFP4, MXFP8 = 0, 1, 2, 3
GROUP = {AFFINE: 64, MXFP4: 32, NVFP4: 16, MXFP8: 32}
BITS = {AFFINE: 4, MXFP4: 4, NVFP4: 4, MXFP8: 8}
MODE_NAMES = {AFFINE: "affine", MXFP4: "mxfp4", NVFP4: "nvfp4", MXFP8: "mxfp8"}

_lib = None

_P = C.c_void_p
_I64 = C.c_int64


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_P)


def lib():
    """Load the oracle library, building it first only if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433
            _b.build()
        L = C.CDLL(LIB_PATH)
        sig = {
            "bo_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "bo_bf16_from_f32": (C.c_uint16, [C.c_float]),
            "bo_bf16_from_f64": (C.c_uint16, [C.c_double]),
            "bo_e2m1_decode": (C.c_double, [C.c_int]),
            "bo_e2m1_encode": (C.c_int, [C.c_float]),
            "bo_e4m3_decode": (C.c_double, [C.c_int]),
            "bo_e4m3_encode": (C.c_int, [C.c_float]),
            "bo_e8m0_decode": (C.c_double, [C.c_int]),
            "bo_e2m1_encode_array": (None, [_P, _I64, _P]),
            "bo_e4m3_encode_array": (None, [_P, _I64, _P]),
            "bo_bf16_from_f32_array": (None, [_P, _I64, _P]),
            "bo_bf16_from_f64_array": (None, [_P, _I64, _P]),
            "bo_bf16_to_f64_array": (None, [_P, _I64, _P]),
            "bo_amax": (C.c_float, [_P, _I64]),
            "bo_nvfp4_global_scale": (C.c_float, [C.c_float]),
            "bo_alpha": (C.c_float, [C.c_float, C.c_float]),
            "bo_quantize_nvfp4": (None, [_P, _I64, _I64, C.c_int, _P, _P, _P, _P, _P]),
            "bo_quantize_mxfp4": (None, [_P, _I64, _I64, _P, _P]),
            "bo_quantize_nvfp4_sr": (None, [_P, _I64, _I64, C.c_int, _P, _P, _P, _P, _P, _P]),
            "bo_quantize_mxfp4_sr": (None, [_P, _I64, _I64, _P, _P, _P]),
            "bo_quantize_affine_g": (None, [_P, _I64, _I64, C.c_int, C.c_int, _P, _P, _P]),
            "bo_quantize_mxfp8": (None, [_P, _I64, _I64, _P, _P]),
            "bo_dequantize_g": (None, [C.c_int, C.c_int, C.c_int, _P, _P, _P, _I64, _I64, _P]),
            "bo_dequant_exact_g": (None, [C.c_int, C.c_int, C.c_int, _P, _P, _P, _I64, _I64, _P]),
            "bo_e2m1_encode_sr": (C.c_int, [C.c_float, C.c_uint32]),
            "bo_quantize_affine": (None, [_P, _I64, _I64, _P, _P, _P]),
            "bo_dequantize_nvfp4": (None, [_P, _P, _P, _I64, _I64, _P]),
            "bo_dequantize_mxfp4": (None, [_P, _P, _I64, _I64, _P]),
            "bo_dequantize_affine": (None, [_P, _P, _P, _I64, _I64, _P]),
            "bo_dequant_exact": (None, [C.c_int, _P, _P, _P, _P, _I64, _I64, _P]),
            "bo_matmul_f64": (None, [_P, _P, _I64, _I64, _I64, C.c_double, _P, _P]),
            "bo_matmul_f64_pairs": (None, [_P, _P, _I64, _P, _P, _I64, C.c_double, _P, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# --------------------------------------------------------------------------
# scalar / array codecs
# --------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_from_f32(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().bo_bf16_from_f32_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().bo_bf16_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().bo_bf16_to_f64_array(_ptr(bits), bits.size, _ptr(out))
    return out


def e2m1_table() -> np.ndarray:
    return np.array([lib().bo_e2m1_decode(c) for c in range(16)], np.float64)


def e4m3_table() -> np.ndarray:
    return np.array([lib().bo_e4m3_decode(c) for c in range(256)], np.float64)


def e8m0_table() -> np.ndarray:
    return np.array([lib().bo_e8m0_decode(c) for c in range(256)], np.float64)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().bo_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_encode_sr(v: float, r: int) -> int:
    """Stochastic rounding of one fp32 value to an E2M1 code (reading R15)."""
    return int(lib().bo_e2m1_encode_sr(float(np.float32(v)), int(r) & 0xFFFFFFFF))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().bo_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def amax(x_bits: np.ndarray) -> np.float32:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    return np.float32(lib().bo_amax(_ptr(x_bits), x_bits.size))


def global_scale(amax_value) -> np.float32:
    return np.float32(lib().bo_nvfp4_global_scale(float(np.float32(amax_value))))


def alpha(g_x, g_w) -> np.float32:
    return np.float32(lib().bo_alpha(float(np.float32(g_x)), float(np.float32(g_w))))


# --------------------------------------------------------------------------
# quantized tensors
# --------------------------------------------------------------------------

@dataclass
class QTensor:
    mode: int
    rows: int
    cols: int
    codes: np.ndarray                  # uint32 [rows, cols/8]
    scales: np.ndarray                 # uint8 [rows, cols/g] (uint16 bf16 for affine)
    biases: Optional[np.ndarray] = None  # uint16 bf16 [rows, cols/64], affine only
    g: Optional[np.float32] = None     # NVFP4 global scale (None: no global scale)
    amax: Optional[np.float32] = None  # NVFP4 tensor amax when computed
    bits: int = 4                      # code width (8: affine 8-bit, MXFP8)
    group: Optional[int] = None        # group size (None: the mode's default)

    @property
    def group_size(self) -> int:
        return self.group if self.group is not None else GROUP[self.mode]

    @property
    def variant(self) -> bool:
        """A format variant: MXFP8, or affine other than 4-bit group 64."""
        return self.mode == MXFP8 or (self.mode == AFFINE and
                                      (self.bits, self.group_size) != (4, 64))


def quantize(mode: int, x_bits: np.ndarray, use_global: bool = True,
             g: Optional[float] = None, rbits: Optional[np.ndarray] = None,
             bits: Optional[int] = None, group: Optional[int] = None) -> QTensor:
    """Quantize a bf16 [rows, cols] tensor.  For NVFP4, use_global selects a
    per-tensor global scale, either the given g or amax/2688 computed here.
    rbits (uint32 [rows, cols], NVFP4 / MXFP4 only) selects stochastic
    rounding of the codes with those random words (reading R15)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim == 1:
        x_bits = x_bits.reshape(1, -1)
    rows, cols = x_bits.shape
    G = group if group is not None else GROUP[mode]
    nbits = bits if bits is not None else BITS[mode]
    if cols % G:
        raise ValueError(f"cols={cols} is not a multiple of the group size {G}")
    if mode == MXFP8:
        if (nbits, G) != (8, 32):
            raise ValueError("MXFP8 is 8-bit with groups of 32")
        codes = np.zeros((rows, cols // 4), np.uint32)
        scales = np.zeros((rows, cols // G), np.uint8)
        lib().bo_quantize_mxfp8(_ptr(x_bits), rows, cols, _ptr(codes), _ptr(scales))
        return QTensor(mode, rows, cols, codes, scales, bits=8, group=32)
    if mode == AFFINE and (nbits, G) != (4, 64):
        if nbits not in (4, 8) or G not in (32, 64, 128):
            raise ValueError(f"affine ({nbits} bits, group {G}) is not a supported variant")
        codes = np.zeros((rows, cols * nbits // 32), np.uint32)
        scales = np.zeros((rows, cols // G), np.uint16)
        biases = np.zeros((rows, cols // G), np.uint16)
        lib().bo_quantize_affine_g(_ptr(x_bits), rows, cols, nbits, G, _ptr(codes),
                                   _ptr(scales), _ptr(biases))
        return QTensor(mode, rows, cols, codes, scales, biases, bits=nbits, group=G)
    if (nbits, G) != (BITS[mode], GROUP[mode]):
        raise ValueError(f"{MODE_NAMES[mode]} has no ({nbits} bits, group {G}) variant")
    if rbits is not None:
        if mode == AFFINE:
            raise ValueError("stochastic rounding applies to NVFP4 and MXFP4")
        rbits = np.ascontiguousarray(rbits, dtype=np.uint32).reshape(rows, cols)
    codes = np.zeros((rows, cols // 8), np.uint32)
    L = lib()
    if mode == NVFP4:
        scales = np.zeros((rows, cols // G), np.uint8)
        g_out = np.zeros(1, np.float32)
        amax_out = np.full(1, np.nan, np.float32)
        g_in = None if g is None else np.array([g], np.float32)
        if rbits is None:
            L.bo_quantize_nvfp4(_ptr(x_bits), rows, cols, int(bool(use_global)), _ptr(g_in),
                                _ptr(codes), _ptr(scales), _ptr(g_out), _ptr(amax_out))
        else:
            L.bo_quantize_nvfp4_sr(_ptr(x_bits), rows, cols, int(bool(use_global)), _ptr(g_in),
                                   _ptr(rbits), _ptr(codes), _ptr(scales), _ptr(g_out),
                                   _ptr(amax_out))
        return QTensor(mode, rows, cols, codes, scales, None,
                       np.float32(g_out[0]) if use_global else None,
                       None if np.isnan(amax_out[0]) else np.float32(amax_out[0]))
    if mode == MXFP4:
        scales = np.zeros((rows, cols // G), np.uint8)
        if rbits is None:
            L.bo_quantize_mxfp4(_ptr(x_bits), rows, cols, _ptr(codes), _ptr(scales))
        else:
            L.bo_quantize_mxfp4_sr(_ptr(x_bits), rows, cols, _ptr(rbits), _ptr(codes),
                                   _ptr(scales))
        return QTensor(mode, rows, cols, codes, scales)
    if mode == AFFINE:
        scales = np.zeros((rows, cols // G), np.uint16)
        biases = np.zeros((rows, cols // G), np.uint16)
        L.bo_quantize_affine(_ptr(x_bits), rows, cols, _ptr(codes), _ptr(scales), _ptr(biases))
        return QTensor(mode, rows, cols, codes, scales, biases)
    raise ValueError(f"unknown mode {mode}")


def dequantize(q: QTensor) -> np.ndarray:
    """bf16 bits [rows, cols] (NVFP4 includes the global scale when present)."""
    out = np.empty((q.rows, q.cols), np.uint16)
    L = lib()
    if q.variant:
        L.bo_dequantize_g(q.mode, q.bits, q.group_size, _ptr(q.codes), _ptr(q.scales),
                          _ptr(q.biases), q.rows, q.cols, _ptr(out))
        return out
    if q.mode == NVFP4:
        g = None if q.g is None else np.array([q.g], np.float32)
        L.bo_dequantize_nvfp4(_ptr(q.codes), _ptr(q.scales), _ptr(g), q.rows, q.cols, _ptr(out))
    elif q.mode == MXFP4:
        L.bo_dequantize_mxfp4(_ptr(q.codes), _ptr(q.scales), q.rows, q.cols, _ptr(out))
    else:
        L.bo_dequantize_affine(_ptr(q.codes), _ptr(q.scales), _ptr(q.biases), q.rows, q.cols, _ptr(out))
    return out


def dequant_exact(q: QTensor, with_g: bool = True, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Exact real dequantized values in fp64, [rows, cols] (or the selected
    rows).  with_g=False leaves NVFP4's global scale out (the qq operand)."""
    codes, scales, biases = q.codes, q.scales, q.biases
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        codes = np.ascontiguousarray(codes[rows])
        scales = np.ascontiguousarray(scales[rows])
        biases = None if biases is None else np.ascontiguousarray(biases[rows])
    nrows = codes.shape[0]
    out = np.empty((nrows, q.cols), np.float64)
    if q.variant:
        lib().bo_dequant_exact_g(q.mode, q.bits, q.group_size, _ptr(codes), _ptr(scales),
                                 _ptr(biases), nrows, q.cols, _ptr(out))
        return out
    g = None
    if q.mode == NVFP4 and with_g and q.g is not None:
        g = np.array([q.g], np.float32)
    lib().bo_dequant_exact(q.mode, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(g),
                           nrows, q.cols, _ptr(out))
    return out


# --------------------------------------------------------------------------
# matmul references
# --------------------------------------------------------------------------

def matmul_f64(A: np.ndarray, B: np.ndarray, scale: float = 1.0):
    """y = scale * A @ B.T and denom = |scale| * |A| @ |B|.T, plain fp64 loops."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    d = np.empty((M, N), np.float64)
    lib().bo_matmul_f64(_ptr(A), _ptr(B), M, N, K, float(scale), _ptr(y), _ptr(d))
    return y, d


def matmul_pairs(A_rows: np.ndarray, B_rows: np.ndarray, ai, bi, scale: float = 1.0):
    A_rows = np.ascontiguousarray(A_rows, np.float64)
    B_rows = np.ascontiguousarray(B_rows, np.float64)
    ai = np.ascontiguousarray(ai, np.int64)
    bi = np.ascontiguousarray(bi, np.int64)
    K = A_rows.shape[1]
    y = np.empty(ai.shape, np.float64)
    d = np.empty(ai.shape, np.float64)
    lib().bo_matmul_f64_pairs(_ptr(A_rows), _ptr(B_rows), K, _ptr(ai), _ptr(bi), ai.size,
                              float(scale), _ptr(y), _ptr(d))
    return y, d


def matmul_wonly(x_bits: np.ndarray, w: QTensor):
    """Weight-only product y = x . dq(W)^T (NVFP4 includes g_w).
    Returns (y fp64 [M,N], denom [M,N])."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    return matmul_f64(x, dequant_exact(w, with_g=True))


def matmul_dense(x_bits: np.ndarray, w: QTensor, rows: Optional[np.ndarray] = None):
    """Dense prefill path ("mlx: opt-in dense GEMM for nvfp4 prefill
    (dequantise to bf16 above a row threshold)"): W dequantized to bf16 by
    the dequantize rule (NVFP4 with its global scale, one rounding to bf16),
    then y = x . W_bf16^T computed exactly.  Returns (y, denom); with `rows`,
    the bf16 weights of those rows only (for sampled checks), as (W_bf16
    rows in fp64) instead."""
    Wb = bf16_to_f64(dequantize(w))
    if rows is not None:
        return Wb[np.asarray(rows, np.int64)]
    x = bf16_to_f64(np.atleast_2d(x_bits))
    return matmul_f64(x, Wb)


def qq_operands(x_bits: np.ndarray, w: QTensor):
    """x quantized with W's mode; returns (qx, A = dq0(qx), B = dq0(W), alpha)."""
    qx = quantize(w.mode, np.atleast_2d(x_bits), use_global=(w.mode == NVFP4 and w.g is not None))
    A = dequant_exact(qx, with_g=False)
    B = dequant_exact(w, with_g=False)
    if w.mode == NVFP4 and w.g is not None:
        a = alpha(qx.g, w.g)
    else:
        a = np.float32(1.0)
    return qx, A, B, a


def matmul_qq(x_bits: np.ndarray, w: QTensor):
    """qq product y = alpha * dq0(q(x)) . dq0(W)^T.  Returns (y, denom, qx, alpha)."""
    qx, A, B, a = qq_operands(x_bits, w)
    y, d = matmul_f64(A, B, float(a))
    return y, d, qx, a


def norm_err(y_bits: np.ndarray, y_ref: np.ndarray, denom: np.ndarray) -> np.ndarray:
    """|y - y_ref| / sum_k |a_k b_k|; where the denominator is 0 the error is
    0 if y == 0 exactly and inf otherwise."""
    y = bf16_to_f32(y_bits).astype(np.float64)
    diff = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0),
                     np.where(diff == 0, 0.0, np.inf))
    return e
