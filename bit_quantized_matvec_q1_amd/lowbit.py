"""Thin ctypes binding to liblowbit.so: the C ABI's entry points under the same names.

Argument marshalling only -- every step of every product runs in the HIP kernels behind the C ABI.
Tensors are torch device tensors (torch supplies device memory and streams); the stream defaults to
torch's current stream on the tensors' device.  A non-LB_OK status raises LowbitError.  If the shared
library is not built, importing this module raises ImportError: there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

Q1_0, Q2_0_G64, TERNARY_PLANAR, Q8_0, TERNARY_B3 = 1, 2, 3, 4, 5
ACT_Q8_0, ACT_I8_ROW, ACT_F32_Q8_0 = 1, 2, 3
LB_OK, LB_EINVAL, LB_ESHAPE, LB_EALIGN, LB_EUNSUPPORTED, LB_EDEVICE, LB_ENOMEM = range(7)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblowbit.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (python -m bit_quantized_matvec_q1_amd.build); "
                      "the HIP library is the only implementation of this package")

_P, _I, _I64, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float

lib = ctypes.CDLL(LIB_PATH)

# name -> (restype, argtypes), mirroring include/lowbit.h
SIGNATURES = {
    "lowbit_status_str": (ctypes.c_char_p, [_I]),
    "lowbit_last_error": (ctypes.c_char_p, []),
    "lowbit_weight_bytes": (_I64, [_I, _I64, _I64]),
    "lowbit_pack_weights": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "lowbit_unpack_weights": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "lowbit_quantize_act": (_I, [_I, _P, _I64, _I64, _P, _P, _P]),
    "lowbit_matvec": (_I, [_I, _P, _I64, _I64, _F, _I, _P, _P, _P, _P]),
    "lowbit_gemm": (_I, [_I, _P, _I64, _I64, _F, _I, _P, _P, _I64, _P, _P]),
    "lowbit_block_sums": (_I, [_I, _P, _I64, _I64, _I, _P, _P, _I64, _P, _P]),
    "dense_head_matvec": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "dense_head_matvec_i8": (_I, [_P, _P, _I64, _I64, _P, _P, _P]),
    "lowbit_matvec_popcount": (_I, [_P, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P]),
    "lowbit_batch_create": (_I, [_P, ctypes.c_int32, _P]),
    "lowbit_matvec_batched": (_I, [_P, _P]),
    "lowbit_batch_destroy": (None, [_P]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args


class LowbitError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = lib.lowbit_last_error().decode() or lib.lowbit_status_str(status).decode()
        super().__init__(f"{fn}: {lib.lowbit_status_str(status).decode()} ({msg})")


class lb_matvec_desc(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("afmt", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("W", ctypes.c_void_p),
        ("w_tensor_scale", ctypes.c_float),
        ("xq", ctypes.c_void_p),
        ("xscale", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
    ]


def _ptr(t):
    """A device tensor's address (ints pass through as raw addresses).  Host tensors and strided views are
    refused: the kernels take dense device buffers, and a host address in a kernel is a memory fault."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"device tensor required, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor required (the C ABI takes dense row-major buffers)")
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(st: int, fn: str) -> None:
    if st != LB_OK:
        raise LowbitError(st, fn)


def lowbit_weight_bytes(fmt: int, N: int, K: int) -> int:
    return lib.lowbit_weight_bytes(fmt, N, K)


def lowbit_pack_weights(fmt, blocks, N, K, packed, stream=None):
    _check(lib.lowbit_pack_weights(fmt, _ptr(blocks), N, K, _ptr(packed), _stream(stream, packed)),
           "lowbit_pack_weights")


def lowbit_unpack_weights(fmt, packed, N, K, blocks, stream=None):
    _check(lib.lowbit_unpack_weights(fmt, _ptr(packed), N, K, _ptr(blocks), _stream(stream, packed)),
           "lowbit_unpack_weights")


def lowbit_quantize_act(afmt, x, M, K, xq, xscale, stream=None):
    _check(lib.lowbit_quantize_act(afmt, _ptr(x), M, K, _ptr(xq), _ptr(xscale), _stream(stream, x)),
           "lowbit_quantize_act")


def lowbit_matvec(fmt, W, N, K, w_tensor_scale, afmt, xq, xscale, y, stream=None):
    _check(lib.lowbit_matvec(fmt, _ptr(W), N, K, float(w_tensor_scale), afmt, _ptr(xq), _ptr(xscale), _ptr(y),
                             _stream(stream, y)), "lowbit_matvec")


def lowbit_gemm(fmt, W, N, K, w_tensor_scale, afmt, Xq, Xscale, M, Y, stream=None):
    _check(lib.lowbit_gemm(fmt, _ptr(W), N, K, float(w_tensor_scale), afmt, _ptr(Xq), _ptr(Xscale), M, _ptr(Y),
                           _stream(stream, Y)), "lowbit_gemm")


def lowbit_block_sums(fmt, W, N, K, afmt, Xq, Xscale, M, sums, stream=None):
    _check(lib.lowbit_block_sums(fmt, _ptr(W), N, K, afmt, _ptr(Xq), _ptr(Xscale), M, _ptr(sums),
                                 _stream(stream, sums)), "lowbit_block_sums")


def dense_head_matvec(W, N, K, x, y, stream=None):
    _check(lib.dense_head_matvec(_ptr(W), N, K, _ptr(x), _ptr(y), _stream(stream, y)), "dense_head_matvec")


def lowbit_matvec_popcount(W, N, K, w_tensor_scale, xq, xscale, y, row_sums=None, stream=None):
    _check(lib.lowbit_matvec_popcount(_ptr(W), N, K, float(w_tensor_scale), _ptr(xq), _ptr(xscale), _ptr(y),
                                      _ptr(row_sums), _stream(stream, xq)), "lowbit_matvec_popcount")


def dense_head_matvec_i8(W, row_scale, N, K, x, y, stream=None):
    _check(lib.dense_head_matvec_i8(_ptr(W), _ptr(row_scale), N, K, _ptr(x), _ptr(y), _stream(stream, y)),
           "dense_head_matvec_i8")


class Batch:
    """A work list of decode products prepared once (lowbit_batch_create) and launched by run()."""

    def __init__(self, descs):
        arr = (lb_matvec_desc * len(descs))(*descs)
        handle = ctypes.c_void_p()
        _check(lib.lowbit_batch_create(ctypes.cast(arr, ctypes.c_void_p), len(descs), ctypes.byref(handle)),
               "lowbit_batch_create")
        self._h = handle

    def run(self, stream=None):
        s = _stream(stream) if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib.lowbit_matvec_batched(self._h, s), "lowbit_matvec_batched")

    def close(self):
        if self._h:
            lib.lowbit_batch_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def desc(fmt, W, N, K, xq, xscale, y, w_tensor_scale=1.0, afmt=None, x=None) -> lb_matvec_desc:
    """One work-list entry.  With x (fp32 activations) and afmt ACT_F32_Q8_0 the product quantises x to
    q8_0 in its own launch; xq and xscale are then ignored (pass None)."""
    if afmt is None:
        afmt = ACT_F32_Q8_0 if x is not None else ACT_I8_ROW if fmt in (TERNARY_PLANAR, TERNARY_B3) else ACT_Q8_0
    return lb_matvec_desc(fmt, afmt, N, K, _ptr(W), float(w_tensor_scale), _ptr(xq), _ptr(xscale), _ptr(y), _ptr(x))
