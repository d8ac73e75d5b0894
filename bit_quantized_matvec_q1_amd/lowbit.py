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
    "lowbit_batch_launches": (ctypes.c_int32, [_P]),
    "lowbit_batch_destroy": (None, [_P]),
    "lowbit_matvec_batched_static": (_I, [_P, ctypes.c_int32, _P]),
    "lowbit_read_probe": (_I, [_P, _I64, _P, _P]),
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
    """A device tensor's address (ints pass through as raw addresses, unchecked).  Host tensors and strided
    views are refused: the kernels take dense device buffers, and a host address in a kernel is a memory
    fault."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"device tensor required, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor required (the C ABI takes dense row-major buffers)")
    return t.data_ptr()


_F16_BITS = (torch.uint16, torch.int16, torch.float16)  # binary16 scales travel as their 16-bit patterns
_BF16_BITS = (torch.uint16, torch.int16, torch.bfloat16)


def _check_arg(t, name, count, dtypes=None):
    """Check that tensor t holds at least `count` elements of one of `dtypes` (or, with dtypes None, at
    least `count` bytes of any dtype).  The kernels read and write exactly the extents the sizes imply, so
    a short buffer would be a read or write past its end: refused with ValueError.  None and raw int
    addresses are not checked (raw addresses are the caller's responsibility)."""
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: a torch tensor, an int address or None is required")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not accepted (expected one of {[str(d) for d in dtypes]})")
    have = t.numel() if dtypes is not None else t.numel() * t.element_size()
    if count > 0 and have < count:
        unit = "elements" if dtypes is not None else "bytes"
        raise ValueError(f"{name}: needs at least {count} {unit}, has {have}")


def _args(*specs):
    """Addresses of the arguments (t, name, count[, dtypes]) after checking every one of them: all sizes and
    dtypes first, then the device and layout checks of _ptr."""
    for spec in specs:
        _check_arg(*spec)
    return [_ptr(spec[0]) for spec in specs]


def _pos(*vals):
    """Sizes as the C ABI sees them, for the extents checks: negative ones are left for the library to refuse
    (LB_ESHAPE), and a product with no rows (any size 0 but K) touches no buffer, so all extents are 0."""
    v = [max(int(x), 0) for x in vals]
    if len(v) > 1 and (v[0] == 0 or (len(v) > 2 and v[2] == 0)):  # (N, K[, M]): N == 0 or M == 0
        return [0] * len(v)
    return v


def _wbytes(fmt, N, K):
    n = lib.lowbit_weight_bytes(fmt, N, K)
    return max(n, 0)


def _scale_spec(t, name, afmt, M, K):
    """Activation scales: binary16 [M][K/32] for q8_0, fp32 [M] for per-row int8."""
    if afmt == ACT_I8_ROW:
        return (t, name, M, (torch.float32,))
    return (t, name, M * (K // 32), _F16_BITS)


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
    nb = _wbytes(fmt, N, K)  # the ggml block stream and the device layout have the same byte count
    pb, pp = _args((blocks, "blocks", nb), (packed, "packed", nb))
    _check(lib.lowbit_pack_weights(fmt, pb, N, K, pp, _stream(stream, packed)), "lowbit_pack_weights")


def lowbit_unpack_weights(fmt, packed, N, K, blocks, stream=None):
    nb = _wbytes(fmt, N, K)
    pp, pb = _args((packed, "packed", nb), (blocks, "blocks", nb))
    _check(lib.lowbit_unpack_weights(fmt, pp, N, K, pb, _stream(stream, packed)), "lowbit_unpack_weights")


def lowbit_quantize_act(afmt, x, M, K, xq, xscale, stream=None):
    m, k = _pos(M, K)
    px, pq, ps = _args((x, "x", m * k, (torch.float32,)), (xq, "xq", m * k, (torch.int8,)),
                       _scale_spec(xscale, "xscale", afmt, m, k))
    _check(lib.lowbit_quantize_act(afmt, px, M, K, pq, ps, _stream(stream, x)), "lowbit_quantize_act")


def lowbit_matvec(fmt, W, N, K, w_tensor_scale, afmt, xq, xscale, y, stream=None):
    n, k = _pos(N, K)
    pw, pq, ps, py = _args((W, "W", _wbytes(fmt, n, k)), (xq, "xq", k, (torch.int8,)),
                           _scale_spec(xscale, "xscale", afmt, 1, k), (y, "y", n, (torch.float32,)))
    _check(lib.lowbit_matvec(fmt, pw, N, K, float(w_tensor_scale), afmt, pq, ps, py, _stream(stream, y)),
           "lowbit_matvec")


def lowbit_gemm(fmt, W, N, K, w_tensor_scale, afmt, Xq, Xscale, M, Y, stream=None):
    n, k, m = _pos(N, K, M)
    pw, pq, ps, py = _args((W, "W", _wbytes(fmt, n, k)), (Xq, "Xq", m * k, (torch.int8,)),
                           _scale_spec(Xscale, "Xscale", afmt, m, k), (Y, "Y", m * n, (torch.float32,)))
    _check(lib.lowbit_gemm(fmt, pw, N, K, float(w_tensor_scale), afmt, pq, ps, M, py, _stream(stream, Y)),
           "lowbit_gemm")


def lowbit_block_sums(fmt, W, N, K, afmt, Xq, Xscale, M, sums, stream=None):
    n, k, m = _pos(N, K, M)
    per_row = fmt in (TERNARY_PLANAR, TERNARY_B3)  # one sum per row; else one per 32-block of K
    pw, pq, ps, pz = _args((W, "W", _wbytes(fmt, n, k)), (Xq, "Xq", m * k, (torch.int8,)),
                           _scale_spec(Xscale, "Xscale", afmt, m, k),
                           (sums, "sums", m * n * (1 if per_row else k // 32), (torch.int32,)))
    _check(lib.lowbit_block_sums(fmt, pw, N, K, afmt, pq, ps, M, pz, _stream(stream, sums)), "lowbit_block_sums")


def dense_head_matvec(W, N, K, x, y, stream=None):
    n, k = _pos(N, K)
    pw, px, py = _args((W, "W", n * k, _BF16_BITS), (x, "x", k, (torch.float32,)), (y, "y", n, (torch.float32,)))
    _check(lib.dense_head_matvec(pw, N, K, px, py, _stream(stream, y)), "dense_head_matvec")


def lowbit_matvec_popcount(W, N, K, w_tensor_scale, xq, xscale, y, row_sums=None, stream=None):
    n, k = _pos(N, K)
    pw, pq, ps, py, pr = _args((W, "W", _wbytes(TERNARY_PLANAR, n, k)), (xq, "xq", k, (torch.int8,)),
                               (xscale, "xscale", 1, (torch.float32,)), (y, "y", n, (torch.float32,)),
                               (row_sums, "row_sums", n, (torch.int32,)))
    _check(lib.lowbit_matvec_popcount(pw, N, K, float(w_tensor_scale), pq, ps, py, pr, _stream(stream, xq)),
           "lowbit_matvec_popcount")


def dense_head_matvec_i8(W, row_scale, N, K, x, y, stream=None):
    n, k = _pos(N, K)
    pw, pr, px, py = _args((W, "W", n * k, (torch.int8,)), (row_scale, "row_scale", n, (torch.float32,)),
                           (x, "x", k, (torch.float32,)), (y, "y", n, (torch.float32,)))
    _check(lib.dense_head_matvec_i8(pw, pr, N, K, px, py, _stream(stream, y)), "dense_head_matvec_i8")


def lowbit_read_probe(buf, nbytes, sink, stream=None):
    pb, ps = _args((buf, "buf", nbytes), (sink, "sink", 65536, (torch.int32, torch.uint32)))
    _check(lib.lowbit_read_probe(pb, nbytes, ps, _stream(stream, buf)), "lowbit_read_probe")


class Batch:
    """A work list of decode products prepared once (lowbit_batch_create) and launched by run().  The batch
    holds the tensors its descriptors point to until close(), so none of them can be freed (and its memory
    handed to another tensor) while the batch can still write into it."""

    def __init__(self, descs):
        arr = (lb_matvec_desc * len(descs))(*descs)
        handle = ctypes.c_void_p()
        _check(lib.lowbit_batch_create(ctypes.cast(arr, ctypes.c_void_p), len(descs), ctypes.byref(handle)),
               "lowbit_batch_create")
        self._h = handle
        self._keep = [getattr(d, "_tensors", ()) for d in descs]

    def run(self, stream=None):
        if not self._h:
            raise ValueError("batch is closed")
        s = _stream(stream) if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib.lowbit_matvec_batched(self._h, s), "lowbit_matvec_batched")

    def launches(self):
        """Kernel launches one run() makes (lowbit_batch_launches)."""
        if not self._h:
            raise ValueError("batch is closed")
        return int(lib.lowbit_batch_launches(self._h))

    def close(self):
        if self._h:
            lib.lowbit_batch_destroy(self._h)
            self._h = None
        self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def desc(fmt, W, N, K, xq, xscale, y, w_tensor_scale=1.0, afmt=None, x=None) -> lb_matvec_desc:
    """One work-list entry, its buffers checked against the sizes like lowbit_matvec's.  With x (fp32
    activations) and afmt ACT_F32_Q8_0 the product quantises x to q8_0 in its own launch; xq and xscale
    are then ignored (pass None).  The entry keeps references to its tensors (a Batch built from it holds
    them)."""
    if afmt is None:
        afmt = ACT_F32_Q8_0 if x is not None else ACT_I8_ROW if fmt in (TERNARY_PLANAR, TERNARY_B3) else ACT_Q8_0
    n, k = _pos(N, K)
    if afmt == ACT_F32_Q8_0:
        pw, py, px = _args((W, "W", _wbytes(fmt, n, k)), (y, "y", n, (torch.float32,)), (x, "x", k, (torch.float32,)))
        pq, ps = _ptr(xq), _ptr(xscale)
    else:
        pw, py, pq, ps = _args((W, "W", _wbytes(fmt, n, k)), (y, "y", n, (torch.float32,)),
                               (xq, "xq", k, (torch.int8,)), _scale_spec(xscale, "xscale", afmt, 1, k))
        px = _ptr(x)
    d = lb_matvec_desc(fmt, afmt, N, K, pw, float(w_tensor_scale), pq, ps, py, px)
    d._tensors = tuple(t for t in (W, xq, xscale, y, x) if isinstance(t, torch.Tensor))
    return d
