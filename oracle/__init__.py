"""CPU oracle for the packed low-bit x int8 product -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import this
package.  It wraps ``lowbit_oracle.c`` (plain scalar C, single-threaded, built with gcc
``-O2 -ffp-contract=off``) through ctypes and shares nothing with the HIP library.

Parity unpinned: ggml's exact fp32 operation order for the Q1_0/Q2_0_g64/Q8_0 outputs and the absolute
Q1_0 sign polarity relative to ggml (bit 1 is read as +1 here); everything else is pinned by
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lowbit_oracle.c")
_LIB = os.path.join(_HERE, "liblowbit_oracle.so")

Q1_0, Q2_0_G64, TERNARY_PLANAR, Q8_0, TERNARY_B3 = 1, 2, 3, 4, 5
QK8 = 32

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]
# LOWBIT_ORACLE_SANITIZE=1: a separate build with AddressSanitizer and UBSan (any report aborts the run).
# Python must then load the ASan runtime first:
#   LOWBIT_ORACLE_SANITIZE=1 LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#       python -m pytest tests/test_oracle_formats.py tests/test_oracle_quant.py \
#       tests/test_oracle_products.py tests/test_oracle_b3.py -q
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _sanitized() -> bool:
    return os.environ.get("LOWBIT_ORACLE_SANITIZE", "") not in ("", "0")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (a few seconds).  Called by __graft_entry__.build() and on first use."""
    lib_path, flags = _LIB, CFLAGS
    if _sanitized():
        lib_path, flags = _LIB.replace(".so", "_san.so"), CFLAGS + SANITIZE_FLAGS
    if force or not os.path.exists(lib_path) or os.path.getmtime(lib_path) < os.path.getmtime(_SRC):
        tmp = lib_path + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *flags, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, lib_path)
    return lib_path


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "lbo_half_to_float": (ctypes.c_float, [ctypes.c_uint16]),
            "lbo_float_to_half_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "lbo_bf16_to_float": (ctypes.c_float, [ctypes.c_uint16]),
            "lbo_block_weights": (I64, [I]),
            "lbo_block_bytes": (I64, [I]),
            "lbo_weight_bytes": (I64, [I, I64, I64]),
            "lbo_decode": (I, [I, P, I64, I64, P, P]),
            "lbo_encode": (I, [I, P, P, I64, I64, P]),
            "lbo_quantize_q8_0": (I, [P, I64, I64, P, P]),
            "lbo_quantize_i8_row": (I, [P, I64, I64, P, P]),
            "lbo_block_sums_multiply": (I, [I, P, I64, I64, P, P, I64, P]),
            "lbo_block_sums_select": (I, [I, P, I64, I64, P, P, I64, P]),
            "lbo_block_sums_offset": (I, [I, P, I64, I64, P, P, I64, P]),
            "lbo_matvec_q": (I, [I, P, I64, I64, P, P, P, I64, P, P]),
            "lbo_matvec_planar": (I, [P, I64, I64, P, ctypes.c_float, ctypes.c_float, P, I64, P, P]),
            "lbo_head_matvec": (I, [P, I64, I64, P, P, I64, P, P]),
            "lbo_head_matvec_i8": (I, [P, P, I64, I64, P, P, I64, P, P]),
            "lbo_b3_decode": (I, [P, I64, I64, P]),
            "lbo_b3_encode": (I, [P, I64, I64, P]),
            "lbo_matvec_b3": (I, [P, I64, I64, P, ctypes.c_float, ctypes.c_float, P, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(_lib, name)
            f.restype, f.argtypes = res, args
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _rows(rows, N):
    if rows is None:
        return None, N
    r = _c(rows, np.int64)
    return r, r.size


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed (rc={rc})")


# --- conversions ----------------------------------------------------------------------------------

def half_to_float(h: int) -> float:
    return lib().lbo_half_to_float(int(h))


def float_to_half(f: float) -> int:
    return lib().lbo_float_to_half_rne(float(f))


def halves_to_float(h: np.ndarray) -> np.ndarray:
    f = lib().lbo_half_to_float
    return np.array([f(int(v)) for v in np.asarray(h, dtype=np.uint16).ravel()], dtype=np.float32).reshape(
        np.shape(h))


def bf16_to_float(b: int) -> float:
    return lib().lbo_bf16_to_float(int(b))


# --- sizes, decode, encode ----------------------------------------------------------------------

def block_weights(fmt: int) -> int:
    return lib().lbo_block_weights(fmt)


def block_bytes(fmt: int) -> int:
    return lib().lbo_block_bytes(fmt)


def weight_bytes(fmt: int, N: int, K: int) -> int:
    return lib().lbo_weight_bytes(fmt, N, K)


def decode(fmt: int, raw: np.ndarray, N: int, K: int):
    """-> (w int8 [N][K], d float32 [N][K/QK] or None for planar)"""
    raw = _c(raw, np.uint8)
    w = np.empty((N, K), dtype=np.int8)
    d = None if fmt == TERNARY_PLANAR else np.empty((N, K // block_weights(fmt)), dtype=np.float32)
    _check(lib().lbo_decode(fmt, _p(raw), N, K, _p(w), _p(d)), "decode")
    return w, d


def encode(fmt: int, w: np.ndarray, dh, N: int, K: int) -> np.ndarray:
    """w int8 [N][K]; dh binary16 bits [N][K/QK] (ignored for planar) -> format bytes."""
    w = _c(w, np.int8)
    dhc = None if dh is None else _c(dh, np.uint16)
    raw = np.empty(weight_bytes(fmt, N, K), dtype=np.uint8)
    _check(lib().lbo_encode(fmt, _p(w), _p(dhc), N, K, _p(raw)), "encode")
    return raw


# --- quantisers ---------------------------------------------------------------------------------

def quantize_q8_0(x: np.ndarray):
    """x float32 [M][K] -> (q int8 [M][K], dh uint16 binary16 bits [M][K/32])"""
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    dh = np.empty((M, K // QK8), dtype=np.uint16)
    _check(lib().lbo_quantize_q8_0(_p(x), M, K, _p(q), _p(dh)), "quantize_q8_0")
    return q, dh


def quantize_i8_row(x: np.ndarray):
    """x float32 [M][K] -> (q int8 [M][K], s float32 [M])"""
    x = _c(np.atleast_2d(x), np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    _check(lib().lbo_quantize_i8_row(_p(x), M, K, _p(q), _p(s)), "quantize_i8_row")
    return q, s


# --- integer sums and outputs -------------------------------------------------------------------

def _sums(fn, fmt, raw, N, K, q, rows):
    raw = _c(raw, np.uint8)
    q = _c(q, np.int8).ravel()
    r, n = _rows(rows, N)
    out = np.empty((n, K // QK8), dtype=np.int32)
    _check(fn(fmt, _p(raw), N, K, _p(q), _p(r), n, _p(out)), fn.__name__)
    return out


def block_sums(fmt, raw, N, K, q, rows=None, form="multiply"):
    """Exact per-(row, q8_0 block) integer sums, int32 [nrows][K/32]."""
    fn = {"multiply": lib().lbo_block_sums_multiply, "select": lib().lbo_block_sums_select,
          "offset": lib().lbo_block_sums_offset}[form]
    return _sums(fn, fmt, raw, N, K, q, rows)


def matvec_q(fmt, raw, N, K, q, dh, rows=None):
    """ggml-format output in fp64 -> (y float64 [nrows], A float64 [nrows])"""
    raw = _c(raw, np.uint8)
    q = _c(q, np.int8).ravel()
    dh = _c(dh, np.uint16).ravel()
    r, n = _rows(rows, N)
    y = np.empty(n, dtype=np.float64)
    A = np.empty(n, dtype=np.float64)
    _check(lib().lbo_matvec_q(fmt, _p(raw), N, K, _p(q), _p(dh), _p(r), n, _p(y), _p(A)), "matvec_q")
    return y, A


def matvec_planar(raw, N, K, q, s_x, s_w, rows=None):
    """-> (acc int32 [nrows], y float32 [nrows])"""
    raw = _c(raw, np.uint8)
    q = _c(q, np.int8).ravel()
    r, n = _rows(rows, N)
    acc = np.empty(n, dtype=np.int32)
    y = np.empty(n, dtype=np.float32)
    _check(lib().lbo_matvec_planar(_p(raw), N, K, _p(q), float(s_x), float(s_w), _p(r), n, _p(acc), _p(y)),
           "matvec_planar")
    return acc, y


def b3_decode(raw, N, K):
    """base-3 beats -> w int8 [N][K] in {-1, 0, +1}"""
    raw = _c(raw, np.uint8)
    w = np.empty((N, K), dtype=np.int8)
    _check(lib().lbo_b3_decode(_p(raw), N, K, _p(w)), "b3_decode")
    return w


def b3_encode(w, N, K):
    """w int8 [N][K] in {-1, 0, +1} -> base-3 beat bytes"""
    w = _c(w, np.int8)
    raw = np.empty(weight_bytes(TERNARY_B3, N, K), dtype=np.uint8)
    _check(lib().lbo_b3_encode(_p(w), N, K, _p(raw)), "b3_encode")
    return raw


def matvec_b3(raw, N, K, q, s_x, s_w, rows=None):
    """-> (acc int32 [nrows], y float32 [nrows]) with y = ((float)acc * s_x) * s_w"""
    raw = _c(raw, np.uint8)
    q = _c(q, np.int8).ravel()
    r, n = _rows(rows, N)
    acc = np.empty(n, dtype=np.int32)
    y = np.empty(n, dtype=np.float32)
    _check(lib().lbo_matvec_b3(_p(raw), N, K, _p(q), float(s_x), float(s_w), _p(r), n, _p(acc), _p(y)), "matvec_b3")
    return acc, y


def head_matvec(W, N, K, x, rows=None):
    """W uint16 bf16 bits [N][K], x float32 [K] -> (y float64 [nrows], A float64 [nrows])"""
    W = _c(W, np.uint16)
    x = _c(x, np.float32).ravel()
    r, n = _rows(rows, N)
    y = np.empty(n, dtype=np.float64)
    A = np.empty(n, dtype=np.float64)
    _check(lib().lbo_head_matvec(_p(W), N, K, _p(x), _p(r), n, _p(y), _p(A)), "head_matvec")
    return y, A


def head_matvec_i8(W, s_w, N, K, x, rows=None):
    """W int8 [N][K], s_w float32 [N] (one scale per row), x float32 [K] -> (y float64, A float64) [nrows]"""
    W = _c(W, np.int8)
    s_w = _c(s_w, np.float32).ravel()
    x = _c(x, np.float32).ravel()
    r, n = _rows(rows, N)
    y = np.empty(n, dtype=np.float64)
    A = np.empty(n, dtype=np.float64)
    _check(lib().lbo_head_matvec_i8(_p(W), _p(s_w), N, K, _p(x), _p(r), n, _p(y), _p(A)), "head_matvec_i8")
    return y, A


def gemm_q(fmt, raw, N, K, Q, DH, m_rows=None, n_rows=None):
    """Prefill output Y[m][n] for activation rows m (q8_0 rows Q [M][K], DH [M][K/32]) -> (Y, A) fp64."""
    Q = np.atleast_2d(Q)
    DH = np.atleast_2d(DH)
    ms = range(Q.shape[0]) if m_rows is None else list(m_rows)
    Y, A = [], []
    for m in ms:
        y, a = matvec_q(fmt, raw, N, K, Q[m], DH[m], n_rows)
        Y.append(y)
        A.append(a)
    return np.array(Y), np.array(A)


def tolerance_ok(y, y_ref, A, n_terms, rel=1e-5):
    """The fp32 acceptance rule: |y - y_ref| <= rel * max(|y_ref|, A / sqrt(n_terms)) element-wise.

    A is the sum of the magnitudes of the terms being added and n_terms their count: below A/sqrt(n),
    an output is the residue of cancellation and any change of float order moves it by ~2^-24 * A.
    Returns (ok: bool, worst ratio of |error| to its allowance, number of rows where the floor binds)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    floor = np.asarray(A, dtype=np.float64) / np.sqrt(float(n_terms))
    allow = rel * np.maximum(np.abs(y_ref), floor)
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allow > 0, err / allow, np.where(err > 0, np.inf, 0.0))
    return bool(np.all(err <= allow)), float(ratio.max(initial=0.0)), int(np.sum(floor > np.abs(y_ref)))
