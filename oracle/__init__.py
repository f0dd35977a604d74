"""CPU oracle for ggml block-quantized dequantize / GEMV / GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg import this module.  The GPU library never
does, and the two share no code.

The arithmetic lives in ``qk_oracle.cpp`` (plain C++ with a C interface,
fp64 accumulation, no FMA contraction); this module is numpy marshalling
around it.  Function by function, the source cites the passages of the "llama_cpp 0.12.1 -> 0.12.2"
ggml-cuda.cu diff page that each step follows.

Layout conventions (ggml's: ne0 is the contiguous dimension):
  * W: ``rows`` rows of ``k`` weights, each row k/32 blocks back to back.
  * X: ``n`` activation columns of length ``k``; column j starts at j*ldx.
  * Y: ``n`` output columns of length ``m``; returned as an (n, m) array.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FORMATS = {"q4_0": 0, "q4_1": 1, "q8_0": 2, "q5_0": 3, "q5_1": 4}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.orc_half_to_float.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_float.restype = ctypes.c_float
    lib.orc_float_to_half.argtypes = [ctypes.c_float]
    lib.orc_float_to_half.restype = ctypes.c_uint16
    lib.orc_block_bytes.argtypes = [ctypes.c_int]
    lib.orc_block_bytes.restype = ctypes.c_int
    lib.orc_code.argtypes = [ctypes.c_int, u8p, ctypes.c_int]
    lib.orc_code.restype = ctypes.c_int
    lib.orc_value.argtypes = [ctypes.c_int, u8p, ctypes.c_int]
    lib.orc_value.restype = ctypes.c_float
    lib.orc_dequantize_f32.argtypes = [ctypes.c_int, vp, i64, i64, vp]
    lib.orc_dequantize_f32.restype = None
    lib.orc_dequantize_f16.argtypes = [ctypes.c_int, vp, i64, i64, vp]
    lib.orc_dequantize_f16.restype = None
    lib.orc_dot.argtypes = [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, i64, i64, vp, vp]
    lib.orc_dot.restype = None
    lib.orc_dot_entries.argtypes = [ctypes.c_int, vp, i64, vp, ctypes.c_int, i64,
                                    vp, vp, i64, vp, vp]
    lib.orc_dot_entries.restype = None
    lib.orc_dot_id.argtypes = [ctypes.c_int, vp, i64, i64, i64, i64, vp, i64, i64, i64,
                               vp, i64, i64, vp, vp]
    lib.orc_dot_id.restype = None
    lib.orc_quantize_x8_block.argtypes = [vp, vp]
    lib.orc_quantize_x8_block.restype = ctypes.c_float
    lib.orc_quantize_x8.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.orc_quantize_x8.restype = None
    lib.orc_dot_x8.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64, vp, vp]
    lib.orc_dot_x8.restype = None
    _lib = lib
    return lib


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    return FORMATS[fmt]


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def half_to_float(bits):
    """Exact binary16 -> fp32 for one 16-bit pattern."""
    return _load().orc_half_to_float(int(bits))


def float_to_half(v):
    """fp32 -> binary16 bits, round to nearest even."""
    return _load().orc_float_to_half(float(np.float32(v)))


def halves_to_float(bits):
    """Vector form of half_to_float (loops in Python; small inputs only)."""
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    lib = _load()
    return np.array([lib.orc_half_to_float(int(b)) for b in bits], dtype=np.float32)


def floats_to_half(vals):
    """Vector form of float_to_half (loops in Python; small inputs only)."""
    vals = np.asarray(vals, dtype=np.float32).ravel()
    lib = _load()
    return np.array([lib.orc_float_to_half(float(v)) for v in vals], dtype=np.uint16)


def block_bytes(fmt):
    return _load().orc_block_bytes(_fmt(fmt))


def _check_w(fmt, w, rows, k):
    if k % 32 != 0:
        raise ValueError("k must be a multiple of 32")
    w = np.ascontiguousarray(np.asarray(w, dtype=np.uint8).ravel())
    need = rows * (k // 32) * block_bytes(fmt)
    if w.size < need:
        raise ValueError(f"weight buffer holds {w.size} bytes, needs {need}")
    return w


def code(fmt, block, t):
    """Integer code of element t of one block (bytes)."""
    b = np.ascontiguousarray(np.asarray(block, dtype=np.uint8))
    return _load().orc_code(_fmt(fmt), b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), int(t))


def value(fmt, block, t):
    """fp32 value of element t of one block (bytes)."""
    b = np.ascontiguousarray(np.asarray(block, dtype=np.uint8))
    return _load().orc_value(_fmt(fmt), b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), int(t))


def dequantize_f32(fmt, w, rows, k):
    w = _check_w(fmt, w, rows, k)
    out = np.empty(rows * k, dtype=np.float32)
    _load().orc_dequantize_f32(_fmt(fmt), _ptr(w), rows, k, _ptr(out))
    return out.reshape(rows, k)


def dequantize_f16(fmt, w, rows, k):
    """Returns binary16 bit patterns (uint16)."""
    w = _check_w(fmt, w, rows, k)
    out = np.empty(rows * k, dtype=np.uint16)
    _load().orc_dequantize_f16(_fmt(fmt), _ptr(w), rows, k, _ptr(out))
    return out.reshape(rows, k)


def _check_x(x, k, n, ldx, x_is_f16):
    dt = np.uint16 if x_is_f16 else np.float32
    x = np.ascontiguousarray(np.asarray(x).ravel())
    if x.dtype != dt:
        raise TypeError(f"x must be {np.dtype(dt).name} (got {x.dtype})")
    if n > 0 and x.size < (n - 1) * ldx + k:
        raise ValueError("x buffer too small for n, ldx, k")
    return x


def dot(fmt, w, m, k, x, n, ldx=None, x_is_f16=False):
    """fp64 y[j, i] = sum_c W[i,c] X[c,j] and s[j, i] = sum_c |W[i,c] X[c,j]|.

    ``x`` is fp32, or binary16 bit patterns (uint16) when x_is_f16.
    Returns (y, s), each of shape (n, m), float64.
    """
    ldx = k if ldx is None else ldx
    w = _check_w(fmt, w, m, k)
    x = _check_x(x, k, n, ldx, x_is_f16)
    y = np.empty(n * m, dtype=np.float64)
    s = np.empty(n * m, dtype=np.float64)
    _load().orc_dot(_fmt(fmt), _ptr(w), m, k, _ptr(x), int(bool(x_is_f16)), ldx, n,
                    _ptr(y), _ptr(s))
    return y.reshape(n, m), s.reshape(n, m)


def dot_entries(fmt, w, m, k, x, ldx, ii, jj, x_is_f16=False):
    """Like dot() but only for entries (ii[e], jj[e]); returns (y, s) of shape (count,)."""
    w = _check_w(fmt, w, m, k)
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    if ii.shape != jj.shape:
        raise ValueError("ii and jj must have the same shape")
    if ii.size and (ii.min() < 0 or ii.max() >= m or jj.min() < 0):
        raise ValueError("entry index out of range")
    n = int(jj.max()) + 1 if jj.size else 0
    x = _check_x(x, k, n, ldx, x_is_f16)
    y = np.empty(ii.size, dtype=np.float64)
    s = np.empty(ii.size, dtype=np.float64)
    _load().orc_dot_entries(_fmt(fmt), _ptr(w), k, _ptr(x), int(bool(x_is_f16)), ldx,
                            _ptr(ii), _ptr(jj), ii.size, _ptr(y), _ptr(s))
    return y, s


def dot_id(fmt, w, n_experts, expert_stride, m, k, ids, n_used, n_tokens, x,
           x_slot, x_tok, ld_ids=None):
    """Expert-indexed products (mixture-of-experts decode).

    For token t and slot s, expert e = ids[t*ld_ids + s] (matrix at byte
    e*expert_stride of ``w``) times the fp32 vector x[t*x_tok + s*x_slot :][:k].
    Returns (y, s) of shape (n_tokens, n_used, m), float64; an id outside
    [0, n_experts) gives NaN rows.
    """
    ld_ids = n_used if ld_ids is None else ld_ids
    w = np.ascontiguousarray(np.asarray(w, dtype=np.uint8).ravel())
    if k % 32 != 0:
        raise ValueError("k must be a multiple of 32")
    if expert_stride < m * (k // 32) * block_bytes(fmt):
        raise ValueError("expert_stride smaller than one expert matrix")
    if n_experts > 0 and w.size < (n_experts - 1) * expert_stride + m * (k // 32) * block_bytes(fmt):
        raise ValueError("weight buffer too small for the expert stack")
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
    if n_tokens > 0 and ids.size < (n_tokens - 1) * ld_ids + n_used:
        raise ValueError("ids buffer too small")
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    if n_tokens > 0 and n_used > 0 and x.size < (n_tokens - 1) * x_tok + (n_used - 1) * x_slot + k:
        raise ValueError("x buffer too small")
    y = np.empty(n_tokens * n_used * m, dtype=np.float64)
    s = np.empty(n_tokens * n_used * m, dtype=np.float64)
    _load().orc_dot_id(_fmt(fmt), _ptr(w), n_experts, expert_stride, m, k, _ptr(ids), ld_ids,
                       n_used, n_tokens, _ptr(x), x_slot, x_tok, _ptr(y), _ptr(s))
    return y.reshape(n_tokens, n_used, m), s.reshape(n_tokens, n_used, m)


def quantize_x8(x, k, n, ldx=None):
    """8-bit activation codes with power-of-two block scales.

    Returns (q, d): q int8 of shape (n, k), d float32 of shape (n, k/32)."""
    ldx = k if ldx is None else ldx
    if k % 32 != 0:
        raise ValueError("k must be a multiple of 32")
    x = _check_x(x, k, n, ldx, False)
    q = np.empty(n * k, dtype=np.int8)
    d = np.empty(n * (k // 32), dtype=np.float32)
    _load().orc_quantize_x8(_ptr(x), k, n, ldx, _ptr(q), _ptr(d))
    return q.reshape(n, k), d.reshape(n, k // 32)


def dot_x8(fmt, w, m, k, x, n, ldx=None):
    """Products with the 8-bit-quantized activations (fp64) and their
    tolerance scale; returns (y, s), each of shape (n, m)."""
    ldx = k if ldx is None else ldx
    w = _check_w(fmt, w, m, k)
    x = _check_x(x, k, n, ldx, False)
    y = np.empty(n * m, dtype=np.float64)
    s = np.empty(n * m, dtype=np.float64)
    _load().orc_dot_x8(_fmt(fmt), _ptr(w), m, k, _ptr(x), n, ldx, _ptr(y), _ptr(s))
    return y.reshape(n, m), s.reshape(n, m)
