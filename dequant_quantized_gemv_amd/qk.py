"""Thin Python binding of libqk (include/qk.h).

Argument marshalling only: tensors are passed as device pointers with the
current HIP stream; every step of the computation runs in the library's gfx950
kernels.  The library must be built (``python -m dequant_quantized_gemv_amd.build``
or ``__graft_entry__.build()``); loading fails loudly otherwise, and there is no
CPU fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqk.so")

# enum qk_format / qk_dtype / qk_status (include/qk.h)
QK_Q4_0, QK_Q4_1, QK_Q8_0, QK_Q5_0, QK_Q5_1 = 1, 2, 3, 4, 5
QK_F32, QK_F16 = 0, 1
QK_OK, QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED, QK_ERR_ALIGNMENT, QK_ERR_LAUNCH = 0, 1, 2, 3, 4

FORMATS = {"q4_0": QK_Q4_0, "q4_1": QK_Q4_1, "q8_0": QK_Q8_0, "q5_0": QK_Q5_0, "q5_1": QK_Q5_1}
SYMBOLS = ("qk_block_bytes", "qk_row_bytes", "qk_status_string", "qk_version",
           "qk_dequantize", "qk_mul_mat_vec", "qk_mul_mat_vec_x8", "qk_mul_mat_vec_batched",
           "qk_mul_mat_vec_id", "qk_mul_mat")
QK_MAX_BATCH = 16


class MatVecItem(ctypes.Structure):
    """struct qk_mat_vec_item (include/qk.h)."""
    _fields_ = [("w", ctypes.c_void_p), ("m", ctypes.c_int64), ("k", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class QKError(RuntimeError):
    def __init__(self, status, call):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} (status {status})")


_lib = None


def load():
    """Load libqk.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m dequant_quantized_gemv_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.qk_block_bytes.argtypes = [ci]
    lib.qk_block_bytes.restype = ctypes.c_size_t
    lib.qk_row_bytes.argtypes = [ci, i64]
    lib.qk_row_bytes.restype = ctypes.c_size_t
    lib.qk_status_string.argtypes = [ci]
    lib.qk_status_string.restype = ctypes.c_char_p
    lib.qk_version.argtypes = []
    lib.qk_version.restype = ci
    lib.qk_dequantize.argtypes = [ci, vp, i64, i64, ci, vp, vp]
    lib.qk_dequantize.restype = ci
    lib.qk_mul_mat_vec.argtypes = [ci, vp, i64, i64, vp, i64, i64, vp, i64, vp]
    lib.qk_mul_mat_vec.restype = ci
    lib.qk_mul_mat_vec_x8.argtypes = [ci, vp, i64, i64, vp, i64, i64, vp, i64, vp]
    lib.qk_mul_mat_vec_x8.restype = ci
    lib.qk_mul_mat_vec_batched.argtypes = [ci, ctypes.POINTER(MatVecItem), ci, i64, vp]
    lib.qk_mul_mat_vec_batched.restype = ci
    lib.qk_mul_mat_vec_id.argtypes = [ci, vp, i64, i64, i64, i64, vp, i64, i64, i64,
                                      vp, i64, i64, vp, i64, i64, vp]
    lib.qk_mul_mat_vec_id.restype = ci
    lib.qk_mul_mat.argtypes = [ci, vp, i64, i64, vp, i64, i64, vp, i64, vp]
    lib.qk_mul_mat.restype = ci
    _lib = lib
    return lib


def status_string(status):
    return load().qk_status_string(int(status)).decode()


def block_bytes(fmt):
    return load().qk_block_bytes(_fmt(fmt))


def row_bytes(fmt, k):
    return load().qk_row_bytes(_fmt(fmt), int(k))


def _fmt(fmt):
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}")
        return FORMATS[fmt]
    return int(fmt)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream) if not hasattr(stream, "cuda_stream") else stream.cuda_stream


def _check(status, call):
    if status != QK_OK:
        raise QKError(status, call)


# ---------------------------------------------------------------------------
# Raw entry points (pointers and sizes, same names and argument order as C)
# ---------------------------------------------------------------------------

def qk_dequantize(fmt, w_ptr, rows, k, out_dtype, out_ptr, stream=0):
    return load().qk_dequantize(_fmt(fmt), w_ptr, rows, k, out_dtype, out_ptr, stream)


def qk_mul_mat_vec(fmt, w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream=0):
    return load().qk_mul_mat_vec(_fmt(fmt), w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream)


def qk_mul_mat_vec_x8(fmt, w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream=0):
    return load().qk_mul_mat_vec_x8(_fmt(fmt), w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream)


def make_items(items):
    """ctypes array of MatVecItem from (w_ptr, m, k, x_ptr, ldx, y_ptr, ldy) tuples."""
    arr = (MatVecItem * max(len(items), 1))()
    for i, it in enumerate(items):
        arr[i] = MatVecItem(*it)
    return arr


def qk_mul_mat_vec_batched(fmt, items, count, n, stream=0):
    """items: a ctypes MatVecItem array (see make_items) or None."""
    return load().qk_mul_mat_vec_batched(_fmt(fmt), items, count, n, stream)


def qk_mul_mat_vec_id(fmt, w_ptr, n_experts, expert_stride, m, k, ids_ptr, ld_ids, n_used,
                      n_tokens, x_ptr, x_slot, x_tok, y_ptr, y_slot, y_tok, stream=0):
    return load().qk_mul_mat_vec_id(_fmt(fmt), w_ptr, n_experts, expert_stride, m, k, ids_ptr,
                                    ld_ids, n_used, n_tokens, x_ptr, x_slot, x_tok, y_ptr,
                                    y_slot, y_tok, stream)


def qk_mul_mat(fmt, w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream=0):
    return load().qk_mul_mat(_fmt(fmt), w_ptr, m, k, x_ptr, n, ldx, y_ptr, ldy, stream)


# ---------------------------------------------------------------------------
# torch-tensor conveniences (allocation by torch, compute by libqk)
#
# The C ABI sees only pointers, so these wrappers check every tensor on the
# host before anything is launched: dtype, shape, a contiguous innermost
# dimension, enough weight bytes, one CUDA device for all operands.  A
# mismatch raises TypeError or ValueError and enqueues nothing.
# ---------------------------------------------------------------------------

_BLOCK_BYTES = {QK_Q4_0: 18, QK_Q4_1: 20, QK_Q8_0: 34, QK_Q5_0: 22, QK_Q5_1: 24}


def _weight_check(fmt, w, rows, k):
    import torch
    code = _fmt(fmt)
    if code not in _BLOCK_BYTES:
        raise ValueError(f"unknown format {fmt!r}")
    if rows < 0 or k < 0 or k % 32 != 0:
        raise ValueError(f"bad shape rows={rows}, k={k} (k must be a non-negative multiple of 32)")
    if not isinstance(w, torch.Tensor) or w.dtype != torch.uint8:
        raise TypeError("w must be a uint8 tensor of block bytes")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    need = rows * (k // 32) * _BLOCK_BYTES[code]
    if w.numel() < need:
        raise ValueError(f"w holds {w.numel()} bytes, a {rows} x {k} matrix needs {need}")


def _cols_check(t, name, dtype, n, length):
    """t is (n, >= length) of dtype with contiguous rows (ggml columns)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} tensor")
    if t.dim() != 2 or t.shape[0] != n or t.shape[1] < length:
        raise ValueError(f"{name} must have shape ({n}, >= {length}), got {tuple(t.shape)}")
    if n > 0 and length > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous columns (stride(1) == 1)")


def _same_device(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a CUDA device")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def dequantize(fmt, w, rows, k, out_dtype="f32", out=None, stream=None):
    """Dequantize a rows x k matrix held as block bytes in a uint8 CUDA tensor."""
    import torch
    if out_dtype not in ("f32", "f16"):
        raise ValueError(f"out_dtype must be 'f32' or 'f16', got {out_dtype!r}")
    dt = {"f32": (QK_F32, torch.float32), "f16": (QK_F16, torch.float16)}[out_dtype]
    _weight_check(fmt, w, rows, k)
    if out is None:
        out = torch.empty((rows, k), dtype=dt[1], device=w.device)
    if not isinstance(out, torch.Tensor) or out.dtype != dt[1]:
        raise TypeError(f"out must be a {dt[1]} tensor for out_dtype {out_dtype!r}")
    if tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous ({rows}, {k}) tensor")
    _same_device(w, out)
    st = qk_dequantize(fmt, w.data_ptr(), rows, k, dt[0], out.data_ptr(), _stream(stream))
    _check(st, "qk_dequantize")
    return out


def _gemv_args(fmt, w, m, k, x, y):
    import torch
    if x.dim() == 1:
        x = x.view(1, -1)
    n = x.shape[0]
    if not 1 <= n <= 8:
        raise ValueError(f"1..8 activation columns, got {n}")
    _weight_check(fmt, w, m, k)
    _cols_check(x, "x", torch.float32, n, k)
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
    _cols_check(y, "y", torch.float32, n, m)
    _same_device(w, x, y)
    return x, y, n


def mul_mat_vec(fmt, w, m, k, x, y=None, stream=None):
    """y (n, m) = x (n, k) @ W^T for 1..8 fp32 columns; rows of x and y are the
    ggml columns (contiguous, ldx = x.stride(0), ldy = y.stride(0))."""
    x, y, n = _gemv_args(fmt, w, m, k, x, y)
    st = qk_mul_mat_vec(fmt, w.data_ptr(), m, k, x.data_ptr(), n, x.stride(0),
                        y.data_ptr(), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat_vec")
    return y


def mul_mat_vec_x8(fmt, w, m, k, x, y=None, stream=None):
    """As mul_mat_vec, with the activations quantized to 8 bits per 32-element
    block inside the kernel and integer dot products (qk_mul_mat_vec_x8)."""
    x, y, n = _gemv_args(fmt, w, m, k, x, y)
    st = qk_mul_mat_vec_x8(fmt, w.data_ptr(), m, k, x.data_ptr(), n, x.stride(0),
                           y.data_ptr(), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat_vec_x8")
    return y


def mul_mat_vec_batched(fmt, problems, ys=None, stream=None):
    """One launch for several GEMVs of one format and column count.
    problems: list of (w, m, k, x) with x shaped (n, k) fp32; returns the ys."""
    import torch
    if not problems:
        return []
    if len(problems) > QK_MAX_BATCH:
        raise ValueError(f"at most {QK_MAX_BATCH} problems per launch")
    n = problems[0][3].shape[0] if problems[0][3].dim() == 2 else 1
    if ys is None:
        ys = [torch.empty((n, m), dtype=torch.float32, device=x.device) for (_, m, _, x) in problems]
    if len(ys) != len(problems):
        raise ValueError("one output per problem")
    tup = []
    for (w, m, k, x), y in zip(problems, ys):
        x2 = x.view(1, -1) if x.dim() == 1 else x
        if x2.shape[0] != n:
            raise ValueError("every x must have the same number of columns")
        x2, y, _ = _gemv_args(fmt, w, m, k, x2, y)
        _same_device(problems[0][0], w)
        tup.append((w.data_ptr(), m, k, x2.data_ptr(), x2.stride(0), y.data_ptr(), y.stride(0)))
    arr = make_items(tup)
    st = qk_mul_mat_vec_batched(fmt, arr, len(tup), n, _stream(stream))
    _check(st, "qk_mul_mat_vec_batched")
    return ys


def mul_mat_vec_id(fmt, w, n_experts, m, k, ids, x, y=None, expert_stride=None, stream=None):
    """Expert-indexed GEMV: y[t, s] = W[ids[t, s]] @ x[t] (x shaped (n_tokens, k),
    shared by a token's slots) or x[t, s] (x shaped (n_tokens, n_used, k)).
    w: uint8 CUDA tensor holding n_experts matrices, expert_stride bytes apart
    (default: packed); ids: int32 CUDA tensor (n_tokens, n_used).  Returns y
    shaped (n_tokens, n_used, m) fp32."""
    import torch
    if not isinstance(ids, torch.Tensor) or ids.dtype != torch.int32 or ids.dim() != 2 or ids.stride(1) != 1:
        raise TypeError("ids must be int32 (n_tokens, n_used) with contiguous rows")
    n_tokens, n_used = ids.shape
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.stride(-1) != 1:
        raise TypeError("x must be float32 with contiguous vectors")
    if x.dim() == 2 and x.shape[0] == n_tokens and x.shape[1] >= k:
        x_slot, x_tok = 0, x.stride(0)
    elif x.dim() == 3 and tuple(x.shape[:2]) == (n_tokens, n_used) and x.shape[2] >= k:
        x_slot, x_tok = x.stride(1), x.stride(0)
    else:
        raise ValueError(f"x must be ({n_tokens}, >= {k}) or ({n_tokens}, {n_used}, >= {k}), "
                         f"got {tuple(x.shape)}")
    one = m * (k // 32) * _BLOCK_BYTES.get(_fmt(fmt), 0)
    if expert_stride is None:
        expert_stride = one
    if n_experts < 1 or expert_stride < one:
        raise ValueError("n_experts >= 1 and expert_stride >= one expert matrix")
    _weight_check(fmt, w, m, k)
    if w.numel() < (n_experts - 1) * expert_stride + one:
        raise ValueError(f"w holds {w.numel()} bytes, the stack needs {(n_experts - 1) * expert_stride + one}")
    if y is None:
        y = torch.empty((n_tokens, n_used, m), dtype=torch.float32, device=x.device)
    if not isinstance(y, torch.Tensor) or y.dtype != torch.float32:
        raise TypeError("y must be a float32 tensor")
    if tuple(y.shape) != (n_tokens, n_used, m) or (m > 0 and y.stride(2) != 1):
        raise ValueError(f"y must have shape ({n_tokens}, {n_used}, {m}) with contiguous rows")
    _same_device(w, ids, x, y)
    st = qk_mul_mat_vec_id(fmt, w.data_ptr(), n_experts, expert_stride, m, k, ids.data_ptr(),
                           ids.stride(0), n_used, n_tokens, x.data_ptr(), x_slot, x_tok,
                           y.data_ptr(), y.stride(1), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat_vec_id")
    return y


def mul_mat(fmt, w, m, k, x, y=None, stream=None):
    """y (n, m) = x (n, k, fp16) @ f16(W)^T on the matrix cores."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise TypeError("x must be a 2-D float16 tensor (n, k)")
    n = x.shape[0]
    _weight_check(fmt, w, m, k)
    _cols_check(x, "x", torch.float16, n, k)
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
    _cols_check(y, "y", torch.float32, n, m)
    _same_device(w, x, y)
    st = qk_mul_mat(fmt, w.data_ptr(), m, k, x.data_ptr(), n, x.stride(0),
                    y.data_ptr(), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat")
    return y
