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
QK_Q4_0, QK_Q4_1, QK_Q8_0 = 1, 2, 3
QK_F32, QK_F16 = 0, 1
QK_OK, QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED, QK_ERR_ALIGNMENT, QK_ERR_LAUNCH = 0, 1, 2, 3, 4

FORMATS = {"q4_0": QK_Q4_0, "q4_1": QK_Q4_1, "q8_0": QK_Q8_0}
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
# ---------------------------------------------------------------------------

def dequantize(fmt, w, rows, k, out_dtype="f32", out=None, stream=None):
    """Dequantize a rows x k matrix held as block bytes in a uint8 CUDA tensor."""
    import torch
    dt = {"f32": (QK_F32, torch.float32), "f16": (QK_F16, torch.float16)}[out_dtype]
    if out is None:
        out = torch.empty((rows, k), dtype=dt[1], device=w.device)
    st = qk_dequantize(fmt, w.data_ptr(), rows, k, dt[0], out.data_ptr(), _stream(stream))
    _check(st, "qk_dequantize")
    return out


def mul_mat_vec(fmt, w, m, k, x, y=None, stream=None):
    """y (n, m) = x (n, k) @ W^T for 1..8 fp32 columns; rows of x and y are the
    ggml columns (contiguous, ldx = x.stride(0), ldy = y.stride(0))."""
    import torch
    if x.dim() == 1:
        x = x.view(1, -1)
    n = x.shape[0]
    if x.dtype != torch.float32 or x.stride(1) != 1:
        raise TypeError("x must be float32 with contiguous columns")
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
    st = qk_mul_mat_vec(fmt, w.data_ptr(), m, k, x.data_ptr(), n, x.stride(0),
                        y.data_ptr(), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat_vec")
    return y


def mul_mat_vec_x8(fmt, w, m, k, x, y=None, stream=None):
    """As mul_mat_vec, with the activations quantized to 8 bits per 32-element
    block inside the kernel and integer dot products (qk_mul_mat_vec_x8)."""
    import torch
    if x.dim() == 1:
        x = x.view(1, -1)
    n = x.shape[0]
    if x.dtype != torch.float32 or x.stride(1) != 1:
        raise TypeError("x must be float32 with contiguous columns")
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
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
    n = problems[0][3].shape[0] if problems[0][3].dim() == 2 else 1
    if ys is None:
        ys = [torch.empty((n, m), dtype=torch.float32, device=x.device) for (_, m, _, x) in problems]
    tup = []
    for (w, m, k, x), y in zip(problems, ys):
        x2 = x.view(1, -1) if x.dim() == 1 else x
        if x2.dtype != torch.float32 or x2.stride(1) != 1 or x2.shape[0] != n:
            raise TypeError("every x must be float32 (n, k) with contiguous columns and the same n")
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
    if ids.dtype != torch.int32 or ids.dim() != 2 or ids.stride(1) != 1:
        raise TypeError("ids must be int32 (n_tokens, n_used) with contiguous rows")
    n_tokens, n_used = ids.shape
    if x.dtype != torch.float32 or x.stride(-1) != 1:
        raise TypeError("x must be float32 with contiguous vectors")
    if x.dim() == 2:
        x_slot, x_tok = 0, x.stride(0)
    elif x.dim() == 3:
        x_slot, x_tok = x.stride(1), x.stride(0)
    else:
        raise TypeError("x must be (n_tokens, k) or (n_tokens, n_used, k)")
    if expert_stride is None:
        expert_stride = m * row_bytes(fmt, k)
    if y is None:
        y = torch.empty((n_tokens, n_used, m), dtype=torch.float32, device=x.device)
    st = qk_mul_mat_vec_id(fmt, w.data_ptr(), n_experts, expert_stride, m, k, ids.data_ptr(),
                           ids.stride(0), n_used, n_tokens, x.data_ptr(), x_slot, x_tok,
                           y.data_ptr(), y.stride(1), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat_vec_id")
    return y


def mul_mat(fmt, w, m, k, x, y=None, stream=None):
    """y (n, m) = x (n, k, fp16) @ f16(W)^T on the matrix cores."""
    import torch
    n = x.shape[0]
    if x.dtype != torch.float16 or x.stride(1) != 1:
        raise TypeError("x must be float16 with contiguous columns")
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
    st = qk_mul_mat(fmt, w.data_ptr(), m, k, x.data_ptr(), n, x.stride(0),
                    y.data_ptr(), y.stride(0), _stream(stream))
    _check(st, "qk_mul_mat")
    return y
