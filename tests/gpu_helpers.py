"""Helpers for the GPU parity tests: device buffers with guard bands, the
tolerance check against the fp64 oracle, and the oracle run over row ranges
in host threads (full-size workloads checked on every output in seconds)."""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from dequant_quantized_gemv_amd import synth

# formats of the dequantize and GEMV entry points; the GEMM takes the first three
FMTS = ["q4_0", "q4_1", "q8_0", "q5_0", "q5_1"]
GEMM_FMTS = list(FMTS)  # (Q5_0 / Q5_1 through the register-staged tile)
# fp16 scale ranges of the synthetic weights per format
D_RANGE = {"q4_0": synth.D_Q4, "q4_1": synth.D_Q4, "q8_0": synth.D_Q8, "q5_0": synth.D_Q8,
           "q5_1": synth.D_Q8}
BLOCK_BYTES = {"q4_0": 18, "q4_1": 20, "q8_0": 34, "q5_0": 22, "q5_1": 24}

CANARY_BYTE = 0xA5
GUARD = 4096  # bytes of guard band before and after every output


def torch():
    import torch as _t
    return _t


def to_dev_bytes(arr, offset=0):
    """Copy a uint8 numpy array to the GPU at `offset` bytes past a 256-aligned
    allocation; returns (holder, data_ptr)."""
    t = torch()
    arr = np.array(arr, dtype=np.uint8, copy=True)
    buf = t.empty(arr.size + offset + 16, dtype=t.uint8, device="cuda")
    buf[offset:offset + arr.size].copy_(t.from_numpy(arr))
    return buf, buf.data_ptr() + offset


class Guarded:
    """An output buffer of `nbytes` with canary bands on both sides."""

    def __init__(self, nbytes, offset=0, fill=CANARY_BYTE):
        t = torch()
        self.nbytes = nbytes
        self.offset = offset
        self.buf = t.full((GUARD + offset + nbytes + GUARD,), fill, dtype=t.uint8, device="cuda")
        self.ptr = self.buf.data_ptr() + GUARD + offset

    def host(self, dtype):
        t = torch()
        t.cuda.synchronize()
        raw = self.buf.cpu().numpy()
        body = raw[GUARD + self.offset:GUARD + self.offset + self.nbytes]
        return body.view(dtype)

    def guards_intact(self):
        raw = self.buf.cpu().numpy()
        before = raw[:GUARD + self.offset]
        after = raw[GUARD + self.offset + self.nbytes:]
        return bool(np.all(before == CANARY_BYTE) and np.all(after == CANARY_BYTE))


def x_dev(x2d, ld, dtype, offset_elems=0):
    """Columns x2d[j] (length k) laid out with stride ld elements, starting
    offset_elems past an aligned allocation.  Returns (holder, ptr)."""
    t = torch()
    n, k = x2d.shape
    es = np.dtype(dtype).itemsize
    flat = np.zeros(offset_elems + max(n - 1, 0) * ld + k + 8, dtype=dtype)
    for j in range(n):
        flat[offset_elems + j * ld: offset_elems + j * ld + k] = x2d[j]
    dev = t.from_numpy(flat.view(np.uint8).copy()).to("cuda")
    return dev, dev.data_ptr() + offset_elems * es


def assert_within(y, yref, s, rel, what=""):
    """|y - yref| <= rel * S elementwise; where S == 0 the result must be 0.
    Anything not shown to be within the bound fails: a NaN or infinite output
    (whose comparison is never true) included."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - yref)
    lim = rel * s
    bad = ~(err <= lim)
    zero = s == 0
    bad |= zero & (y != 0)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside {rel}*S; first {idx.tolist()}: "
            f"y={y[bad][:5]} ref={yref[bad][:5]} S={s[bad][:5]}")
    return float(np.max(err / np.where(s > 0, s, 1)))


def host_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def oracle_rows(fn, fmt, w, m, k, *args, **kw):
    """fn(fmt, w_rows, rows, k, *args, **kw) -> (y (n, rows), s (n, rows)),
    called on row ranges of W in host threads (the oracle's C entry points
    release the GIL) and concatenated: the oracle's own result, row for row."""
    rb = (k // 32) * BLOCK_BYTES[fmt]
    threads = host_threads()
    step = max(1, -(-m // (threads * 4)))
    chunks = [(r, min(m, r + step)) for r in range(0, m, step)]
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda c: fn(fmt, w[c[0] * rb:c[1] * rb], c[1] - c[0], k, *args, **kw), chunks))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def gemm_reference(oracle, fmt, w, m, k, xh):
    """Every output of a GEMM against fp16 activations xh (n, k): the fp64
    product of the oracle's fp32 weights with the exactly decoded
    activations, and S = |W| |X| (a matmul as a step; the product itself is
    pinned against the oracle's dot products on the CPU)."""
    rb = (k // 32) * BLOCK_BYTES[fmt]
    threads = host_threads()
    step = max(1, -(-m // (threads * 4)))
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r: oracle.dequantize_f32(fmt, w[r * rb:min(m, r + step) * rb],
                                                             min(m, r + step) - r, k), range(0, m, step)))
    wf = np.concatenate(parts, axis=0).astype(np.float64)
    xf = np.asarray(xh, dtype=np.float16).astype(np.float64)
    return xf @ wf.T, np.abs(xf) @ np.abs(wf).T
