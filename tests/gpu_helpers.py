"""Helpers for the GPU parity tests: device buffers with guard bands, and the
tolerance check against the fp64 oracle."""
import numpy as np

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
    """|y - yref| <= rel * S elementwise; where S == 0 the result must be 0."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - yref)
    lim = rel * s
    bad = err > lim
    zero = s == 0
    bad |= zero & (y != 0)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside {rel}*S; first {idx.tolist()}: "
            f"y={y[bad][:5]} ref={yref[bad][:5]} S={s[bad][:5]}")
    return float(np.max(err / np.where(s > 0, s, 1)))
