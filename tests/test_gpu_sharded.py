"""GPU parity of the GEMV at one GPU's share of a tensor-parallel layer, called
through the C ABI, against the CPU oracle.

Row shards (q, k, v, gate, up) are whole rows of the full matrix; K shards (o,
down) give partial sums that the GPUs would add with one all-reduce.  On one GPU
the test computes every shard in turn and checks that row shards reproduce the
full GEMV bit for bit and that the K-shard partial sums add up to the full
product within the GEMV bound (|sum - exact| <= 1e-4 * S, S of the full row).
"""
import sys

import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import qk, synth
from tests.gpu_helpers import D_RANGE, FMTS, Guarded, assert_within, to_dev_bytes, x_dev, torch

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _stream():
    return torch().cuda.current_stream().cuda_stream


def _gemv(fmt, w, m, k, x2d):
    n = x2d.shape[0]
    hw, wp = to_dev_bytes(w)
    hx, xp = x_dev(x2d, k, np.float32)
    out = Guarded(n * m * 4)
    st = qk.qk_mul_mat_vec(fmt, wp, m, k, xp, n, k, out.ptr, m, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32).reshape(n, m)
    assert out.guards_intact()
    del hw, hx
    return y


def _k_shard(fmt, w, m, k, parts, i):
    """Columns [i*k/parts, (i+1)*k/parts) of every row, as a contiguous matrix."""
    bs = synth.BLOCK_BYTES[fmt]
    nb = k // 32
    per = nb // parts
    blocks = w.reshape(m, nb, bs)
    return np.ascontiguousarray(blocks[:, i * per:(i + 1) * per, :]).ravel()


@pytest.mark.parametrize("fmt", FMTS)
def test_k_shard_partial_sums_add_up(fmt):
    """down 4096 x 11008 split 8 ways along K (43 blocks a shard, rows not
    4-byte aligned for Q4_0 / Q8_0): the partial sums add up to the full
    product."""
    m, k, parts = 4096, 11008, synth.TP
    _say("k shards", fmt)
    w = synth.quant_matrix(fmt, m, k, seed=71, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, 2, seed=71, tensor_id=2)
    ks = k // parts
    total = np.zeros((2, m), dtype=np.float64)
    for i in range(parts):
        y = _gemv(fmt, _k_shard(fmt, w, m, k, parts, i), m, ks,
                  np.ascontiguousarray(x[:, i * ks:(i + 1) * ks]))
        total += y.astype(np.float64)
    yref, s = oracle.dot(fmt, w, m, k, x, 2)
    assert_within(total, yref, s, TOL, f"k shards {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_row_shards_match_full_gemv_bitwise(fmt):
    """gate 11008 x 4096 split 8 ways by rows: every shard's outputs are the
    full GEMV's rows, bit for bit."""
    m, k, parts = 11008, 4096, synth.TP
    _say("row shards", fmt)
    w = synth.quant_matrix(fmt, m, k, seed=73, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, 1, seed=73, tensor_id=2)
    full = _gemv(fmt, w, m, k, x)
    rows = m // parts
    rb = (k // 32) * synth.BLOCK_BYTES[fmt]
    for i in range(parts):
        y = _gemv(fmt, w[i * rows * rb:(i + 1) * rows * rb], rows, k, x)
        assert np.array_equal(y.view(np.uint32), full[:, i * rows:(i + 1) * rows].view(np.uint32))


def test_share_layer_grouped_full():
    """The 7B-shaped layer's one-GPU share (q, k, v 512 x 4096; o 4096 x 512;
    gate, up 1376 x 4096; down 4096 x 1376) in one grouped launch, every
    output checked, and bitwise equal to separate launches."""
    cfg = synth.WORKLOADS["gemv_q4_0_decode_layer_tp8_share"]
    seed = synth.workload_seed(cfg["id"])
    _say("share layer grouped")
    holds, tups, outs, probs = [], [], [], []
    for tid, (name, m, k) in enumerate(cfg["layer"]):
        w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        x = synth.activations(k, 1, seed=seed, tensor_id=100 + tid)
        hw, wp = to_dev_bytes(w)
        hx, xp = x_dev(x, k, np.float32)
        out = Guarded(m * 4)
        holds += [hw, hx]
        outs.append(out)
        probs.append((w, m, k, x))
        tups.append((wp, m, k, xp, k, out.ptr, m))
    st = qk.qk_mul_mat_vec_batched("q4_0", qk.make_items(tups), len(tups), 1, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    for (w, m, k, x), out in zip(probs, outs):
        y = out.host(np.float32)
        assert out.guards_intact()
        yref, s = oracle.dot("q4_0", w, m, k, x, 1)
        assert_within(y[None, :], yref, s, TOL, f"share {m}x{k}")
        assert np.array_equal(y.view(np.uint32), _gemv("q4_0", w, m, k, x)[0].view(np.uint32))
    del holds
