"""GPU: the library's launches captured in a HIP graph (torch.cuda.CUDAGraph)
give the eager results on every replay.

The entry points allocate nothing and record no memory fills, so a captured
launch sequence can be replayed; each test replays several times, with eager
work and synchronisation between the replays, and compares every replay bit
for bit with the eager launch.
"""
import sys

import numpy as np
import pytest

from dequant_quantized_gemv_amd import qk, synth
from tests.gpu_helpers import D_RANGE, FMTS, GEMM_FMTS, torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _replays_match(t, run, outs, replays=4):
    """Eager run, then capture and replay; every replay equals the eager bits."""
    run()
    t.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            run()
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    for r in range(replays):
        for o in outs:
            o.fill_(float("nan"))      # eager work between replays
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, w in zip(outs, want):
            assert t.equal(o.view(t.int32), w.view(t.int32)), f"replay {r} differs"



# (m, k): a 128-multiple k (direct-to-LDS GEMM, whole activation windows), a
# ragged k of 67 blocks (register-staged GEMM, partial window, odd pair
# count), a tall matrix (two rows per wave in the 1-column GEMV), and 20
# blocks (the small-batch GEMM tile on 16, a second launch adding the other 4).
SHAPES = [(300, 2048), (257, 32 * 67), (16403, 1024), (300, 640)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_graph_gemv_batched_expert_x8_gemm_dequant(fmt, m, k):
    t = torch()
    dev = "cuda"
    _say("graph replays", fmt, m, k)
    w = t.from_numpy(synth.quant_matrix(fmt, m, k, seed=3, tensor_id=1, d_range=D_RANGE[fmt])).to(dev)
    x = t.from_numpy(synth.activations(k, 3, seed=3, tensor_id=2)).to(dev)
    x1 = x[:1].contiguous()
    xh = x.half().contiguous()
    y1 = t.empty((3, m), device=dev)
    y1n = t.empty((1, m), device=dev)
    y2 = t.empty((3, m), device=dev)
    y3 = t.empty((3, m), device=dev)
    yd = t.empty((m, k), device=dev)
    ydh = t.empty((m, k), dtype=t.float16, device=dev)
    ne, nu = 6, 2
    me = min(m, 300)
    ws = t.from_numpy(synth.quant_matrix(fmt, ne * me, k, seed=4, tensor_id=1, d_range=D_RANGE[fmt])).to(dev)
    ids = t.tensor([[5, 1], [0, 5]], dtype=t.int32, device=dev)
    ye = t.empty((2, nu, me), device=dev)
    yb = [t.empty((3, m), device=dev), t.empty((3, me), device=dev)]

    def run():
        qk.mul_mat_vec(fmt, w, m, k, x, y=y1)
        qk.mul_mat_vec(fmt, w, m, k, x1, y=y1n)
        qk.mul_mat_vec_x8(fmt, w, m, k, x, y=y2)
        if fmt in GEMM_FMTS:
            qk.mul_mat(fmt, w, m, k, xh, y=y3)
        qk.dequantize(fmt, w, m, k, "f32", out=yd)
        qk.dequantize(fmt, w, m, k, "f16", out=ydh)
        qk.mul_mat_vec_id(fmt, ws, ne, me, k, ids, x[:2], y=ye)
        qk.mul_mat_vec_batched(fmt, [(w, m, k, x), (ws, me, k, x)], ys=yb)

    outs = [y1, y1n, y2, yd, ydh, ye] + yb + ([y3] if fmt in GEMM_FMTS else [])
    _replays_match(t, run, outs)


def test_graph_empty_sum_fill():
    """k == 0 writes the empty sum with a fill kernel, not a memory fill, so a
    captured launch sets the outputs to 0 again on every replay."""
    t = torch()
    _say("graph replays k == 0")
    dummy = t.zeros(64, dtype=t.uint8, device="cuda")
    y = t.empty((2, 5), device="cuda")
    yg = t.empty((40, 7), device="cuda")

    def run():
        s = t.cuda.current_stream().cuda_stream
        assert qk.qk_mul_mat_vec("q4_1", dummy.data_ptr(), 5, 0, dummy.data_ptr(), 2, 0, y.data_ptr(), 5,
                                 s) == qk.QK_OK
        assert qk.qk_mul_mat("q8_0", dummy.data_ptr(), 7, 0, dummy.data_ptr(), 40, 0, yg.data_ptr(), 7,
                             s) == qk.QK_OK

    _replays_match(t, run, [y, yg])
    assert t.count_nonzero(y).item() == 0 and t.count_nonzero(yg).item() == 0
