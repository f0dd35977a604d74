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
from tests.gpu_helpers import torch

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


def test_graph_gemv_batched_expert_x8_gemm_dequant():
    t = torch()
    dev = "cuda"
    _say("graph replays")
    m, k = 300, 2048
    w = t.from_numpy(synth.quant_matrix("q4_0", m, k, seed=3, tensor_id=1, d_range=synth.D_Q4)).to(dev)
    x = t.from_numpy(synth.activations(k, 3, seed=3, tensor_id=2)).to(dev)
    xh = x.half().contiguous()
    y1 = t.empty((3, m), device=dev)
    y2 = t.empty((3, m), device=dev)
    y3 = t.empty((3, m), device=dev)
    yd = t.empty((m, k), device=dev)
    ne, nu = 6, 2
    ws = t.from_numpy(synth.quant_matrix("q4_0", ne * m, k, seed=4, tensor_id=1, d_range=synth.D_Q4)).to(dev)
    ids = t.tensor([[5, 1], [0, 5]], dtype=t.int32, device=dev)
    ye = t.empty((2, nu, m), device=dev)
    yb = [t.empty((3, m), device=dev) for _ in range(2)]

    def run():
        qk.mul_mat_vec("q4_0", w, m, k, x, y=y1)
        qk.mul_mat_vec_x8("q4_0", w, m, k, x, y=y2)
        qk.mul_mat("q4_0", w, m, k, xh, y=y3)
        qk.dequantize("q4_0", w, m, k, "f32", out=yd)
        qk.mul_mat_vec_id("q4_0", ws, ne, m, k, ids, x[:2], y=ye)
        qk.mul_mat_vec_batched("q4_0", [(w, m, k, x), (ws, m, k, x)], ys=yb)

    _replays_match(t, run, [y1, y2, y3, yd, ye] + yb)
