"""GPU parity of the expert-indexed GEMV (qk_mul_mat_vec_id) and of the
short-row GEMV shapes (several rows per wave) it relies on, called through the
C ABI, against the CPU oracle on the same seeded inputs.

Bar: within 1e-4 * S per element, S = sum_c |W[i,c] x[c]| from the fp64
oracle (S == 0 must give exactly 0); an expert id outside the stack gives NaN
outputs; every output buffer carries guard bands that must come back
untouched, and the gaps between strided outputs stay untouched too.
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import qk, synth
from tests.gpu_helpers import D_RANGE, FMTS, Guarded, assert_within, to_dev_bytes, x_dev, torch

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
TOL = 1e-4
CANARY32 = 0xA5A5A5A5


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _stream():
    return torch().cuda.current_stream().cuda_stream


def _stack(fmt, n_experts, m, k, seed, pad=0):
    """n_experts random m x k matrices, `pad` bytes apart; (bytes, stride)."""
    one = m * (k // 32) * synth.BLOCK_BYTES[fmt]
    w = synth.quant_matrix(fmt, n_experts * m, k, seed=seed, tensor_id=1, d_range=D_RANGE[fmt])
    if pad == 0:
        return w, one
    out = np.zeros(n_experts * (one + pad), dtype=np.uint8)
    for e in range(n_experts):
        out[e * (one + pad):e * (one + pad) + one] = w[e * one:(e + 1) * one]
    return out, one + pad


def _gpu_id(fmt, w, n_experts, stride, m, k, ids, x, layout="token", ld_ids=None, w_off=0,
            x_off=0):
    """Run qk_mul_mat_vec_id.  ids: (n_tokens, n_used) int32.  x: (n_tokens, k)
    (shared by a token's slots) or (n_tokens, n_used, k).  layout: "token"
    (y[t, s] at (t*n_used + s)*m), "slot" (at (s*n_tokens + t)*m) or "gap"
    (padded strides).  Returns y as (n_tokens, n_used, m)."""
    n_tokens, n_used = ids.shape
    ld_ids = n_used if ld_ids is None else ld_ids
    t = torch()
    idf = np.full(max((n_tokens - 1) * ld_ids + n_used, 1), 12345, dtype=np.int32)
    for tt in range(n_tokens):
        idf[tt * ld_ids:tt * ld_ids + n_used] = ids[tt]
    ids_dev = t.from_numpy(idf).to("cuda")
    hw, wp = to_dev_bytes(w, w_off)
    if x.ndim == 2:
        x_slot, x_tok = 0, k
        flat = x.reshape(n_tokens, k)
    else:
        x_slot, x_tok = k, n_used * k
        flat = x.reshape(n_tokens * n_used, k)
    hx, xp = x_dev(flat, k, np.float32, x_off)
    if layout == "token":
        y_slot, y_tok = m, n_used * m
    elif layout == "slot":
        y_slot, y_tok = n_tokens * m, m
    else:
        y_slot, y_tok = m + 3, n_used * (m + 3) + 5
    span = (n_tokens - 1) * y_tok + (n_used - 1) * y_slot + m
    out = Guarded(span * 4)
    st = qk.qk_mul_mat_vec_id(fmt, wp, n_experts, stride, m, k, ids_dev.data_ptr(), ld_ids,
                              n_used, n_tokens, xp, x_slot, x_tok, out.ptr, y_slot, y_tok,
                              _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    flat_y = out.host(np.float32)
    assert out.guards_intact(), "mul_mat_vec_id wrote outside its output"
    y = np.empty((n_tokens, n_used, m), dtype=np.float32)
    touched = np.zeros(span, dtype=bool)
    for tt in range(n_tokens):
        for s in range(n_used):
            p = tt * y_tok + s * y_slot
            y[tt, s] = flat_y[p:p + m]
            touched[p:p + m] = True
    assert np.all(flat_y[~touched].view(np.uint32) == CANARY32), "a gap between outputs was written"
    del hw, hx, ids_dev
    return y


def _oracle_id(fmt, w, n_experts, stride, m, k, ids, x):
    n_tokens, n_used = ids.shape
    if x.ndim == 2:
        return oracle.dot_id(fmt, w, n_experts, stride, m, k, ids, n_used, n_tokens, x, 0, k)
    return oracle.dot_id(fmt, w, n_experts, stride, m, k, ids, n_used, n_tokens, x, k, n_used * k)


# ---------------------------------------------------------------------------
# expert-indexed GEMV
# ---------------------------------------------------------------------------

def test_expert_hand_worked_exact():
    """The hand-derived 3-expert Q4_0 stack: every output exact."""
    with open(GOLDEN) as f:
        case = json.load(f)["expert_dots"][0]
    w = np.concatenate([np.frombuffer(bytes.fromhex(r.replace(" ", "")), dtype=np.uint8)
                        for e in case["experts_hex"] for r in e])
    m, k = case["m"], case["k"]
    ids = np.array(case["ids"], dtype=np.int32)
    n_tokens, n_used = ids.shape
    tau = np.arange(k)
    base = ((tau % 7) - 3).astype(np.float32)
    x = np.stack([np.stack([(2 * t + s + 1) * base for s in range(n_used)])
                  for t in range(n_tokens)]).astype(np.float32)
    _say("expert hand-worked")
    y = _gpu_id("q4_0", w, case["n_experts"], m * (k // 32) * 18, m, k, ids, x)
    want = np.array([[[float(Fraction(v)) for v in r] for r in tt] for tt in case["y"]])
    assert np.array_equal(y.astype(np.float64), want)


# (m, k, n_experts, n_used, n_tokens, shared x)
EXPERT_SHAPES = [
    (768, 2048, 16, 8, 1, True),     # gate / up of the expert workload (half-wave rows)
    (2048, 768, 16, 8, 1, False),    # down (quarter-wave rows, 12 of 16 lanes)
    (61, 544, 5, 3, 4, False),       # ragged rows and an odd pair count
    (33, 32, 4, 2, 3, True),         # one block per row (eighth-wave rows)
    (130, 4096, 3, 2, 2, False),     # full-wave rows
    (9, 11008, 3, 2, 1, True),       # rows of several chunks
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,ne,nu,nt,shared", EXPERT_SHAPES)
def test_expert_within_tolerance(fmt, m, k, ne, nu, nt, shared):
    _say("expert", fmt, m, k, ne, nu, nt, shared)
    w, stride = _stack(fmt, ne, m, k, seed=31 + k)
    ids = synth.expert_ids(nt, nu, ne, seed=31, tensor_id=m)
    x = synth.activations(k, nt * (1 if shared else nu), seed=31, tensor_id=2)
    x = x.reshape(nt, k) if shared else x.reshape(nt, nu, k)
    y = _gpu_id(fmt, w, ne, stride, m, k, ids, x)
    yref, s = _oracle_id(fmt, w, ne, stride, m, k, ids, x)
    assert_within(y, yref, s, TOL, f"expert {fmt} {m}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_expert_layouts_and_generic_path(fmt):
    """Slot-outer and padded outputs, padded expert stride, a row stride in
    ids, repeated experts, and the 2-byte-aligned generic path (stack offset
    by 2 bytes, x offset by one float)."""
    m, k, ne, nu, nt = 45, 1056, 6, 3, 3
    w, stride = _stack(fmt, ne, m, k, seed=41, pad=34)
    ids = np.array([[5, 0, 5], [2, 2, 1], [0, 4, 3]], dtype=np.int32)
    x = synth.activations(k, nt * nu, seed=41, tensor_id=3).reshape(nt, nu, k)
    yref, s = _oracle_id(fmt, w, ne, stride, m, k, ids, x)
    for layout, ld_ids, w_off, x_off in (("slot", 3, 0, 0), ("gap", 5, 0, 0), ("token", 4, 2, 1)):
        _say("expert layout", fmt, layout, ld_ids, w_off, x_off)
        y = _gpu_id(fmt, w, ne, stride, m, k, ids, x, layout=layout, ld_ids=ld_ids,
                    w_off=w_off, x_off=x_off)
        assert_within(y, yref, s, TOL, f"expert layout {fmt} {layout}")


def test_expert_bad_ids_give_nan():
    m, k, ne = 40, 2048, 4
    w, stride = _stack("q4_0", ne, m, k, seed=43)
    ids = np.array([[1, -1, 3], [4, 0, 2 ** 31 - 1]], dtype=np.int32)
    x = synth.activations(k, 2, seed=43, tensor_id=2)
    _say("expert bad ids")
    y = _gpu_id("q4_0", w, ne, stride, m, k, ids, x)
    yref, s = _oracle_id("q4_0", w, ne, stride, m, k, ids, x)
    bad = (ids < 0) | (ids >= ne)
    assert np.isnan(y[bad]).all()
    assert_within(y[~bad], yref[~bad], s[~bad], TOL, "expert valid slots")


@pytest.mark.parametrize("fmt", FMTS)
def test_expert_slots_match_single_gemv_bitwise(fmt):
    """Each (token, slot) is computed exactly as qk_mul_mat_vec computes one
    column of the selected expert."""
    m, k, ne = 96, 2048, 5
    w, stride = _stack(fmt, ne, m, k, seed=47)
    ids = np.array([[4, 1], [0, 4]], dtype=np.int32)
    x = synth.activations(k, 4, seed=47, tensor_id=2).reshape(2, 2, k)
    _say("expert vs single", fmt)
    y = _gpu_id(fmt, w, ne, stride, m, k, ids, x)
    for t in range(2):
        for s in range(2):
            e = ids[t, s]
            hw, wp = to_dev_bytes(w[e * stride:e * stride + m * (k // 32) * synth.BLOCK_BYTES[fmt]])
            hx, xp = x_dev(x[t, s][None, :], k, np.float32)
            out = Guarded(m * 4)
            st = qk.qk_mul_mat_vec(fmt, wp, m, k, xp, 1, k, out.ptr, m, _stream())
            assert st == qk.QK_OK
            assert np.array_equal(out.host(np.float32).view(np.uint32), y[t, s].view(np.uint32))
            del hw, hx


def test_expert_empty_rows():
    """k == 0: every output is the empty sum 0, NaN for an id outside the stack."""
    ids = np.array([[0, 7, 1]], dtype=np.int32)
    x = np.zeros((1, 0), dtype=np.float32)
    _say("expert k=0")
    y = _gpu_id("q8_0", np.zeros(16, np.uint8), 2, 0, 5, 0, ids, x)
    assert np.isnan(y[0, 1]).all()
    assert np.all(y[0, [0, 2]] == 0.0)


def test_expert_full_workload():
    """The expert workload at full size: 128-expert Q4_0 stacks of gate/up
    (768 x 2048, one shared vector) and down (2048 x 768, one vector per
    slot), 8 experts used by one token; every output checked."""
    cfg = synth.WORKLOADS["gemv_q4_0_moe_experts"]
    seed = synth.workload_seed(cfg["id"])
    ne, nu, nt = cfg["n_experts"], cfg["n_used"], cfg["n_tokens"]
    for tid, (name, m, k) in enumerate(cfg["layer"]):
        _say("expert workload", name, m, k)
        w = synth.quant_matrix("q4_0", ne * m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        stride = m * (k // 32) * 18
        ids = synth.expert_ids(nt, nu, ne, seed=seed, tensor_id=50)
        shared = name != "down"
        x = synth.activations(k, nt * (1 if shared else nu), seed=seed, tensor_id=100 + tid)
        x = x.reshape(nt, k) if shared else x.reshape(nt, nu, k)
        y = _gpu_id("q4_0", w, ne, stride, m, k, ids, x)
        yref, s = _oracle_id("q4_0", w, ne, stride, m, k, ids, x)
        assert_within(y, yref, s, TOL, f"expert workload {name}")


# ---------------------------------------------------------------------------
# short rows and empty rows through the plain GEMV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [64, 512, 544, 768, 1024, 1056, 2048, 2080])
@pytest.mark.parametrize("w_off", [0, 2])
def test_gemv_short_rows(fmt, k, w_off):
    """One column, rows of 1 to 33 pairs (8-, 16-, 32- and 64-lane row
    segments), 61 rows (a ragged last group), aligned and generic paths."""
    m = 61
    _say("gemv short rows", fmt, k, w_off)
    w = synth.quant_matrix(fmt, m, k, seed=53, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, 1, seed=53, tensor_id=2)
    hw, wp = to_dev_bytes(w, w_off)
    hx, xp = x_dev(x, k, np.float32)
    out = Guarded(m * 4)
    st = qk.qk_mul_mat_vec(fmt, wp, m, k, xp, 1, k, out.ptr, m, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32)
    assert out.guards_intact()
    yref, s = oracle.dot(fmt, w, m, k, x, 1)
    assert_within(y[None, :], yref, s, TOL, f"short rows {fmt} k={k}")
    del hw, hx


def test_gemv_empty_rows():
    """k == 0: the outputs are the empty sum 0, alone and inside a grouped
    launch next to an ordinary problem."""
    t = torch()
    _say("gemv k=0")
    out = Guarded(3 * 7 * 4)
    dummy = t.zeros(64, dtype=t.uint8, device="cuda")
    st = qk.qk_mul_mat_vec("q4_0", dummy.data_ptr(), 5, 0, dummy.data_ptr(), 3, 0, out.ptr, 7,
                           _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32).reshape(3, 7)
    assert out.guards_intact()
    assert np.all(y[:, :5] == 0.0) and np.all(y[:, 5:].view(np.uint32) == CANARY32)
    m, k = 20, 1024
    w = synth.quant_matrix("q4_0", m, k, seed=57, tensor_id=1, d_range=synth.D_Q4)
    x = synth.activations(k, 1, seed=57, tensor_id=2)
    hw, wp = to_dev_bytes(w)
    hx, xp = x_dev(x, k, np.float32)
    o1, o2 = Guarded(m * 4), Guarded(6 * 4)
    arr = qk.make_items([(wp, m, k, xp, k, o1.ptr, m), (dummy.data_ptr(), 6, 0, xp, 0, o2.ptr, 6)])
    st = qk.qk_mul_mat_vec_batched("q4_0", arr, 2, 1, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    yref, s = oracle.dot("q4_0", w, m, k, x, 1)
    assert_within(o1.host(np.float32)[None, :], yref, s, TOL, "batched next to k=0")
    assert np.all(o2.host(np.float32) == 0.0)
    assert o1.guards_intact() and o2.guards_intact()
    del hw, hx, dummy
