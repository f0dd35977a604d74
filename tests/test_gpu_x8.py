"""GPU parity of the GEMV with 8-bit activations (qk_mul_mat_vec_x8), called
through the C ABI, against the CPU oracle's product with the same quantized
activations (oracle.dot_x8: every code decision is exact, so both sides take
the same ones).

Bar: |y - y_ref| <= 1e-4 * S per element, S the sum of the magnitudes of the
per-block terms (oracle.dot_x8); S == 0 must give exactly 0.  Guard bands
around every output must come back untouched.
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import qk, synth
from tests.gpu_helpers import D_RANGE, FMTS, Guarded, assert_within, oracle_rows, to_dev_bytes, x_dev, torch

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
TOL = 1e-4


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _gemv_x8(fmt, w, m, k, x2d, ldx=None, ldy=None, w_off=0, x_off=0):
    n = x2d.shape[0]
    ldx = k if ldx is None else ldx
    ldy = m if ldy is None else ldy
    hw, wp = to_dev_bytes(w, w_off)
    hx, xp = x_dev(x2d, ldx, np.float32, x_off)
    out = Guarded(((n - 1) * ldy + m) * 4)
    st = qk.qk_mul_mat_vec_x8(fmt, wp, m, k, xp, n, ldx, out.ptr, ldy,
                              torch().cuda.current_stream().cuda_stream)
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32)
    assert out.guards_intact(), "mul_mat_vec_x8 wrote outside its output"
    del hw, hx
    return np.stack([y[j * ldy: j * ldy + m] for j in range(n)])


def test_x8_hand_worked_exact():
    """The golden dots whose activations quantize without loss: exact."""
    with open(GOLDEN) as f:
        g = json.load(f)
    dots = {c["name"]: c for c in g["dots"]}
    byname = {b["name"]: b for b in g["blocks"]}
    for case in g["x8_dots"]:
        base = dots[case["dot"]]
        fmt, m, k = base["fmt"], base["m"], base["k"]
        hexs = base["rows_hex"] if "rows_hex" in base else [byname[b]["bytes_hex"] for b in base["blocks"]]
        w = np.concatenate([np.frombuffer(bytes.fromhex(h.replace(" ", "")), dtype=np.uint8) for h in hexs])
        t = np.arange(k)
        x = {"t+1": t + 1.0, "(t mod 7) - 3": (t % 7) - 3.0}[base["x_rule"]].astype(np.float32)
        _say("x8 hand-worked", case["name"])
        y = _gemv_x8(fmt, w, m, k, x[None, :])
        assert list(y[0].astype(np.float64)) == [float(Fraction(v)) for v in case["y"]]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (3, 96, 2), (61, 544, 1), (100, 4096, 8),
                                   (259, 11008, 3), (33, 1376, 4), (17, 2048, 5), (8, 256, 7)])
def test_x8_within_tolerance(fmt, m, k, n):
    _say("x8", fmt, m, k, n)
    w = synth.quant_matrix(fmt, m, k, seed=91, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, n, seed=91, tensor_id=2)
    y = _gemv_x8(fmt, w, m, k, x)
    yref, s = oracle.dot_x8(fmt, w, m, k, x, n)
    assert_within(y, yref, s, TOL, f"x8 {fmt} {m}x{k} n={n}")


@pytest.mark.parametrize("fmt", FMTS)
def test_x8_strides_and_unaligned(fmt):
    """2-byte aligned weights (generic path), activations only 4-byte aligned
    with a padded stride, padded output stride."""
    m, k, n = 45, 1056, 3
    w = synth.quant_matrix(fmt, m, k, seed=93, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, n, seed=93, tensor_id=2)
    yref, s = oracle.dot_x8(fmt, w, m, k, x, n)
    for w_off, x_off, ldx, ldy in ((2, 0, None, None), (0, 1, 1061, 50), (2, 3, 1057, 47)):
        _say("x8 strides", fmt, w_off, x_off, ldx, ldy)
        y = _gemv_x8(fmt, w, m, k, x, ldx=ldx, ldy=ldy, w_off=w_off, x_off=x_off)
        assert_within(y, yref, s, TOL, f"x8 strides {fmt} {w_off} {x_off}")


@pytest.mark.parametrize("fmt", FMTS)
def test_x8_adversarial_activations(fmt):
    """Zero blocks, fp32-subnormal blocks, exact ties (codes of the form
    k + 1/2), and block magnitudes from 1e-20 to 1e20 in one column."""
    m, k = 40, 32 * 12
    w = synth.quant_matrix(fmt, m, k, seed=95, tensor_id=1, d_range=D_RANGE[fmt])
    rng = np.random.default_rng(95)
    x = rng.standard_normal((2, k))
    x[0, 0:32] = 0.0
    x[0, 32:64] = np.float32(3e-40) * np.sign(x[0, 32:64])
    x[0, 64:96] = (np.arange(32) - 16) + 0.5                      # d = 1/8, q = 8x exactly
    x[0, 96:128] = np.concatenate([[127.0], (np.arange(31) - 15) + 0.5])  # d = 1: ties
    x[1] *= 10.0 ** rng.integers(-20, 21, 12).repeat(32)
    x = x.astype(np.float32)
    _say("x8 adversarial", fmt)
    y = _gemv_x8(fmt, w, m, k, x)
    yref, s = oracle.dot_x8(fmt, w, m, k, x, 2)
    assert_within(y, yref, s, TOL, f"x8 adversarial {fmt}")


def test_x8_empty_rows():
    """k == 0: the empty sum 0."""
    t = torch()
    out = Guarded(2 * 5 * 4)
    dummy = t.zeros(64, dtype=t.uint8, device="cuda")
    st = qk.qk_mul_mat_vec_x8("q4_1", dummy.data_ptr(), 5, 0, dummy.data_ptr(), 2, 0, out.ptr, 5,
                              t.cuda.current_stream().cuda_stream)
    assert st == qk.QK_OK
    assert np.all(out.host(np.float32) == 0.0) and out.guards_intact()


@pytest.mark.parametrize("fmt", FMTS)
def test_x8_nonfinite_activations_give_nan(fmt):
    """A block holding an infinity or a NaN has a NaN scale: every output of
    its column is NaN; the other columns stay within tolerance."""
    m, k = 70, 32 * 6
    w = synth.quant_matrix(fmt, m, k, seed=97, tensor_id=1, d_range=D_RANGE[fmt])
    x = synth.activations(k, 4, seed=97, tensor_id=2)
    x[0, 70] = np.inf
    x[1, 5] = -np.inf
    x[2, 190] = np.nan
    _say("x8 non-finite", fmt)
    y = _gemv_x8(fmt, w, m, k, x)
    yref, s = oracle.dot_x8(fmt, w, m, k, x, 4)
    assert np.isnan(yref[:3]).all() and np.isnan(y[:3]).all()
    assert_within(y[3:], yref[3:], s[3:], TOL, f"x8 finite column {fmt}")


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_x8_full_q4_1_11008x4096(n):
    """The Q4_1 11008 x 4096 workload with 8-bit activations: every output
    against the oracle."""
    cfg = synth.WORKLOADS["gemv_q4_1_11008x4096"]
    seed = synth.workload_seed(cfg["id"])
    m, k = cfg["m"], cfg["k"]
    w = synth.quant_matrix("q4_1", m, k, seed=seed, tensor_id=0, d_range=cfg["d"], m_range=cfg["mr"])
    x = np.ascontiguousarray(synth.activations(k, 8, seed=seed, tensor_id=100)[:n])
    _say("x8 full q4_1", n)
    y = _gemv_x8("q4_1", w, m, k, x)
    yref, s = oracle_rows(oracle.dot_x8, "q4_1", w, m, k, x, n)
    assert_within(y, yref, s, TOL, f"x8 full q4_1 n={n}")
