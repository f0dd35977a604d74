"""Seeded random-shape sweep of every compute entry point against the oracle.

The hand-picked cases in the other GPU test files pin the named workloads,
the edge values and each code path on purpose; this sweep draws shapes,
column counts, leading dimensions and pointer offsets at random (one fixed
seed per entry point, so the cases are the same on every run) to cover the
combinations between them: ragged row groups with the generic load path,
launch shapes that switch at row-count thresholds, short rows sharing a wave,
leading dimensions that break 16-byte alignment, and so on.  Bars as in the
parity tests: dequantize bit-exact, products within 1e-4 * S (GEMV, expert
GEMV, 8-bit-activation GEMV against its own quantization) or 1e-2 * S (GEMM).
"""
import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import synth
from tests.gpu_helpers import assert_within
from tests.test_gpu_experts import _gpu_id, _oracle_id, _stack
from tests.test_gpu_parity import (GEMM_TOL, GEMV_TOL, _gpu_dequant, _gpu_gemm, _gpu_gemv,
                                   _gpu_gemv_batched, _oracle_bits, _say, _weights)
from tests.test_gpu_x8 import _gemv_x8

pytestmark = pytest.mark.gpu


def _cases(seed, count, draw):
    rng = np.random.default_rng(seed)
    return [draw(rng) for _ in range(count)]


def _fmt(rng):
    return ("q4_0", "q4_1", "q8_0")[int(rng.integers(0, 3))]


def _as_q5(cases, seed):
    """The same draws with the format replaced by Q5_0 or Q5_1 (own stream)."""
    rng = np.random.default_rng(seed)
    return [dict(c, fmt=("q5_0", "q5_1")[int(rng.integers(0, 2))]) for c in cases]


def _draw_dequant(rng):
    dtype = ["f32", "f16"][int(rng.integers(0, 2))]
    es = 4 if dtype == "f32" else 2
    return dict(fmt=_fmt(rng), rows=int(rng.integers(1, 301)), nb=int(rng.integers(1, 201)),
                dtype=dtype, w_off=int(rng.choice([0, 0, 2, 6, 16])),
                out_off=int(rng.choice([0, 0, 1, 3])) * es)


def _draw_gemv(rng):
    m, nb, n = int(rng.integers(1, 601)), int(rng.integers(1, 401)), int(rng.integers(1, 9))
    k = 32 * nb
    return dict(fmt=_fmt(rng), m=m, k=k, n=n, ldx=k + int(rng.choice([0, 0, 1, 4, 37])),
                ldy=m + int(rng.choice([0, 0, 1, 3])), w_off=int(rng.choice([0, 0, 2, 4])),
                x_off=int(rng.choice([0, 0, 1, 3])))


def _draw_batched(rng):
    count, n = int(rng.integers(2, 17)), int(rng.integers(1, 9))
    items = [(int(rng.integers(1, 400)), 32 * int(rng.integers(1, 300)), int(rng.choice([0, 0, 2])),
              int(rng.choice([0, 0, 1])))
             for _ in range(count)]
    return dict(fmt=_fmt(rng), n=n, items=items)


def _draw_expert(rng):
    ne = int(rng.integers(1, 13))
    return dict(fmt=_fmt(rng), ne=ne, m=int(rng.integers(1, 300)), k=32 * int(rng.integers(1, 100)),
                nu=int(rng.integers(1, ne + 1)), nt=int(rng.integers(1, 5)),
                shared=bool(rng.integers(0, 2)), layout=["token", "slot", "gap"][int(rng.integers(0, 3))],
                pad=int(rng.choice([0, 0, 2, 64])), w_off=int(rng.choice([0, 0, 2])))


def _draw_gemm(rng):
    m, nb, n = int(rng.integers(1, 401)), int(rng.integers(1, 101)), int(rng.integers(1, 201))
    k = 32 * nb
    return dict(fmt=_fmt(rng), m=m, k=k, n=n, ldx=k + int(rng.choice([0, 0, 0, 3, 8])),
                ldy=m + int(rng.choice([0, 0, 1, 4])), w_off=int(rng.choice([0, 0, 2])),
                x_off=int(rng.choice([0, 0, 1, 8])))


def _draw_gemm_small(rng):
    # k a multiple of 128 and at most 128 columns: the 64 x 32 small-batch tile
    # (with aligned, 8-element-multiple strides; other strides take the
    # register-staged path)
    m, n = int(rng.integers(1, 701)), int(rng.integers(1, 129))
    nb = 16 * int(rng.integers(1, 5)) + 4 * int(rng.integers(0, 4))  # leftover blocks: second launch
    k = 32 * nb
    return dict(fmt=_fmt(rng), m=m, k=k, n=n, ldx=k + int(rng.choice([0, 0, 8, 3])),
                ldy=m + int(rng.choice([0, 0, 4, 1])), w_off=0, x_off=int(rng.choice([0, 0, 0, 8])))


DEQUANT = _cases(0xD0, 24, _draw_dequant)
GEMV = _cases(0xD1, 40, _draw_gemv)
GEMV_X8 = _cases(0xD2, 20, _draw_gemv)
BATCHED = _cases(0xD3, 12, _draw_batched)
EXPERT = _cases(0xD4, 12, _draw_expert)
DEQUANT += _as_q5(_cases(0xE0, 10, _draw_dequant), 0xE0)
GEMV += _as_q5(_cases(0xE1, 20, _draw_gemv), 0xE1)
GEMV_X8 += _as_q5(_cases(0xE2, 10, _draw_gemv), 0xE2)
BATCHED += _as_q5(_cases(0xE3, 6, _draw_batched), 0xE3)
EXPERT += _as_q5(_cases(0xE4, 6, _draw_expert), 0xE4)
GEMM = _cases(0xD5, 16, _draw_gemm) + _as_q5(_cases(0xE5, 8, _draw_gemm), 0xE5)
GEMM_SMALL = _cases(0xD6, 12, _draw_gemm_small) + _as_q5(_cases(0xE6, 4, _draw_gemm_small), 0xE6)


@pytest.mark.parametrize("c", DEQUANT, ids=[f"dq{i}" for i in range(len(DEQUANT))])
def test_sweep_dequantize(c):
    _say("sweep dequant", c)
    k = 32 * c["nb"]
    w = _weights(c["fmt"], c["rows"], k, seed=60)
    got = _gpu_dequant(c["fmt"], w, c["rows"], k, c["dtype"], w_off=c["w_off"], out_off=c["out_off"])
    assert np.array_equal(got, _oracle_bits(c["fmt"], w, c["rows"], k, c["dtype"]))


@pytest.mark.parametrize("c", GEMV, ids=[f"gemv{i}" for i in range(len(GEMV))])
def test_sweep_gemv(c):
    _say("sweep gemv", c)
    w = _weights(c["fmt"], c["m"], c["k"], seed=61)
    x = synth.activations(c["k"], c["n"], seed=61, tensor_id=2)
    y = _gpu_gemv(c["fmt"], w, c["m"], c["k"], x, ldx=c["ldx"], ldy=c["ldy"], w_off=c["w_off"],
                  x_off=c["x_off"])
    yref, s = oracle.dot(c["fmt"], w, c["m"], c["k"], x, c["n"])
    assert_within(y, yref, s, GEMV_TOL, f"sweep gemv {c}")


@pytest.mark.parametrize("c", GEMV_X8, ids=[f"x8_{i}" for i in range(len(GEMV_X8))])
def test_sweep_gemv_x8(c):
    _say("sweep gemv x8", c)
    w = _weights(c["fmt"], c["m"], c["k"], seed=62)
    x = synth.activations(c["k"], c["n"], seed=62, tensor_id=2)
    y = _gemv_x8(c["fmt"], w, c["m"], c["k"], x, ldx=c["ldx"], ldy=c["ldy"], w_off=c["w_off"],
                 x_off=c["x_off"])
    yref, s = oracle.dot_x8(c["fmt"], w, c["m"], c["k"], x, c["n"])
    assert_within(y, yref, s, GEMV_TOL, f"sweep gemv x8 {c}")


@pytest.mark.parametrize("c", BATCHED, ids=[f"grp{i}" for i in range(len(BATCHED))])
def test_sweep_gemv_batched(c):
    _say("sweep batched", c["fmt"], c["n"], c["items"])
    probs = []
    for i, (m, k, _, _) in enumerate(c["items"]):
        probs.append((_weights(c["fmt"], m, k, seed=63, tid=i), m, k,
                      synth.activations(k, c["n"], seed=63, tensor_id=20 + i)))
    ys = _gpu_gemv_batched(c["fmt"], probs, c["n"], w_offs=[it[2] for it in c["items"]],
                           x_offs=[it[3] for it in c["items"]])
    for (w, m, k, x), y in zip(probs, ys):
        yref, s = oracle.dot(c["fmt"], w, m, k, x, c["n"])
        assert_within(y, yref, s, GEMV_TOL, f"sweep batched {c['fmt']} {m}x{k} n={c['n']}")


@pytest.mark.parametrize("c", EXPERT, ids=[f"moe{i}" for i in range(len(EXPERT))])
def test_sweep_expert(c):
    _say("sweep expert", c)
    w, stride = _stack(c["fmt"], c["ne"], c["m"], c["k"], seed=64, pad=c["pad"])
    rng = np.random.default_rng(64)
    ids = np.stack([rng.choice(c["ne"], c["nu"], replace=False) for _ in range(c["nt"])]).astype(np.int32)
    if c["shared"]:
        x = synth.activations(c["k"], c["nt"], seed=64, tensor_id=2)
    else:
        x = synth.activations(c["k"], c["nt"] * c["nu"], seed=64, tensor_id=2).reshape(c["nt"], c["nu"], c["k"])
    y = _gpu_id(c["fmt"], w, c["ne"], stride, c["m"], c["k"], ids, x, layout=c["layout"], w_off=c["w_off"])
    yref, s = _oracle_id(c["fmt"], w, c["ne"], stride, c["m"], c["k"], ids, x)
    assert_within(y, yref.reshape(y.shape), s.reshape(y.shape), GEMV_TOL, f"sweep expert {c}")


@pytest.mark.parametrize("c", GEMM, ids=[f"gemm{i}" for i in range(len(GEMM))])
def test_sweep_gemm(c):
    _say("sweep gemm", c)
    w = _weights(c["fmt"], c["m"], c["k"], seed=65)
    xh = synth.activations(c["k"], c["n"], seed=65, tensor_id=2, dtype=np.float16)
    y = _gpu_gemm(c["fmt"], w, c["m"], c["k"], xh, ldx=c["ldx"], ldy=c["ldy"], x_off=c["x_off"],
                  w_off=c["w_off"])
    yref, s = oracle.dot(c["fmt"], w, c["m"], c["k"], xh.view(np.uint16), c["n"], x_is_f16=True)
    assert_within(y, yref, s, GEMM_TOL, f"sweep gemm {c}")


@pytest.mark.parametrize("c", GEMM_SMALL, ids=[f"gemm_small{i}" for i in range(len(GEMM_SMALL))])
def test_sweep_gemm_small_batch(c):
    _say("sweep gemm small batch", c)
    w = _weights(c["fmt"], c["m"], c["k"], seed=66)
    xh = synth.activations(c["k"], c["n"], seed=66, tensor_id=2, dtype=np.float16)
    y = _gpu_gemm(c["fmt"], w, c["m"], c["k"], xh, ldx=c["ldx"], ldy=c["ldy"], x_off=c["x_off"],
                  w_off=c["w_off"])
    yref, s = oracle.dot(c["fmt"], w, c["m"], c["k"], xh.view(np.uint16), c["n"], x_is_f16=True)
    assert_within(y, yref, s, GEMM_TOL, f"sweep gemm small batch {c}")
