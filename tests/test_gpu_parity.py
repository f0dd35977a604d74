"""GPU parity: libqk's gfx950 kernels, called through the C ABI, against the
CPU oracle on the same seeded inputs.

Bars: dequantize is bit-exact (fp32 and fp16); GEMV within 1e-4 * S and GEMM
within 1e-2 * S per element, S = sum_c |W[i,c] x[c,j]| from the fp64 oracle
(an element with S == 0 must be exactly 0).  Every output buffer carries guard
bands that must come back untouched.
"""
import json
from fractions import Fraction
import os
import sys

import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import qk, synth
from tests.gpu_helpers import (D_RANGE, FMTS, GEMM_FMTS, Guarded, assert_within, gemm_reference,
                               oracle_rows, to_dev_bytes, x_dev, torch)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
GEMV_TOL = 1e-4
GEMM_TOL = 1e-2


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _stream():
    return torch().cuda.current_stream().cuda_stream


def _weights(fmt, m, k, seed=11, tid=1):
    return synth.quant_matrix(fmt, m, k, seed=seed, tensor_id=tid, d_range=D_RANGE[fmt])


# ---------------------------------------------------------------------------
# dequantize
# ---------------------------------------------------------------------------

def _gpu_dequant(fmt, w, rows, k, dtype, w_off=0, out_off=0):
    hold, wp = to_dev_bytes(w, w_off)
    es = 4 if dtype == "f32" else 2
    out = Guarded(rows * k * es, offset=out_off)
    st = qk.qk_dequantize(fmt, wp, rows, k, qk.QK_F32 if dtype == "f32" else qk.QK_F16,
                          out.ptr, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    res = out.host(np.uint32 if dtype == "f32" else np.uint16).reshape(rows, k)
    assert out.guards_intact(), "dequantize wrote outside its output"
    del hold
    return res


def _oracle_bits(fmt, w, rows, k, dtype):
    if dtype == "f32":
        return oracle.dequantize_f32(fmt, w, rows, k).view(np.uint32)
    return oracle.dequantize_f16(fmt, w, rows, k)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,k", [(1, 32), (3, 64), (7, 96), (3, 2080), (33, 4096), (5, 11008)])
def test_dequantize_bit_exact(fmt, dtype, rows, k):
    _say("dequant", fmt, dtype, rows, k)
    w = _weights(fmt, rows, k)
    got = _gpu_dequant(fmt, w, rows, k, dtype)
    assert np.array_equal(got, _oracle_bits(fmt, w, rows, k, dtype))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("w_off,out_off", [(2, 0), (0, 4), (6, 12)])
def test_dequantize_unaligned_paths(fmt, dtype, w_off, out_off):
    rows, k = 9, 2080  # 585 blocks: several workgroups and a ragged tail
    _say("dequant unaligned", fmt, dtype, w_off, out_off)
    w = _weights(fmt, rows, k, seed=12)
    got = _gpu_dequant(fmt, w, rows, k, dtype, w_off=w_off, out_off=out_off)
    assert np.array_equal(got, _oracle_bits(fmt, w, rows, k, dtype))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out_off", [0, 4])
def test_dequantize_chunk_loop(fmt, dtype, out_off):
    """More chunks of 128 blocks than the aligned-input kernel launches
    workgroups (8 per CU): workgroups take further chunks while the previous
    one's outputs are written, and the last chunk is ragged (67 blocks,
    whose Q4_0 / Q4_1 bytes end 6 / 12 bytes past a 16-byte boundary)."""
    rows, k = 8195, 2080  # 532 675 blocks = 4161 full chunks + 67 blocks
    _say("dequant chunk loop", fmt, dtype, out_off)
    w = _weights(fmt, rows, k, seed=13)
    got = _gpu_dequant(fmt, w, rows, k, dtype, out_off=out_off)
    assert np.array_equal(got, _oracle_bits(fmt, w, rows, k, dtype))


def _edge_blocks(fmt):
    """Subnormal and negative d, q = 8 (Q4_0) / 16 (Q5_0) with d < 0 (sign
    of zero), Q8 -128/127, Q5 codes 0 and 31, fp16 overflow to +-inf, +-0 d."""
    dbits = np.array([0x0001, 0x03FF, 0x8001, 0xB800, 0x7BFF, 0xFBFF, 0x0000, 0x8000,
                      0x3C00, 0x2E66], dtype=np.uint16)
    nb = dbits.size
    if fmt == "q8_0":
        codes = np.tile(np.array([-128, 127, 0, -1, 1, 64, -64, 100] * 4), (nb, 1))
    elif fmt in ("q5_0", "q5_1"):
        codes = np.tile(np.array([16, 0, 31, 15, 17, 1, 30, 16] * 4), (nb, 1))
    else:
        codes = np.tile(np.array([8, 0, 15, 7, 9, 1, 14, 8] * 4), (nb, 1))
    mbits = np.array([0x8001, 0x0001, 0xB800, 0x3800, 0x7BFF, 0x0000, 0x8000, 0xBC00,
                      0x2E66, 0xAE66], dtype=np.uint16)
    return synth.pack_blocks(fmt, dbits, codes, m_bits=mbits), nb


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_edge_values(fmt, dtype):
    _say("dequant edge", fmt, dtype)
    w, nb = _edge_blocks(fmt)
    got = _gpu_dequant(fmt, w, nb, 32, dtype)
    want = _oracle_bits(fmt, w, nb, 32, dtype)
    assert np.array_equal(got, want)
    if dtype == "f16":
        assert np.isinf(want.view(np.float16)).any()   # the overflow case is exercised


def test_dequantize_hand_worked_blocks():
    with open(GOLDEN) as f:
        g = json.load(f)
    for blk in g["blocks"]:
        _say("dequant golden", blk["name"])
        raw = np.frombuffer(bytes.fromhex(blk["bytes_hex"].replace(" ", "")), dtype=np.uint8)
        got = _gpu_dequant(blk["fmt"], raw, 1, 32, "f32").view(np.float32).ravel()
        want = np.array([float(v) for v in blk["values"]], dtype=np.float32)
        assert np.array_equal(got, want)
        for t in blk["positive_zero_at"]:
            assert got[t].view(np.uint32) == 0
        for t in blk.get("negative_zero_at", []):
            assert got[t].view(np.uint32) == 0x80000000


def test_dequantize_full_config0():
    """4096 x 4096 Q4_0 -> fp32, every element bit-exact."""
    cfg = synth.WORKLOADS["dequant_q4_0_4096x4096_f32"]
    seed = synth.workload_seed(cfg["id"])
    _say("dequant full", cfg)
    w = synth.quant_matrix("q4_0", cfg["m"], cfg["k"], seed=seed, tensor_id=0, d_range=cfg["d"])
    got = _gpu_dequant("q4_0", w, cfg["m"], cfg["k"], "f32")
    assert np.array_equal(got, oracle.dequantize_f32("q4_0", w, cfg["m"], cfg["k"]).view(np.uint32))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def _gpu_gemv(fmt, w, m, k, x2d, ldx=None, ldy=None, w_off=0, x_off=0, stream=None):
    n = x2d.shape[0]
    ldx = k if ldx is None else ldx
    ldy = m if ldy is None else ldy
    hw, wp = to_dev_bytes(w, w_off)
    hx, xp = x_dev(x2d, ldx, np.float32, x_off)
    out = Guarded(((n - 1) * ldy + m) * 4)
    st = qk.qk_mul_mat_vec(fmt, wp, m, k, xp, n, ldx, out.ptr, ldy,
                           _stream() if stream is None else stream)
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32)
    assert out.guards_intact(), "mul_mat_vec wrote outside its output"
    cols = np.stack([y[j * ldy: j * ldy + m] for j in range(n)])
    if ldy > m:   # the gaps between columns are untouched
        gaps = np.concatenate([y[j * ldy + m:(j + 1) * ldy] for j in range(n - 1)] or [y[:0]])
        assert np.all(gaps.view(np.uint32) == 0xA5A5A5A5)
    del hw, hx
    return cols


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_unit_vectors_edge_blocks(fmt):
    """The dequantize edge blocks (all ten: subnormal, negative, zero, largest
    and smallest scales, Q8_0 -128 / 127, Q4_1 offsets of every sign) times
    unit vectors e_c, eight columns per call: every output is exactly the fp32
    weight W[i, c] (one nonzero term, the rest exact zeros)."""
    w, nb = _edge_blocks(fmt)
    k = 32
    W = oracle.dequantize_f32(fmt, w, nb, k)
    assert np.isfinite(W).all()
    _say("gemv unit vectors edge", fmt)
    for c0 in range(0, k, 8):
        x = np.zeros((8, k), np.float32)
        for j in range(8):
            x[j, c0 + j] = 1.0
        y = _gpu_gemv(fmt, w, nb, k, x)
        assert np.array_equal(y, W[:, c0:c0 + 8].T), f"columns {c0}..{c0 + 7}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_subnormal_activations(fmt):
    """Activations in the fp32 subnormal range (N(0,1) scaled by 2^-130) and
    products below the normal range: nothing may be flushed to zero, so the
    outputs stay within 1e-4 * S of the oracle (a flush would give 0 against
    a nonzero reference)."""
    m, k, n = 130, 2080, 3
    _say("gemv subnormal activations", fmt)
    w = _weights(fmt, m, k, seed=48)
    x = (synth.activations(k, n, seed=48, tensor_id=2).astype(np.float64) * 2.0 ** -130).astype(np.float32)
    assert np.all(np.abs(x[x != 0]) < np.finfo(np.float32).tiny)
    y = _gpu_gemv(fmt, w, m, k, x)
    yref, s = oracle.dot(fmt, w, m, k, x, n)
    assert np.all(s > 0)
    assert_within(y, yref, s, GEMV_TOL, f"gemv subnormal {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("m,k,w_off", [(16403, 4096, 0), (16400, 2048, 2), (16403, 1376, 0)])
def test_gemv_two_rows_per_wave(fmt, n, m, k, w_off):
    """Launches past the two-rows-per-wave thresholds (more than 64 rows per
    CU at one column, 32 at two or three: 16 403 rows is past both on 256
    CUs): every output against the oracle on the aligned path (ragged last
    row group), a 2-byte aligned matrix and an odd block count (43 blocks per
    row), both on the generic path (which keeps one row per wave for Q4_1
    above one column and for Q8_0)."""
    _say("gemv two rows per wave", fmt, n, m, k, w_off)
    w = _weights(fmt, m, k, seed=46)
    x = synth.activations(k, n, seed=46, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x, w_off=w_off)
    yref, s = oracle.dot(fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv two rows {fmt} {m}x{k} n={n} w_off={w_off}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (2, 64, 2), (3, 96, 1), (13, 320, 3),
                                   (37, 2080, 5), (100, 4096, 8), (259, 11008, 2),
                                   (17, 4096, 4), (8, 256, 6), (9, 512, 7)])
def test_gemv_within_tolerance(fmt, m, k, n):
    _say("gemv", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=21)
    x = synth.activations(k, n, seed=21, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x)
    yref, s = oracle.dot(fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv {fmt} {m}x{k} n={n}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", [(4096, 4096), (6000, 2048), (3000, 4096)])
def test_gemv_four_columns_either_path(fmt, m, k):
    """Four columns where the dispatcher picks the vector-ALU kernel (a row
    group for every CU, one step per workgroup) or the matrix cores next to
    it: 4096 rows take the vector kernel for every format, 6000 rows of 2048
    the vector kernel for Q4_x / Q5_x and the matrix cores for Q8_0, 3000 rows
    the reverse.  Every output against the oracle, bitwise repeatable."""
    _say("gemv four columns", fmt, m, k)
    w = _weights(fmt, m, k, seed=48)
    x = synth.activations(k, 4, seed=48, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x)
    yref, s = oracle_rows(oracle.dot, fmt, w, m, k, x, 4)
    assert_within(y, yref, s, GEMV_TOL, f"gemv four columns {fmt} {m}x{k}")
    assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(11001, 4096, 5), (20003, 1024, 6), (9000, 2048, 8), (5000, 4096, 7),
                                   (20001, 4096, 4)])
def test_gemv_matrix_cores_many_rounds(fmt, m, k, n):
    """Matrix-core launches whose workgroups run two or more rounds of
    row-quads (the partial sums of a row-quad's waves then meet through a
    per-round LDS counter, no barrier): the pairs of a row split over 4, 1, 2
    and 4 waves, uneven row-quad counts per workgroup, a last round with
    fewer row-quads than slots and a partial last row-quad.  Every output
    against the oracle, bitwise repeatable."""
    _say("gemv matrix cores many rounds", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=49)
    x = synth.activations(k, n, seed=49, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x)
    yref, s = oracle_rows(oracle.dot, fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv many rounds {fmt} {m}x{k} n={n}")
    assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x).view(np.uint32))


@pytest.mark.parametrize("w_off", [0, 2])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(70, 4224, 3), (100, 9216, 5), (33, 8320, 8), (9, 12288, 4)])
def test_gemv_restaged_windows(fmt, m, k, n, w_off):
    """Rows longer than one 4096-weight activation window with 3..8 columns,
    aligned and 2 bytes off: the first window is staged through registers,
    each later one in batches of columns (unaligned Q8_0: the per-float4
    loop); the last window is partial (128 or 1024 weights: fewer float4s
    than threads) except at k = 12288."""
    _say("gemv restaged windows", fmt, m, k, n, w_off)
    w = _weights(fmt, m, k, seed=47)
    x = synth.activations(k, n, seed=47, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x, w_off=w_off)
    yref, s = oracle.dot(fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv restaged {fmt} {m}x{k} n={n}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("w_off,x_off,ldx,ldy", [(2, 0, None, None), (0, 1, None, None),
                                                 (0, 0, 4100, 70), (6, 3, 4133, 65)])
def test_gemv_strides_and_unaligned(fmt, w_off, x_off, ldx, ldy):
    m, k, n = 64, 4096, 3
    _say("gemv strided", fmt, w_off, x_off, ldx, ldy)
    w = _weights(fmt, m, k, seed=22)
    x = synth.activations(k, n, seed=22, tensor_id=2)
    y = _gpu_gemv(fmt, w, m, k, x, ldx=ldx, ldy=ldy, w_off=w_off, x_off=x_off)
    yref, s = oracle.dot(fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv strided {fmt}")


def test_gemv_hand_worked_exact():
    with open(GOLDEN) as f:
        g = json.load(f)
    byname = {b["name"]: b for b in g["blocks"]}
    for case in g["dots"]:
        _say("gemv golden", case["name"])
        if "rows_hex" in case:
            w = np.concatenate([np.frombuffer(bytes.fromhex(r.replace(" ", "")), np.uint8)
                                for r in case["rows_hex"]])
        else:
            w = np.concatenate([np.frombuffer(bytes.fromhex(byname[b]["bytes_hex"].replace(" ", "")), np.uint8)
                                for b in case["blocks"]])
        t = np.arange(case["k"])
        x = {"t+1": t + 1.0, "(t mod 7) - 3": (t % 7) - 3.0}[case["x_rule"]].astype(np.float32)
        y = _gpu_gemv(case["fmt"], w, case["m"], case["k"], x[None, :])
        assert [float(v) for v in y[0]] == [float(Fraction(v)) for v in case["y"]]


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_unit_vectors_and_zero(fmt):
    m, k = 40, 512
    _say("gemv unit", fmt)
    w = _weights(fmt, m, k, seed=23)
    cols = [0, 15, 16, 31, 32, 255, 511, 300]
    x = np.zeros((len(cols), k), np.float32)
    for j, c in enumerate(cols):
        x[j, c] = 1.0
    y = _gpu_gemv(fmt, w, m, k, x)
    W = oracle.dequantize_f32(fmt, w, m, k)
    for j, c in enumerate(cols):
        assert np.array_equal(y[j], W[:, c])
    y0 = _gpu_gemv(fmt, w, m, k, np.zeros((1, k), np.float32))
    assert np.all(y0 == 0)


def test_gemv_adversarial_rows():
    """Rows whose weights nearly cancel: Q4_0 codes mostly 8 with a few 7/9,
    and Q4_1 rows with d*q close to -m."""
    k = 4096
    nb = k // 32
    rng = np.random.default_rng(5)
    # Q4_0
    codes = np.full((4 * nb, 32), 8)
    hit = rng.random(codes.shape) < 0.03
    codes[hit] = rng.choice([7, 9], size=hit.sum())
    dbits = np.full(4 * nb, 0x2A00, dtype=np.uint16)
    w = synth.pack_blocks("q4_0", dbits, codes)
    x = synth.activations(k, 2, seed=31, tensor_id=1)
    x[1] *= 1e4
    y = _gpu_gemv("q4_0", w, 4, k, x)
    yref, s = oracle.dot("q4_0", w, 4, k, x, 2)
    assert_within(y, yref, s, GEMV_TOL, "adversarial q4_0")
    # Q4_1: d = 2^-6, m = -7 * d, so codes 6..8 give tiny weights
    codes = rng.choice([6, 7, 8], size=(4 * nb, 32))
    dbits = np.full(4 * nb, 0x2400, dtype=np.uint16)
    mbits = np.full(4 * nb, np.float16(-7 * 2.0 ** -6).view(np.uint16), dtype=np.uint16)
    w = synth.pack_blocks("q4_1", dbits, codes, m_bits=mbits)
    y = _gpu_gemv("q4_1", w, 4, k, x)
    yref, s = oracle.dot("q4_1", w, 4, k, x, 2)
    assert_within(y, yref, s, GEMV_TOL, "adversarial q4_1")


def test_gemv_side_stream():
    t = torch()
    m, k = 96, 4096
    w = _weights("q8_0", m, k, seed=24)
    x = synth.activations(k, 1, seed=24, tensor_id=2)
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        y = _gpu_gemv("q8_0", w, m, k, x, stream=s.cuda_stream)
    s.synchronize()
    yref, sc = oracle.dot("q8_0", w, m, k, x, 1)
    assert_within(y, yref, sc, GEMV_TOL, "side stream")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 64, 4), (3, 512, 5), (5, 1088, 8), (63, 2112, 4), (1001, 4096, 6),
                                   (257, 1024, 7), (20000, 4096, 4), (4099, 2048, 8)])
def test_gemv_matrix_core_path(fmt, m, k, n):
    """The 4..8-column GEMV on the matrix cores (aligned weights, even block
    count, k <= 4096): a row-quad split over 1, 2 or 4 waves (16, 32 or 64
    pairs per row, ragged pair counts), ragged last row-quads, several rounds
    per workgroup; every output against the oracle, and a second launch
    bitwise equal to the first (the partial sums meet in a fixed order)."""
    _say("gemv matrix cores", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=58)
    x = synth.activations(k, n, seed=58, tensor_id=3)
    y = _gpu_gemv(fmt, w, m, k, x)
    yref, s = oracle_rows(oracle.dot, fmt, w, m, k, x, n)
    assert_within(y, yref, s, GEMV_TOL, f"gemv matrix cores {fmt} {m}x{k} n={n}")
    assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x).view(np.uint32))


def test_gemv_full_config1():
    """Q8_0 4096 x 4096, batch 1: every output against the oracle."""
    cfg = synth.WORKLOADS["gemv_q8_0_4096x4096_n1"]
    seed = synth.workload_seed(cfg["id"])
    _say("gemv full config1")
    w = synth.quant_matrix("q8_0", cfg["m"], cfg["k"], seed=seed, tensor_id=0, d_range=cfg["d"])
    x = synth.activations(cfg["k"], 1, seed=seed, tensor_id=100)
    y = _gpu_gemv("q8_0", w, cfg["m"], cfg["k"], x)
    yref, s = oracle.dot("q8_0", w, cfg["m"], cfg["k"], x, 1)
    assert_within(y, yref, s, GEMV_TOL, "config1")


_CONFIG2 = {}


def _config2():
    """Q4_1 11008 x 4096, its 8-column activation draw and the oracle's
    products for all 8 columns (columns 1..n serve every n)."""
    if not _CONFIG2:
        cfg = synth.WORKLOADS["gemv_q4_1_11008x4096"]
        seed = synth.workload_seed(cfg["id"])
        w = synth.quant_matrix("q4_1", cfg["m"], cfg["k"], seed=seed, tensor_id=0, d_range=cfg["d"],
                               m_range=cfg["mr"])
        x = np.ascontiguousarray(synth.activations(cfg["k"], 8, seed=seed, tensor_id=100))
        yref, s = oracle_rows(oracle.dot, "q4_1", w, cfg["m"], cfg["k"], x, 8)
        _CONFIG2.update(w=w, x=x, yref=yref, s=s, m=cfg["m"], k=cfg["k"])
    return _CONFIG2


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_gemv_full_config2(n):
    """Q4_1 11008 x 4096 with n columns (first n of one 8-column draw): every
    output against the oracle."""
    c = _config2()
    _say("gemv config2", n)
    y = _gpu_gemv("q4_1", c["w"], c["m"], c["k"], c["x"][:n])
    assert_within(y, c["yref"][:n], c["s"][:n], GEMV_TOL, f"config2 n={n}")


_Q5_FULL = {}


@pytest.mark.parametrize("fmt", ["q5_0", "q5_1"])
@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_gemv_q5_full_size(fmt, n):
    """Q5_0 / Q5_1 11008 x 4096 (the Q4_1 workload's shape) with n columns,
    the first n of one 8-column draw: every output against the oracle, on
    the one-column, two-column and matrix-core kernels."""
    if fmt not in _Q5_FULL:
        m, k = 11008, 4096
        w = synth.quant_matrix(fmt, m, k, seed=57, tensor_id=0, d_range=D_RANGE[fmt])
        x = np.ascontiguousarray(synth.activations(k, 8, seed=57, tensor_id=100))
        yref, s = oracle_rows(oracle.dot, fmt, w, m, k, x, 8)
        _Q5_FULL[fmt] = (w, x, yref, s, m, k)
    w, x, yref, s, m, k = _Q5_FULL[fmt]
    _say("gemv q5 full", fmt, n)
    y = _gpu_gemv(fmt, w, m, k, x[:n])
    assert_within(y, yref[:n], s[:n], GEMV_TOL, f"q5 full {fmt} n={n}")


def test_gemv_full_config3():
    """The 7B-shaped layer: q, k, v, o, gate, up, down (Q4_0, batch 1), each
    as its own launch, every output against the oracle."""
    cfg = synth.WORKLOADS["gemv_q4_0_decode_layer"]
    seed = synth.workload_seed(cfg["id"])
    for tid, (name, m, k) in enumerate(cfg["layer"]):
        _say("gemv config3", name, m, k)
        w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        x = synth.activations(k, 1, seed=seed, tensor_id=100 + tid)
        y = _gpu_gemv("q4_0", w, m, k, x)
        yref, s = oracle_rows(oracle.dot, "q4_0", w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"config3 {name}")


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _gpu_gemm(fmt, w, m, k, xh, ldx=None, ldy=None, x_off=0, w_off=0):
    n = xh.shape[0]
    ldx = k if ldx is None else ldx
    ldy = m if ldy is None else ldy
    hw, wp = to_dev_bytes(w, w_off)
    hx, xp = x_dev(xh.view(np.uint16), ldx, np.uint16, x_off)
    out = Guarded(((n - 1) * ldy + m) * 4)
    st = qk.qk_mul_mat(fmt, wp, m, k, xp, n, ldx, out.ptr, ldy, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    y = out.host(np.float32)
    assert out.guards_intact(), "mul_mat wrote outside its output"
    del hw, hx
    return np.stack([y[j * ldy: j * ldy + m] for j in range(n)])


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 32, 1), (130, 96, 3), (128, 128, 128), (257, 640, 129),
                                   (64, 4096, 200), (300, 2080, 17)])
def test_gemm_within_tolerance(fmt, m, k, n):
    _say("gemm", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=41)
    xh = synth.activations(k, n, seed=41, tensor_id=2, dtype=np.float16)
    y = _gpu_gemm(fmt, w, m, k, xh)
    yref, s = oracle.dot(fmt, w, m, k, xh.view(np.uint16), n, x_is_f16=True)
    assert_within(y, yref, s, GEMM_TOL, f"gemm {fmt} {m}x{k} n={n}")


@pytest.mark.parametrize("fmt", GEMM_FMTS)
def test_gemm_strides_and_unaligned(fmt):
    m, k, n = 200, 1024, 70
    _say("gemm strided", fmt)
    w = _weights(fmt, m, k, seed=42)
    xh = synth.activations(k, n, seed=42, tensor_id=2, dtype=np.float16)
    for ldx, ldy, x_off, w_off in ((1030, 203, 1, 2), (1024, 200, 3, 0), (1032, 204, 0, 0)):
        y = _gpu_gemm(fmt, w, m, k, xh, ldx=ldx, ldy=ldy, x_off=x_off, w_off=w_off)
        yref, s = oracle.dot(fmt, w, m, k, xh.view(np.uint16), n, x_is_f16=True)
        assert_within(y, yref, s, GEMM_TOL, f"gemm strided {fmt} {ldx} {ldy} {x_off}")


def test_gemm_matches_exact_fp16_weight_products():
    """Each term uses the fp16 dequantized weight: with one-hot activations
    the GEMM returns exactly the fp16 weights (as fp32)."""
    m, k = 150, 256
    w = _weights("q4_1", m, k, seed=43)
    cols = [0, 31, 32, 100, 255]
    xh = np.zeros((len(cols), k), np.float16)
    for j, c in enumerate(cols):
        xh[j, c] = 1.0
    y = _gpu_gemm("q4_1", w, m, k, xh)
    W16 = oracle.dequantize_f16("q4_1", w, m, k).view(np.float16).astype(np.float32)
    for j, c in enumerate(cols):
        assert np.array_equal(y[j], W16[:, c])


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("m,k", [(300, 256), (77, 160), (129, 32)])
def test_gemm_identity_gives_fp16_weights(fmt, m, k):
    """With X = I (n = k one-hot columns) every output is one fp16 weight:
    Y[j] == f16(W)[:, j] exactly, which pins the placement of every element
    of every block (k = 160 has an odd block count)."""
    _say("gemm identity", fmt, m, k)
    w = _weights(fmt, m, k, seed=44)
    xh = np.eye(k, dtype=np.float16)
    y = _gpu_gemm(fmt, w, m, k, xh)
    W16 = oracle.dequantize_f16(fmt, w, m, k).view(np.float16).astype(np.float32)
    assert np.array_equal(y, W16.T), f"gemm identity {fmt} {m}x{k}"


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("m", [1, 7, 8, 9, 15, 16, 17, 33, 263])
@pytest.mark.parametrize("k", [128, 256])
def test_gemm_identity_direct_load_rows(fmt, m, k):
    """The direct-to-LDS GEMM path (k % 128 == 0, aligned operands) with
    X = I: every output is exactly one fp16 weight.  Rows 8-15 of each
    16-row tile sit 4 bytes later in LDS than rows 0-7 (their chunks load from
    4 bytes earlier); these row counts put real rows on both sides of that
    split, in partial tiles, and with m = 1 every other row of the tile is a
    clamped copy of row 0 whose shifted first chunk must not start before the
    weights."""
    _say("gemm identity direct-load rows", fmt, m, k)
    w = _weights(fmt, m, k, seed=45)
    xh = np.eye(k, dtype=np.float16)
    y = _gpu_gemm(fmt, w, m, k, xh)
    W16 = oracle.dequantize_f16(fmt, w, m, k).view(np.float16).astype(np.float32)
    assert np.array_equal(y, W16.T), f"gemm identity direct-load {fmt} {m}x{k}"


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 512, 1), (63, 512, 5), (64, 1024, 17), (65, 512, 32),
                                   (300, 1024, 32), (1000, 512, 9), (300, 512, 33), (257, 1024, 100),
                                   (70, 512, 128), (130, 640, 8), (300, 896, 40), (65, 11008, 16)])
def test_gemm_small_batch_tile(fmt, m, k, n):
    """Up to 32 columns with k % 128 == 0 and at least 16 blocks (up to 128
    where the 256 x 128 tiles would not cover the CUs) the GEMM takes the
    64 x 32 tile for the first multiple of 16 blocks and adds the 4, 8 or 12
    blocks left over (k = 640, 896, 11008 here) in a second launch; the tile
    whose eight waves each multiply one pair of every eight (eight partial
    sums added through LDS): random activations within 1e-2 * S, and
    one-hot activations (column j picks k index 16j + j % 16, so every
    k group and both halves of a pair are hit) give exactly the fp16
    weights."""
    _say("gemm small batch", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=46)
    xh = synth.activations(k, n, seed=46, tensor_id=2, dtype=np.float16)
    y = _gpu_gemm(fmt, w, m, k, xh)
    yref, s = oracle.dot(fmt, w, m, k, xh.view(np.uint16), n, x_is_f16=True)
    assert_within(y, yref, s, GEMM_TOL, f"gemm small batch {fmt} {m}x{k} n={n}")
    cols = [(16 * j + j % 16) % k for j in range(32)]
    xo = np.zeros((32, k), np.float16)
    for j, c in enumerate(cols):
        xo[j, c] = 1.0
    yo = _gpu_gemm(fmt, w, m, k, xo)
    W16 = oracle.dequantize_f16(fmt, w, m, k).view(np.float16).astype(np.float32)
    assert np.array_equal(yo, W16[:, cols].T), f"gemm small batch one-hot {fmt} {m}x{k}"


@pytest.mark.parametrize("fmt", GEMM_FMTS)
def test_gemm_identity_edge_blocks(fmt):
    """The dequantize edge blocks (subnormal, negative and zero scales, code 8
    with a negative scale, Q8_0 -128 / 127, Q4_1 offsets of every sign)
    through the GEMM with X = I: every output is that block's fp16 weight,
    including fp16-subnormal weights (no flush in the packed fp16 dequant or
    the MFMA).  The two blocks whose fp16 weights overflow to +-inf are left
    out: with X = I their infinities meet the zero activations (inf * 0)."""
    w_all, nb = _edge_blocks(fmt)
    bs = synth.BLOCK_BYTES[fmt]
    keep = [i for i in range(nb) if i not in (4, 5)]
    w = np.concatenate([w_all[i * bs:(i + 1) * bs] for i in keep])
    m, k = len(keep), 32
    _say("gemm identity edge", fmt)
    W16 = oracle.dequantize_f16(fmt, w, m, k).view(np.float16)
    assert np.isfinite(W16).all()
    assert (np.abs(W16[W16 != 0]) < np.float16(6.1035e-05)).any()  # fp16 subnormals occur
    y = _gpu_gemm(fmt, w, m, k, np.eye(k, dtype=np.float16))
    assert np.array_equal(y, W16.astype(np.float32).T)


def test_gemm_q4_1_weights_round_through_fp32():
    """Q4_1's fp16 weight is the RNE of the fp32 value d*q + m (itself one
    rounding): where the exact sum lies just above an fp16 tie that the fp32
    rounding lands on, the two-step value is the even neighbour and a single
    rounding of the exact sum would give the other one.  Rows of such blocks
    (d, m, q found by search over fp16 values), times X = I, must give the
    oracle's fp16 weights bit for bit, as must qk_dequantize to fp16."""
    cases = [(0x3556, 0x0001, 3), (0x5156, 0x0062, 3), (0x5556, 0x00C3, 3), (0x5956, 0x0124, 3),
             (0x5956, 0x0185, 3)]
    rows = []
    for d, mm, q in cases:
        blk = np.zeros(20, dtype=np.uint8)
        blk[0:2] = np.array([d], dtype=np.uint16).view(np.uint8)
        blk[2:4] = np.array([mm], dtype=np.uint16).view(np.uint8)
        blk[4:] = q | (q << 4)
        rows.append(blk)
    w = np.concatenate(rows)
    m, k = len(cases), 32
    W16 = oracle.dequantize_f16("q4_1", w, m, k)
    # the two-step value differs from a direct rounding of the exact sum here
    for (d, mm, q), row in zip(cases, W16):
        exact = float(np.uint16(d).view(np.float16)) * q + float(np.uint16(mm).view(np.float16))
        assert row[0] != np.float16(exact).view(np.uint16), (d, mm, q)
    assert np.array_equal(_gpu_dequant("q4_1", w, m, k, "f16"), W16)
    y = _gpu_gemm("q4_1", w, m, k, np.eye(k, dtype=np.float16))
    assert np.array_equal(y, W16.view(np.float16).astype(np.float32).T)


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("m,k,n", [(257, 640, 129), (300, 2080, 17), (512, 4096, 256)])
def test_gemm_against_fp16_weight_product(fmt, m, k, n):
    """Against the exact product of the oracle's fp16 weights and the fp16
    activations (fp64): each product is exact in fp32, so only the fp32
    accumulation rounds, at most k+1 times: |y - ref| <= (k+1) 2^-24 S16."""
    _say("gemm fp16-weight product", fmt, m, k, n)
    w = _weights(fmt, m, k, seed=45)
    xh = synth.activations(k, n, seed=45, tensor_id=2, dtype=np.float16)
    y = _gpu_gemm(fmt, w, m, k, xh)
    W16 = oracle.dequantize_f16(fmt, w, m, k).view(np.float16).astype(np.float64)
    X = xh.astype(np.float64)
    ref = X @ W16.T
    s16 = np.abs(X) @ np.abs(W16).T
    bound = (k + 1) * 2.0 ** -24 * s16
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}"


def test_gemm_full_config4():
    """Q4_0 14336 x 4096 times fp16 4096 x 512: all 7.3 M outputs against the
    fp64 product of the oracle's weights with the activations."""
    cfg = synth.WORKLOADS["gemm_q4_0_14336x4096_n512"]
    seed = synth.workload_seed(cfg["id"])
    _say("gemm config4")
    w = synth.quant_matrix("q4_0", cfg["m"], cfg["k"], seed=seed, tensor_id=0, d_range=cfg["d"])
    xh = synth.activations(cfg["k"], cfg["n"], seed=seed, tensor_id=100, dtype=np.float16)
    y = _gpu_gemm("q4_0", w, cfg["m"], cfg["k"], xh)
    yref, s = gemm_reference(oracle, "q4_0", w, cfg["m"], cfg["k"], xh)
    assert_within(y, yref, s, GEMM_TOL, "config4")


# ---------------------------------------------------------------------------
# grouped GEMV (one launch, several problems)
# ---------------------------------------------------------------------------

def _gpu_gemv_batched(fmt, probs, n, w_offs=None, x_offs=None):
    """probs: list of (w_bytes, m, k, x2d); returns list of (n, m) outputs."""
    holds, tups, outs = [], [], []
    for i, (w, m, k, x2d) in enumerate(probs):
        hw, wp = to_dev_bytes(w, (w_offs or [0] * len(probs))[i])
        hx, xp = x_dev(x2d, k, np.float32, (x_offs or [0] * len(probs))[i])
        out = Guarded(max(((n - 1) * m + m) * 4, 4))
        holds += [hw, hx]
        outs.append(out)
        tups.append((wp, m, k, xp, k, out.ptr, m))
    arr = qk.make_items(tups)
    st = qk.qk_mul_mat_vec_batched(fmt, arr, len(tups), n, _stream())
    assert st == qk.QK_OK, qk.status_string(st)
    res = []
    for (w, m, k, x2d), out in zip(probs, outs):
        y = out.host(np.float32)
        assert out.guards_intact(), "mul_mat_vec_batched wrote outside an output"
        res.append(np.stack([y[j * m:(j + 1) * m] for j in range(n)]) if m else np.zeros((n, 0)))
    del holds
    return res


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [1, 3, 8])
def test_gemv_batched_mixed_shapes(fmt, n):
    shapes = [(37, 2048), (1, 32), (0, 64), (300, 4096), (16, 11008), (5, 96), (64, 256)]
    _say("gemv batched", fmt, n)
    probs = []
    for i, (m, k) in enumerate(shapes):
        w = _weights(fmt, m, k, seed=60 + i) if m else np.zeros(0, np.uint8)
        x = synth.activations(k, n, seed=60 + i, tensor_id=7)
        probs.append((w, m, k, x))
    ys = _gpu_gemv_batched(fmt, probs, n)
    for (w, m, k, x), y in zip(probs, ys):
        if m == 0:
            continue
        yref, s = oracle.dot(fmt, w, m, k, x, n)
        assert_within(y, yref, s, GEMV_TOL, f"batched {fmt} {m}x{k} n={n}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_batched_matches_single_calls_bitwise(fmt):
    """A grouped launch computes every row exactly as a single call does."""
    shapes = [(130, 4096), (77, 2048), (9, 11008)]
    probs = []
    for i, (m, k) in enumerate(shapes):
        probs.append((_weights(fmt, m, k, seed=70 + i), m, k, synth.activations(k, 2, seed=70 + i, tensor_id=3)))
    ys = _gpu_gemv_batched(fmt, probs, 2)
    for (w, m, k, x), y in zip(probs, ys):
        assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_batched_item_order_does_not_matter(fmt):
    """The launcher reorders items (longest rows first); any order of the same
    items gives bitwise the same outputs."""
    shapes = [(40, 4096), (25, 11008), (64, 2048), (7, 8192)]
    probs = []
    for i, (m, k) in enumerate(shapes):
        probs.append((_weights(fmt, m, k, seed=90 + i), m, k, synth.activations(k, 1, seed=90 + i, tensor_id=4)))
    _say("gemv batched order", fmt)
    ys = _gpu_gemv_batched(fmt, probs, 1)
    order = [2, 0, 3, 1]
    ys2 = _gpu_gemv_batched(fmt, [probs[i] for i in order], 1)
    for pos, i in enumerate(order):
        assert np.array_equal(ys[i].view(np.uint32), ys2[pos].view(np.uint32))
    for (w, m, k, x), y in zip(probs, ys):
        yref, s = oracle.dot(fmt, w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"batched order {fmt} {m}x{k}")


def test_gemv_batched_generic_path_and_sixteen_items():
    """16 items, one of them misaligned (forces the 2-byte generic path for the
    whole launch) and one with an odd block count."""
    probs = []
    for i in range(16):
        m, k = 20 + 3 * i, (96 if i == 5 else 1024)
        probs.append((_weights("q4_0", m, k, seed=80 + i), m, k, synth.activations(k, 1, seed=80 + i, tensor_id=2)))
    _say("gemv batched 16 generic")
    w_offs = [0] * 16
    w_offs[3] = 2
    ys = _gpu_gemv_batched("q4_0", probs, 1, w_offs=w_offs)
    for (w, m, k, x), y in zip(probs, ys):
        yref, s = oracle.dot("q4_0", w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"batched generic {m}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_batched_two_rows_per_wave_generic(fmt):
    """A grouped one-column launch past 64 rows per CU (two rows per wave)
    whose items take the generic path (43-block rows, one item 2-byte
    aligned): every row of every item against the oracle, and bitwise equal
    to separate launches of the same items."""
    shapes = [(16403, 1376, 0), (301, 4096, 2), (77, 2080, 0)]
    _say("gemv batched two rows generic", fmt)
    probs = []
    for i, (m, k, _) in enumerate(shapes):
        probs.append((_weights(fmt, m, k, seed=47, tid=i), m, k,
                      synth.activations(k, 1, seed=47, tensor_id=10 + i)))
    ys = _gpu_gemv_batched(fmt, probs, 1, w_offs=[o for (_, _, o) in shapes])
    for (w, m, k, x), y, (_, _, off) in zip(probs, ys, shapes):
        yref, s = oracle.dot(fmt, w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"batched two rows {fmt} {m}x{k}")
        assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x, w_off=off).view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_batched_two_rows_per_wave_aligned(fmt):
    """A grouped one-column launch past 64 rows per CU on the aligned path
    (two rows per wave, problems from the table, 4-byte aligned weights with
    an even block count): every output of every item against the oracle, and
    bitwise equal to separate launches."""
    shapes = [(16403, 4096), (301, 2048), (77, 8192)]
    _say("gemv batched two rows aligned", fmt)
    probs = []
    for i, (m, k) in enumerate(shapes):
        probs.append((_weights(fmt, m, k, seed=53, tid=i), m, k,
                      synth.activations(k, 1, seed=53, tensor_id=10 + i)))
    ys = _gpu_gemv_batched(fmt, probs, 1)
    for (w, m, k, x), y in zip(probs, ys):
        yref, s = oracle_rows(oracle.dot, fmt, w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"batched two rows aligned {fmt} {m}x{k}")
        assert np.array_equal(y.view(np.uint32), _gpu_gemv(fmt, w, m, k, x).view(np.uint32))


def test_gemv_batched_full_config3():
    """The whole 7B-shaped decode layer in one launch (Q4_0, batch 1): every
    output of every matrix against the oracle."""
    cfg = synth.WORKLOADS["gemv_q4_0_decode_layer"]
    seed = synth.workload_seed(cfg["id"])
    _say("gemv batched config3")
    probs = []
    for tid, (name, m, k) in enumerate(cfg["layer"]):
        w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        probs.append((w, m, k, synth.activations(k, 1, seed=seed, tensor_id=100 + tid)))
    ys = _gpu_gemv_batched("q4_0", probs, 1)
    for tid, ((w, m, k, x), y) in enumerate(zip(probs, ys)):
        yref, s = oracle_rows(oracle.dot, "q4_0", w, m, k, x, 1)
        assert_within(y, yref, s, GEMV_TOL, f"batched config3 item {tid}")
