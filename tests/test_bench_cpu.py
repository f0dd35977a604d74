"""Host-side pieces of bench.py (no GPU): the one-GPU guard, roofline choice,
cold-copy counts, and the threaded oracle helper against a single call."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from dequant_quantized_gemv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_gemv_roofline_picks_the_larger_time():
    m, k = 11008, 4096
    # one and four columns: the HBM time of the algorithmic bytes is the larger
    for n in (1, 4):
        r = bench.gemv_roofline("q4_1", m, k, n, 10e-6)
        assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBPS
    # eight columns: 2*m*k*n flops at the fp32 vector peak take longer than the bytes
    r = bench.gemv_roofline("q4_1", m, k, 8, 20e-6)
    assert r["bound"] == "alu" and r["peak"] == bench.VALU_F32_PEAK_TFLOPS
    t_alu = 2.0 * m * k * 8 / (bench.VALU_F32_PEAK_TFLOPS * 1e12)
    assert abs(r["frac"] - round(t_alu / 20e-6, 4)) < 1e-9


def test_cold_copies_cover_a_gibibyte():
    for nbytes in (17_825_792, 28_180_480, 113_836_032, 33_030_144):
        r = bench.copies_for(nbytes)
        assert r * nbytes >= 1 << 30 and (r - 1) * nbytes < 1 << 30 or r == 2


def test_threaded_oracle_rows_match_one_call():
    m, k = 37, 256
    w = synth.quant_matrix("q4_0", m, k, seed=5, tensor_id=0, d_range=(1e-3, 2e-2))
    x = np.ascontiguousarray(synth.activations(k, 2, seed=5, tensor_id=1))
    y1, s1 = oracle.dot("q4_0", w, m, k, x, 2)
    y4, s4, _ = bench.oracle_rows(oracle.dot, "q4_0", w, m, k, 4, x, 2)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)
