"""Benchmark of the quantized dequantize / GEMV / GEMM hot path on one MI355X.

Headline: Q8_0 GEMV, W 4096 x 4096 times one fp32 activation column
(x ~ N(0,1)), y = W x in fp32.  A step is one qk_mul_mat_vec call (block
decode, fused dequantize + dot products, wave reduction, dispatch).  The same
line carries every workload (dequantize, the Q4_1 GEMV at 1/2/4/8 columns, the
7B-shaped Q4_0 decode layer, the Q4_0 GEMM) and the next rows (8-bit
activations, expert-indexed decode, one GPU's tensor-parallel share, small
GEMM batches) under "configs" and "extras".

Measurement
  * Inputs live in HBM before the timed region.  Every working set here fits
    in the 256 MB Infinity Cache, so each workload rotates through R copies of
    its weights (R * |W| >= 1 GiB): step i reads copy i % R, never
    cache-resident.
  * Steps are issued by a native launch loop (libqk_bench.so: no interpreter
    between launches, so the GPU never waits for the host) on one stream.  W
    warm-up steps, a device synchronization, then K timed steps between two
    HIP events recorded on that stream, and a synchronization.  Before each
    workload's warm-up the GPU's clocks are brought out of their idle state by
    streaming reads of an unrelated buffer (host-side work such as the oracle
    checks leaves the GPU idle for seconds).
  * Per-launch distribution: 20 warm-up launches, then 200 launches with an
    event after every 10 (an event between single launches adds its own cost
    to each); median, p10 and p90 of the per-launch time of the 20 groups.
  * Parity first: before a workload is timed its output is checked against
    the CPU oracle on every element (bit-exact for dequantize, within 1e-4*S
    for the GEMVs, 1e-2*S for the GEMM); after timing, the output of the last
    timed launch must equal the checked one bit for bit.
  * Rooflines: HBM 8 TB/s; fp16 dense MFMA 2.5 PFLOP/s; fp32 vector ALU
    157.3 TFLOP/s, the published figure, which plain (non-packed) fp32 FMAs
    reach on gfx950 too: a wave's FMA issues in two cycles, and the register
    loop timed beside the Q4_1 GEMV (32 independent chains, 16 waves per CU)
    runs near it.  The Q4_1 GEMV is reported against max(HBM time, ALU time);
    the GEMM against the MFMA peak.
  * cpu_baseline: the oracle (plain C++, fp64) timed on this host: one thread on
    a bounded row sample (scaled), and T threads (T = CPUs in the affinity
    mask) over the whole workload, which is also the parity reference.

Options: --quick skips the extras; --headline-only times the headline alone
(for profiler runs); --no-cpu skips the single-thread baseline legs.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CPU_MIN_S = 2.0  # wall seconds of the headline's T-thread oracle timing
MFMA_F16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
COLD_BYTES = 1 << 30
SETTLE_MS = 30.0
DIST_WARMUP, DIST_LAUNCHES, DIST_GROUP = 20, 200, 10
PROFILES = os.path.join(ROOT, "profiles")
GEMV_SOURCES = ["gemv.hip", "gemv.h", "gemv_impl.h", "gemv_n1.hip", "qk_common.h",
                "qk_internal.h"]
METRIC = "effective weight GB/s (% of HBM peak) for Q4_0/Q8_0 GEMV; batched TFLOP/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# native launch loop and ceilings (libqk_bench.so)
# ---------------------------------------------------------------------------

_CALL_FIELDS = [("op", "i"), ("fmt", "i"), ("w", "p"), ("m", "i"), ("k", "i"), ("x", "p"),
                ("n", "i"), ("ldx", "i"), ("y", "p"), ("ldy", "i"), ("out_dtype", "i"),
                ("items", "p"), ("count", "i"), ("n_experts", "i"), ("expert_stride", "i"),
                ("ids", "p"), ("ld_ids", "i"), ("n_used", "i"), ("n_tokens", "i"),
                ("x_slot", "i"), ("x_tok", "i"), ("y_slot", "i"), ("y_tok", "i")]


class QkbCall(ctypes.Structure):
    """struct qkb_call of bench_support.hip: one qk C ABI call."""
    _fields_ = [(n, ctypes.c_int64 if t == "i" else ctypes.c_void_p) for n, t in _CALL_FIELDS]


OPS = {"dequantize": 0, "mul_mat_vec": 1, "mul_mat_vec_x8": 2, "mul_mat_vec_batched": 3,
       "mul_mat_vec_id": 4, "mul_mat": 5, "stream_read": 6}


class Runner:
    """Steps of qk calls issued and timed by the native loop on one stream."""

    def __init__(self, torch):
        self.t = torch
        path = os.path.join(ROOT, "dequant_quantized_gemv_amd", "libqk_bench.so")
        if not os.path.exists(path):
            raise SystemExit(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.qkb_time_steps.argtypes = [ctypes.POINTER(QkbCall), ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
        lib.qkb_time_steps.restype = ctypes.c_int
        lib.qkb_settle.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_double, vp]
        lib.qkb_settle.restype = ctypes.c_int
        lib.qkc_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        lib.qkc_mfma_loop.restype = ctypes.c_int
        lib.qkc_valu_loop.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        lib.qkc_valu_loop.restype = ctypes.c_int
        self.lib = lib
        self.stream = torch.cuda.Stream()
        self.sink = torch.zeros(64, device="cuda")
        self.settle_buf = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")

    @staticmethod
    def call(op, **kw):
        c = QkbCall()
        c.op = OPS[op]
        for name, v in kw.items():
            setattr(c, name, v)
        return c

    def stream_read(self, ptr, nbytes):
        return self.call("stream_read", w=ptr, k=nbytes, y=self.sink.data_ptr())

    def settle(self, ms=SETTLE_MS):
        if ms > 0 and self.lib.qkb_settle(self.settle_buf.data_ptr(), self.settle_buf.numel(),
                                          self.sink.data_ptr(), ms, self.stream.cuda_stream) != 0:
            raise RuntimeError("qkb_settle failed")

    def time_steps(self, variants, warmup, steps, group=0):
        """variants: list (rotation) of lists of QkbCall (one step each).
        Returns (seconds for the timed steps, and with group > 0 the seconds
        per step of each group of `group` consecutive steps, else None)."""
        per = len(variants[0])
        arr = (QkbCall * (per * len(variants)))()
        for v, calls in enumerate(variants):
            assert len(calls) == per
            for j, c in enumerate(calls):
                arr[v * per + j] = c
        total = ctypes.c_float()
        ng = steps // group if group > 0 else 0
        dist = (ctypes.c_float * ng)() if group > 0 else None
        st = self.lib.qkb_time_steps(arr, per, len(variants), warmup, steps, max(group, 1),
                                     self.stream.cuda_stream, ctypes.byref(total), dist)
        if st != 0:
            raise RuntimeError(f"qkb_time_steps failed with status {st}")
        return total.value / 1e3, (np.array(dist[:], dtype=np.float64) / 1e3 / group if group > 0 else None)

    def measure(self, variants, steps, warmup):
        """Settle, W warm-up + K timed steps back to back, then the per-step
        distribution: 20 warm-up steps and 200 timed ones, in groups of 10."""
        self.settle()
        sec, _ = self.time_steps(variants, warmup, steps)
        _, d = self.time_steps(variants, DIST_WARMUP, DIST_LAUNCHES, group=DIST_GROUP)
        return dict(us=sec / steps * 1e6, median_us=float(np.median(d)) * 1e6,
                    p10_us=float(np.percentile(d, 10)) * 1e6, p90_us=float(np.percentile(d, 90)) * 1e6)

    def valu_loop_tflops(self):
        """Plain fp32 FMA rate of a register-only loop over every CU (TFLOP/s)."""
        wgs = self.t.cuda.get_device_properties(0).multi_processor_count
        iters = 20000
        self.settle()
        best = math.inf
        for _ in range(3):
            e0 = self.t.cuda.Event(enable_timing=True)
            e1 = self.t.cuda.Event(enable_timing=True)
            with self.t.cuda.stream(self.stream):
                e0.record(self.stream)
                if self.lib.qkc_valu_loop(wgs, iters, self.sink.data_ptr(), self.stream.cuda_stream) != 0:
                    raise RuntimeError("qkc_valu_loop failed")
                e1.record(self.stream)
            self.t.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        return wgs * 1024 * iters * 32 * 2.0 / best / 1e12

    def mfma_loop_tflops(self):
        """fp16 MFMA rate of a register-only loop over every CU (TFLOP/s)."""
        wgs = self.t.cuda.get_device_properties(0).multi_processor_count
        iters = 4000
        self.settle()
        best = math.inf
        for _ in range(3):
            e0 = self.t.cuda.Event(enable_timing=True)
            e1 = self.t.cuda.Event(enable_timing=True)
            with self.t.cuda.stream(self.stream):
                e0.record(self.stream)
                if self.lib.qkc_mfma_loop(wgs, iters, self.sink.data_ptr(), self.stream.cuda_stream) != 0:
                    raise RuntimeError("qkc_mfma_loop failed")
                e1.record(self.stream)
            self.t.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        return wgs * 8 * iters * 32 * (2.0 * 16 * 16 * 32) / best / 1e12


def rnd(v, nd=3):
    return None if v is None else round(float(v), nd)


def timing_fields(t):
    return {"us_per_step": rnd(t["us"]), "median_us": rnd(t["median_us"]), "p10_us": rnd(t["p10_us"]),
            "p90_us": rnd(t["p90_us"])}


def copies_for(nbytes, minimum=2):
    return max(minimum, math.ceil(COLD_BYTES / max(nbytes, 1)))


def rotation(torch, t, nbytes):
    """[t, copies...]: R tensors, R * nbytes >= 1 GiB."""
    R = copies_for(nbytes)
    return [t] + [t.clone() for _ in range(R - 1)]


def warm_fields(c, variants, nbytes, unit="weight_GBps", flops=None):
    """The first copy's launch repeated (its bytes stay in the 256 MB
    Infinity Cache): W warm-up and K timed launches, labelled as such."""
    sec, _ = c.run.time_steps(variants[:1], c.warmup, c.steps)
    us = sec / c.steps * 1e6
    rec = {"label": "MALL-resident, not HBM (one buffer repeated)", "us_per_step": rnd(us)}
    if flops is not None:
        rec["TFLOPs"] = rnd(flops / (us / 1e6) / 1e12, 1)
    else:
        rec[unit] = rnd(nbytes / (us / 1e6) / 1e9, 1)
    return rec


# ---------------------------------------------------------------------------
# oracle helpers (parity reference and CPU baseline)
# ---------------------------------------------------------------------------

def host_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


BLOCK_BYTES = {"q4_0": 18, "q4_1": 20, "q8_0": 34}


def row_bytes(fmt, k):
    return (k // 32) * BLOCK_BYTES[fmt]


def oracle_rows(fn, fmt, w, m, k, threads, *args):
    """fn(fmt, w_rows, rows, k, *args) -> (y (n, rows), s (n, rows)) over row
    ranges in `threads` host threads (the oracle's C calls release the GIL);
    returns the concatenated (y, s) and the wall time."""
    rb = row_bytes(fmt, k)
    step = max(1, -(-m // (threads * 4)))
    chunks = [(r, min(m, r + step)) for r in range(0, m, step)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda c: fn(fmt, w[c[0] * rb:c[1] * rb], c[1] - c[0], k, *args), chunks))
    el = time.perf_counter() - t0
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1), el


def single_thread_rows(fn, fmt, w, m, k, budget_s, *args):
    """One thread on the first r rows, r grown until the call takes about
    budget_s; returns (rows, seconds)."""
    rb = row_bytes(fmt, k)
    r = min(m, 16)
    while True:
        t0 = time.perf_counter()
        fn(fmt, w[:r * rb], r, k, *args)
        el = time.perf_counter() - t0
        if el >= budget_s or r == m:
            return r, el
        r = min(m, max(r * 2, int(r * budget_s / max(el, 1e-6))))


def within(y, yr, s, rel):
    """Every element: |y - yr| <= rel * S (NaN or inf anywhere fails); returns
    (ok, max |y - yr| / S)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - yr)
    ok = bool(np.all(err <= rel * s)) and bool(np.all(np.isfinite(y)))
    worst = float(np.max(err / np.where(s > 0, s, 1))) if err.size else 0.0
    return ok, worst


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dequant_quantized_gemv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key, sources):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (profiles/<kernel_key>_traffic.md, lines `source_hash: ...` and
    `traffic_bytes_per_launch: ...`), or None when those counters were taken
    on a different version of the kernel source."""
    path = os.path.join(PROFILES, f"{kernel_key}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                rec[k.strip().strip("`* -")] = v.strip().strip("`* ")
    if rec.get("source_hash") != kernel_source_hash(sources):
        return None
    try:
        return int(float(rec["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib):
    """A plain device copy of a known size (for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE): reads and writes `mib` MiB, five times."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB read + {mib} MiB written per copy, 5 copies")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class Ctx:
    def __init__(self, torch, qk, synth, oracle, run, args):
        self.torch, self.qk, self.synth, self.oracle, self.run = torch, qk, synth, oracle, run
        self.steps, self.warmup = args.steps, args.warmup
        self.threads = host_threads()
        self.single = not args.no_cpu
        self.budget = args.cpu_budget


def gemv_roofline(fmt, m, k, n, sec):
    """Roofline of a fp32-activation GEMV launch: HBM for the algorithmic
    bytes, and the fp32 vector ALU for the 2*m*k*n flops; the bound is the
    larger time."""
    wb = m * row_bytes(fmt, k)
    algo = wb + 4 * n * (k + m)
    t_hbm = algo / (HBM_PEAK_GBPS * 1e9)
    t_alu = 2.0 * m * k * n / (VALU_F32_PEAK_TFLOPS * 1e12)
    if t_alu > t_hbm:
        return {"bound": "alu", "achieved": rnd(2.0 * m * k * n / sec / 1e12, 2),
                "peak": VALU_F32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": rnd(t_alu / sec, 4),
                "hbm_frac": rnd(t_hbm / sec, 4)}
    return {"bound": "hbm", "achieved": rnd(algo / sec / 1e9, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": rnd(t_hbm / sec, 4)}


def run_gemv(c, fmt, m, k, ns, seed, d, mr=None, entry="mul_mat_vec", xtid=100, ceiling=False):
    """Single-GEMV workloads (one per column count in ns, all columns from one
    8-column draw): parity on every output, then timing."""
    torch, qk, synth, oracle = c.torch, c.qk, c.synth, c.oracle
    w = synth.quant_matrix(fmt, m, k, seed=seed, tensor_id=0, d_range=d, **({"m_range": mr} if mr else {}))
    nmax = max(ns)
    x_all = synth.activations(k, 8 if nmax > 1 else 1, seed=seed, tensor_id=xtid)[:nmax]
    x_all = np.ascontiguousarray(x_all)
    ref_fn = oracle.dot if entry == "mul_mat_vec" else oracle.dot_x8
    yr, sr, t_mt = oracle_rows(ref_fn, fmt, w, m, k, c.threads, x_all, nmax)
    wd = torch.from_numpy(w).cuda()
    copies = rotation(torch, wd, w.size)
    xd = torch.from_numpy(x_all).cuda()
    out = {}
    wb = w.size
    for n in ns:
        y = torch.empty((n, m), dtype=torch.float32, device="cuda")
        variants = [[c.run.call(entry, fmt=qk.FORMATS[fmt], w=cp.data_ptr(), m=m, k=k, x=xd.data_ptr(), n=n,
                                ldx=k, y=y.data_ptr(), ldy=m)] for cp in copies]
        c.run.time_steps(variants[:1], 0, 1)
        got = y.cpu().numpy()
        ok, worst = within(got, yr[:n], sr[:n], 1e-4)
        if not ok:
            raise SystemExit(f"{fmt} {m}x{k} n={n} {entry}: parity FAILED before timing (max err/S {worst:.3g})")
        t = c.run.measure(variants, c.steps, c.warmup)
        same = bool(np.array_equal(y.cpu().numpy().view(np.uint32), got.view(np.uint32)))
        if not same:
            raise SystemExit(f"{fmt} {m}x{k} n={n}: timed output differs from the checked one")
        sec = t["us"] / 1e6
        rec = {"parity": f"every output within 1e-4*S{'_x8' if entry != 'mul_mat_vec' else ''}",
               "max_err_over_S": float(f"{worst:.3g}"), **timing_fields(t),
               "weight_GBps": rnd(wb / sec / 1e9, 1), "pct_of_hbm_peak": rnd(100 * wb / sec / 1e9 / HBM_PEAK_GBPS, 2),
               "roofline": gemv_roofline(fmt, m, k, n, sec)}
        rec["warm"] = warm_fields(c, variants, wb)
        if ceiling:
            cs, _ = c.run.time_steps([[c.run.stream_read(cp.data_ptr(), wb)] for cp in copies], c.warmup, c.steps)
            rec["stream_read_us"] = rnd(cs / c.steps * 1e6)
            rec["pct_of_stream_read"] = rnd(100 * (cs / c.steps) / sec, 1)
        out[n] = rec
        del y
    cpu = {"threads": c.threads, "threads_GBps": rnd(wb * nmax / max(nmax, 1) / t_mt / 1e9, 4),
           "threads_sample": f"whole {m}x{k} matrix x {nmax} column(s) ({t_mt:.2f} s)"}
    if c.single:
        r, el = single_thread_rows(ref_fn, fmt, w, m, k, c.budget, x_all, nmax)
        cpu["single_thread_GBps"] = rnd(r * row_bytes(fmt, k) / el / 1e9, 4)
        cpu["single_thread_sample"] = f"first {r} of {m} rows x {nmax} column(s), {el:.2f} s, scaled to the matrix"
    del copies, wd, xd
    torch.cuda.empty_cache()
    return out, cpu, dict(w=w, x=x_all)


def run_headline(c):
    synth = c.synth
    cfg = synth.WORKLOADS["gemv_q8_0_4096x4096_n1"]
    seed = synth.workload_seed(cfg["id"])
    m, k = cfg["m"], cfg["k"]
    res, cpu, keep = run_gemv(c, "q8_0", m, k, (1,), seed, cfg["d"], ceiling=True)
    # the T-thread oracle over whole passes of the matrix, repeated for at
    # least CPU_MIN_S seconds (one pass takes milliseconds)
    passes, el = 0, 0.0
    while el < CPU_MIN_S:
        _, _, t = oracle_rows(c.oracle.dot, "q8_0", keep["w"], m, k, c.threads, keep["x"], 1)
        passes, el = passes + 1, el + t
    cpu["threads_GBps"] = rnd(passes * m * row_bytes("q8_0", k) / el / 1e9, 4)
    cpu["threads_sample"] = f"{passes} passes over the whole {m}x{k} matrix x 1 column ({el:.2f} s)"
    r = res[1]
    sec = r["us_per_step"] / 1e6
    wb = m * row_bytes("q8_0", k)
    algo = wb + 4 * (k + m)
    log(f"headline: {r['us_per_step']} us per step (median {r['median_us']})")
    line = {
        "metric": METRIC,
        "value": rnd(wb / sec / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": c.steps,
        "warmup": c.warmup,
        "ms_per_step": rnd(sec * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gemv_q8_0_4096x4096_n1", "format": "q8_0", "m": m, "k": k, "n": 1,
                   "cold_weight_copies": copies_for(wb), "pct_of_hbm_peak": r["pct_of_hbm_peak"]},
        "timing": {"method": "native launch loop on one stream; HIP events around the K timed steps",
                   "clock_settle_ms": SETTLE_MS,
                   "per_launch_us": {"median": r["median_us"], "p10": r["p10_us"], "p90": r["p90_us"],
                                     "launches": DIST_LAUNCHES, "warmup": DIST_WARMUP,
                                     "over": f"groups of {DIST_GROUP} launches"}},
        "roofline": {"bound": "hbm", "achieved": rnd(algo / sec / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": rnd(algo / sec / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": stored_traffic("gemv_q8_0_4096x4096_n1", GEMV_SOURCES)},
        "warm": r["warm"],
        "practical_ceiling": {"stream_read_us": r["stream_read_us"],
                              "stream_read_GBps": rnd(wb / (r["stream_read_us"] / 1e6) / 1e9, 1),
                              "frac_of_stream_read": rnd(r["pct_of_stream_read"] / 100, 4)},
        "parity": r["parity"] + f" (max err/S {r['max_err_over_S']})",
    }
    cb = {"value": cpu["threads_GBps"], "unit": "GB/s", "cores": cpu["threads"], "kind": "oracle",
          "sample": f"{cpu['threads_sample']} in {cpu['threads']} threads", "cpu_model": cpu_model()}
    if "single_thread_GBps" in cpu:
        cb["single_thread_value"] = cpu["single_thread_GBps"]
        cb["single_thread_sample"] = cpu["single_thread_sample"]
    line["cpu_baseline"] = cb
    return line, r, cpu


def run_dequant(c):
    torch, qk, synth, oracle = c.torch, c.qk, c.synth, c.oracle
    cfg = synth.WORKLOADS["dequant_q4_0_4096x4096_f32"]
    seed = synth.workload_seed(cfg["id"])
    m, k = cfg["m"], cfg["k"]
    w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=0, d_range=cfg["d"])
    rb = row_bytes("q4_0", k)
    step = -(-m // (c.threads * 4))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(c.threads) as ex:
        parts = list(ex.map(lambda r: oracle.dequantize_f32("q4_0", w[r * rb:min(m, r + step) * rb],
                                                             min(m, r + step) - r, k), range(0, m, step)))
    t_mt = time.perf_counter() - t0
    ref = np.concatenate(parts, axis=0)
    wd = torch.from_numpy(w).cuda()
    ins = rotation(torch, wd, w.size + m * k * 4)
    outs = [torch.empty((m, k), dtype=torch.float32, device="cuda") for _ in ins]
    variants = [[c.run.call("dequantize", fmt=qk.QK_Q4_0, w=i.data_ptr(), m=m, k=k, out_dtype=qk.QK_F32,
                            y=o.data_ptr())] for i, o in zip(ins, outs)]
    c.run.time_steps(variants[:1], 0, 1)
    if not np.array_equal(outs[0].cpu().numpy().view(np.uint32), ref.view(np.uint32)):
        raise SystemExit("dequantize: parity FAILED before timing")
    t = c.run.measure(variants, c.steps, c.warmup)
    if not all(torch.equal(o.view(torch.int32), outs[0].view(torch.int32)) for o in outs):
        raise SystemExit("dequantize: timed outputs differ from the checked one")
    sec = t["us"] / 1e6
    total = w.size + m * k * 4
    rec = {"parity": "bit-exact on every output", **timing_fields(t),
           "total_GBps": rnd(total / sec / 1e9, 1), "weight_GBps": rnd(w.size / sec / 1e9, 1),
           "pct_of_hbm_peak": rnd(100 * total / sec / 1e9 / HBM_PEAK_GBPS, 2),
           "roofline": {"bound": "hbm", "achieved": rnd(total / sec / 1e9, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": rnd(total / sec / 1e9 / HBM_PEAK_GBPS, 4)},
           "cpu": {"threads": c.threads, "threads_total_GBps": rnd(total / t_mt / 1e9, 4)}}
    rec["warm"] = warm_fields(c, variants, total, unit="total_GBps")
    if c.single:
        r = max(1, m // 8)
        t0 = time.perf_counter()
        oracle.dequantize_f32("q4_0", w[:r * rb], r, k)
        el = time.perf_counter() - t0
        rec["cpu"]["single_thread_total_GBps"] = rnd(r * (rb + 4 * k) / el / 1e9, 4)
        rec["cpu"]["single_thread_sample"] = f"first {r} of {m} rows, {el:.2f} s"
    del ins, outs, wd
    torch.cuda.empty_cache()
    return rec


def run_layer(c, name, with_cpu=True):
    """The 7 GEMVs of one decode layer: one grouped launch per step, and seven
    separate launches per step; plus each matrix's own launches (the sum of
    their median durations)."""
    torch, qk, synth, oracle = c.torch, c.qk, c.synth, c.oracle
    cfg = synth.WORKLOADS[name]
    seed = synth.workload_seed(cfg["id"])
    probs, wtot, t_mt = [], 0, 0.0
    for tid, (nm, m, k) in enumerate(cfg["layer"]):
        w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        x = np.ascontiguousarray(synth.activations(k, 1, seed=seed, tensor_id=100 + tid))
        yr, sr, el = oracle_rows(oracle.dot, "q4_0", w, m, k, c.threads, x, 1)
        t_mt += el
        probs.append(dict(nm=nm, m=m, k=k, w=w, x=x, yr=yr, sr=sr, wd=torch.from_numpy(w).cuda(),
                          xd=torch.from_numpy(x).cuda(), y=torch.empty((1, m), dtype=torch.float32, device="cuda")))
        wtot += w.size
    R = copies_for(wtot)
    for p in probs:
        p["copies"] = [p["wd"]] + [p["wd"].clone() for _ in range(R - 1)]
    item_sets = [qk.make_items([(p["copies"][r].data_ptr(), p["m"], p["k"], p["xd"].data_ptr(), p["k"],
                                 p["y"].data_ptr(), p["m"]) for p in probs]) for r in range(R)]
    grouped = [[c.run.call("mul_mat_vec_batched", fmt=qk.QK_Q4_0, items=ctypes.addressof(s), count=len(probs),
                           n=1)] for s in item_sets]
    separate = [[c.run.call("mul_mat_vec", fmt=qk.QK_Q4_0, w=p["copies"][r].data_ptr(), m=p["m"], k=p["k"],
                            x=p["xd"].data_ptr(), n=1, ldx=p["k"], y=p["y"].data_ptr(), ldy=p["m"])
                 for p in probs] for r in range(R)]
    worst = 0.0

    def check(what):
        nonlocal worst
        outs = []
        for p in probs:
            got = p["y"].cpu().numpy()
            ok, wr = within(got, p["yr"], p["sr"], 1e-4)
            if not ok:
                raise SystemExit(f"{name} {what} {p['nm']}: parity FAILED (max err/S {wr:.3g})")
            worst = max(worst, wr)
            outs.append(got)
        return outs

    out = {"weight_bytes": wtot, "cold_layer_copies": R}
    for label, variants in (("grouped_launch", grouped), ("separate_launches", separate)):
        for p in probs:
            p["y"].fill_(float("nan"))
        c.run.time_steps(variants[:1], 0, 1)
        checked = check(label)
        t = c.run.measure(variants, c.steps, c.warmup)
        after = [p["y"].cpu().numpy() for p in probs]
        if not all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(after, checked)):
            raise SystemExit(f"{name} {label}: timed outputs differ from the checked ones")
        sec = t["us"] / 1e6
        out[label] = {**timing_fields(t), "weight_GBps": rnd(wtot / sec / 1e9, 1),
                      "pct_of_hbm_peak": rnd(100 * wtot / sec / 1e9 / HBM_PEAK_GBPS, 2)}
        if label == "grouped_launch":
            out[label]["warm"] = warm_fields(c, variants, wtot)
            # practical ceiling: one plain streaming read of as many bytes per
            # step, one launch, over as many cold copies
            span = (wtot + 255) // 256 * 256
            big = torch.empty(R * span, dtype=torch.uint8, device="cuda")
            cs, _ = c.run.time_steps([[c.run.stream_read(big.data_ptr() + r * span, wtot)] for r in range(R)],
                                     c.warmup, c.steps)
            out[label]["stream_read_us"] = rnd(cs / c.steps * 1e6)
            out[label]["pct_of_stream_read"] = rnd(100 * (cs / c.steps) / sec, 1)
            del big
    # each matrix alone: the median of its own launches
    med = {}
    for i, p in enumerate(probs):
        _, d = c.run.time_steps([[separate[r][i]] for r in range(R)], DIST_WARMUP, DIST_LAUNCHES,
                                group=DIST_GROUP)
        med[p["nm"]] = float(np.median(d)) * 1e6
    smed = sum(med.values()) / 1e6
    # (each matrix's launches back to back: a launch's time here includes the
    # gap to the next launch, which the grouped launch pays once)
    out["sum_of_kernel_medians"] = {"us": rnd(smed * 1e6), "per_matrix_median_us": {k: rnd(v) for k, v in med.items()},
                                    "weight_GBps": rnd(wtot / smed / 1e9, 1),
                                    "pct_of_hbm_peak": rnd(100 * wtot / smed / 1e9 / HBM_PEAK_GBPS, 2)}
    out["parity"] = "every output within 1e-4*S (grouped and separate launches)"
    out["max_err_over_S"] = float(f"{worst:.3g}")
    sec = out["grouped_launch"]["us_per_step"] / 1e6
    algo = wtot + sum(4 * (p["k"] + p["m"]) for p in probs)
    out["roofline"] = {"bound": "hbm", "achieved": rnd(algo / sec / 1e9, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": rnd(algo / sec / 1e9 / HBM_PEAK_GBPS, 4), "launch": "grouped"}
    if with_cpu:
        out["cpu"] = {"threads": c.threads, "threads_GBps": rnd(wtot / t_mt / 1e9, 4)}
        if c.single:
            p = max(probs, key=lambda q: q["w"].size)
            r, el = single_thread_rows(oracle.dot, "q4_0", p["w"], p["m"], p["k"], c.budget, p["x"], 1)
            out["cpu"]["single_thread_GBps"] = rnd(r * row_bytes("q4_0", p["k"]) / el / 1e9, 4)
            out["cpu"]["single_thread_sample"] = f"first {r} rows of {p['nm']}, {el:.2f} s"
    del probs, item_sets, grouped, separate
    torch.cuda.empty_cache()
    return out


def gemm_reference(oracle, fmt, w, m, k, xh, threads):
    """fp64 product of the oracle's dequantized fp32 weights with the fp16
    activations (decoded exactly), and S = |W| |X|; (n, m) arrays."""
    rb = row_bytes(fmt, k)
    step = -(-m // (threads * 4))
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r: oracle.dequantize_f32(fmt, w[r * rb:min(m, r + step) * rb],
                                                             min(m, r + step) - r, k), range(0, m, step)))
    wf = np.concatenate(parts, axis=0).astype(np.float64)
    xf = xh.astype(np.float64)  # (n, k): fp16 -> fp64 is exact
    y = xf @ wf.T
    s = np.abs(xf) @ np.abs(wf).T
    return y, s


def run_gemm(c):
    torch, qk, synth, oracle = c.torch, c.qk, c.synth, c.oracle
    cfg = synth.WORKLOADS["gemm_q4_0_14336x4096_n512"]
    seed = synth.workload_seed(cfg["id"])
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=0, d_range=cfg["d"])
    xh = synth.activations(k, n, seed=seed, tensor_id=100, dtype=np.float16)
    t0 = time.perf_counter()
    yr, sr = gemm_reference(oracle, "q4_0", w, m, k, xh, c.threads)
    t_ref = time.perf_counter() - t0
    wd = torch.from_numpy(w).cuda()
    xd = torch.from_numpy(xh).cuda()
    wc = rotation(torch, wd, w.size)
    out, keep = {}, {}
    for nb in (n, 16, 64, 128):
        y = torch.empty((nb, m), dtype=torch.float32, device="cuda")
        variants = [[c.run.call("mul_mat", fmt=qk.QK_Q4_0, w=cp.data_ptr(), m=m, k=k, x=xd.data_ptr(), n=nb, ldx=k,
                                y=y.data_ptr(), ldy=m)] for cp in wc]
        c.run.time_steps(variants[:1], 0, 1)
        got = y.cpu().numpy()
        ok, worst = within(got, yr[:nb], sr[:nb], 1e-2)
        if not ok:
            raise SystemExit(f"GEMM n={nb}: parity FAILED before timing (max err/S {worst:.3g})")
        t = c.run.measure(variants, c.steps, c.warmup)
        if not np.array_equal(y.cpu().numpy().view(np.uint32), got.view(np.uint32)):
            raise SystemExit(f"GEMM n={nb}: timed output differs from the checked one")
        sec = t["us"] / 1e6
        tf = 2.0 * m * nb * k / sec / 1e12
        rec = {"parity": "every output within 1e-2*S", "max_err_over_S": float(f"{worst:.3g}"),
               **timing_fields(t), "TFLOPs": rnd(tf, 1), "pct_of_mfma_f16_peak": rnd(100 * tf / MFMA_F16_PEAK_TFLOPS, 2),
               "roofline": {"bound": "mfma", "achieved": rnd(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": rnd(tf / MFMA_F16_PEAK_TFLOPS, 4)}}
        if nb == n:
            rec["warm"] = warm_fields(c, variants, 0, flops=2.0 * m * nb * k)
            out = rec
        else:
            keep[str(nb)] = rec
        del y
    loop = c.run.mfma_loop_tflops()
    out["mfma_loop_TFLOPs"] = rnd(loop, 1)
    out["pct_of_mfma_loop"] = rnd(100 * out["TFLOPs"] / loop, 1)
    out["cpu"] = {"threads": c.threads, "reference": f"fp64 BLAS product of the oracle's weights ({t_ref:.2f} s)"}
    # the oracle's own products: 16 of the 512 columns, scaled by 32
    x16 = np.ascontiguousarray(xh[:16].view(np.uint16))
    _, _, t_mt = oracle_rows(lambda f, ww, mm, kk, xx, nn: oracle.dot(f, ww, mm, kk, xx, nn, x_is_f16=True),
                             "q4_0", w, m, k, c.threads, x16, 16)
    out["cpu"]["threads_TFLOPs"] = rnd(2.0 * m * 16 * k / t_mt / 1e12, 6)
    out["cpu"]["threads_sample"] = f"16 of {n} columns, whole matrix ({t_mt:.2f} s), scaled by {n // 16}"
    if c.single:
        r, el = single_thread_rows(lambda f, ww, mm, kk, xx, nn: oracle.dot(f, ww, mm, kk, xx, nn, x_is_f16=True),
                                   "q4_0", w, m, k, c.budget, x16, 16)
        out["cpu"]["single_thread_TFLOPs"] = rnd(2.0 * r * 16 * k / el / 1e12, 6)
        out["cpu"]["single_thread_sample"] = f"first {r} rows x 16 of {n} columns, {el:.2f} s, scaled"
    out["smaller_batches"] = keep
    del wc, wd, xd
    torch.cuda.empty_cache()
    return out


def run_moe(c):
    """Expert-indexed decode: per token, the gate, up and down projections of
    8 of 128 Q4_0 experts (768 x 2048, 768 x 2048, 2048 x 768), three
    qk_mul_mat_vec_id calls per step.  Expert choices change every step and
    the stacks rotate over copies."""
    torch, qk, synth, oracle = c.torch, c.qk, c.synth, c.oracle
    cfg = synth.WORKLOADS["gemv_q4_0_moe_experts"]
    seed = synth.workload_seed(cfg["id"])
    ne, nu, nt = cfg["n_experts"], cfg["n_used"], cfg["n_tokens"]
    n_sets = 64
    ids = np.stack([synth.expert_ids(nt, nu, ne, seed=seed, tensor_id=50 + i) for i in range(n_sets)])
    ids_d = torch.from_numpy(ids).cuda()
    stacks = []
    for tid, (nm, m, k) in enumerate(cfg["layer"]):
        w = synth.quant_matrix("q4_0", ne * m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        shared = nm != "down"
        x = synth.activations(k, nt * (1 if shared else nu), seed=seed, tensor_id=100 if shared else 100 + tid)
        stacks.append(dict(nm=nm, m=m, k=k, w=w, wd=torch.from_numpy(w).cuda(), x=x,
                           xd=torch.from_numpy(np.ascontiguousarray(x)).cuda(), shared=shared,
                           y=torch.empty((nt, nu, m), dtype=torch.float32, device="cuda"),
                           one=m * row_bytes("q4_0", k)))
    R = copies_for(sum(p["w"].size for p in stacks))
    for p in stacks:
        p["copies"] = [p["wd"]] + [p["wd"].clone() for _ in range(R - 1)]
    variants = []
    for r in range(max(R, n_sets)):
        step = []
        for p in stacks:
            step.append(c.run.call("mul_mat_vec_id", fmt=qk.QK_Q4_0, w=p["copies"][r % R].data_ptr(), n_experts=ne,
                                   expert_stride=p["one"], m=p["m"], k=p["k"], ids=ids_d[r % n_sets].data_ptr(),
                                   ld_ids=nu, n_used=nu, n_tokens=nt, x=p["xd"].data_ptr(),
                                   x_slot=0 if p["shared"] else p["k"], x_tok=p["k"] if p["shared"] else nu * p["k"],
                                   y=p["y"].data_ptr(), y_slot=p["m"], y_tok=nu * p["m"]))
        variants.append(step)
    c.run.time_steps(variants[:1], 0, 1)
    worst, checked = 0.0, []
    for p in stacks:
        xs = p["x"].reshape(nt, p["k"]) if p["shared"] else p["x"].reshape(nt, nu, p["k"])
        yr, sr = oracle.dot_id("q4_0", p["w"], ne, p["one"], p["m"], p["k"], ids[0], nu, nt, xs,
                               0 if p["shared"] else p["k"], p["k"] if p["shared"] else nu * p["k"])
        got = p["y"].cpu().numpy()
        ok, wr = within(got, yr, sr, 1e-4)
        if not ok:
            raise SystemExit(f"expert decode {p['nm']}: parity FAILED (max err/S {wr:.3g})")
        worst = max(worst, wr)
        checked.append(got)
    t = c.run.measure(variants, c.steps, c.warmup)
    sel = sum(nt * nu * p["one"] for p in stacks)
    sec = t["us"] / 1e6
    out = {"parity": "every output within 1e-4*S", "max_err_over_S": float(f"{worst:.3g}"), **timing_fields(t),
           "launches_per_step": len(stacks), "selected_weight_bytes": sel,
           "weight_GBps": rnd(sel / sec / 1e9, 1), "pct_of_hbm_peak": rnd(100 * sel / sec / 1e9 / HBM_PEAK_GBPS, 2)}
    del stacks, variants
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="skip the extras (next rows)")
    ap.add_argument("--headline-only", action="store_true", help="time the headline GEMV only")
    ap.add_argument("--configs", action="store_true", help="(accepted for compatibility: always on)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the single-thread oracle legs")
    ap.add_argument("--cpu-budget", type=float, default=1.5, metavar="S",
                    help="seconds of single-thread oracle work per workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    import torch
    import oracle
    from dequant_quantized_gemv_amd import qk, synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    qk.load()  # fails loudly if libqk.so is not built
    torch.cuda.set_device(0)
    c = Ctx(torch, qk, synth, oracle, Runner(torch), args)
    t_start = time.perf_counter()
    line, _, _ = run_headline(c)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    if not args.headline_only:
        cfgs = {}
        log("C0 dequantize")
        cfgs["C0_dequant_q4_0_4096x4096_f32"] = run_dequant(c)
        cfgs["C1_gemv_q8_0_4096x4096_n1"] = {"see": "headline (value, ms_per_step, roofline, timing)"}
        log("C2 Q4_1 GEMV n = 1, 2, 4, 8")
        cw = synth.WORKLOADS["gemv_q4_1_11008x4096"]
        res, cpu, keep2 = run_gemv(c, "q4_1", cw["m"], cw["k"], (1, 2, 4, 8), synth.workload_seed(cw["id"]), cw["d"],
                                   cw["mr"], ceiling=True)
        loop = c.run.valu_loop_tflops()
        for n, rec in res.items():
            if rec["roofline"]["bound"] == "alu":
                rec["valu_loop_TFLOPs"] = rnd(loop, 1)
                rec["pct_of_valu_loop"] = rnd(100 * rec["roofline"]["achieved"] / loop, 1)
            cfgs[f"C2_gemv_q4_1_11008x4096_n{n}"] = rec
        cfgs["C2_gemv_q4_1_11008x4096_n8"]["cpu"] = cpu
        log("C3 decode layer")
        cfgs["C3_gemv_q4_0_decode_layer"] = run_layer(c, "gemv_q4_0_decode_layer")
        log("C4 GEMM")
        cfgs["C4_gemm_q4_0_14336x4096_n512"] = run_gemm(c)
        line["configs"] = cfgs
        if not args.quick:
            ext = {}
            log("extras: 8-bit activations")
            res, _, _ = run_gemv(c, "q4_1", cw["m"], cw["k"], (1, 2, 4, 8), synth.workload_seed(cw["id"]), cw["d"],
                                 cw["mr"], entry="mul_mat_vec_x8")
            for n, rec in res.items():
                ext[f"gemv_x8_q4_1_11008x4096_n{n}"] = rec
            log("extras: tensor-parallel share")
            share = run_layer(c, "gemv_q4_0_decode_layer_tp8_share", with_cpu=False)
            ext["gemv_q4_0_decode_layer_tp8_share"] = share
            log("extras: expert-indexed decode")
            ext["gemv_q4_0_moe_experts"] = run_moe(c)
            line["extras"] = ext
    line["bench_wall_s"] = rnd(time.perf_counter() - t_start, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--print-source-hash":
        print(kernel_source_hash(GEMV_SOURCES))
        sys.exit(0)
    main()
