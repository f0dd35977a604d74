"""Benchmark of the quantized GEMV hot path on one MI355X.

Default workload: Q8_0 GEMV, W 4096 x 4096 times one fp32 activation column
(x ~ N(0,1)), y = W x in fp32.  A step is one qk_mul_mat_vec call: block
decode, fused dequantize + dot products, wave/workgroup reduction, dispatch.

Measurement
  * Inputs live in HBM before the timed region.  Every working set here fits
    in the 256 MB Infinity Cache, so the benchmark rotates through R copies of
    the weights (R * |W| >= 1 GiB): launch i reads copy i % R, which is never
    cache-resident.
  * Launches are captured into a HIP graph (torch.cuda.CUDAGraph) so host
    launch overhead is out of the way; the timed region is one replay of K
    launches, bracketed by synchronization, timed with HIP events recorded on
    the stream the kernels run on.
  * Before timing, the output is checked against the CPU oracle (every row).
  * metric value = weight bytes per launch * K / elapsed  (effective weight GB/s)
  * roofline.achieved = algorithmic bytes per launch (W + x + y) / average
    launch time; peak = 8 TB/s HBM.
  * cpu_baseline: the oracle (plain C, fp64, one thread) on the same matrix.
  * practical_ceiling: a plain streaming-read kernel (libqk_ceiling.so) over
    the same weight bytes, same rotation and launch pattern; --configs adds
    it per GEMV workload and an MFMA-only loop for the GEMM.

Options: --workload NAME runs another single-GEMV workload as the headline;
--configs also measures every workload and adds them under "configs".
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
GEMV_SOURCES = ["gemv.hip", "gemv.h", "gemv_impl.h", "gemv_n1.hip", "qk_common.h",
                "qk_internal.h"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def load_ceiling():
    """The practical-ceiling kernels (libqk_ceiling.so, built with libqk)."""
    path = os.path.join(ROOT, "dequant_quantized_gemv_amd", "libqk_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.qkc_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.qkc_stream_read.restype = ctypes.c_int
    lib.qkc_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.qkc_mfma_loop.restype = ctypes.c_int
    return lib


def stream_read_time(torch, timer, clib, ptrs, nbytes, steps, warmup):
    """Seconds per streaming read of nbytes, launch i reading ptrs[i % len]
    (the same cold rotation as the kernel it is compared with)."""
    sink = torch.zeros(4, device="cuda")
    R = len(ptrs)

    def rd(i):
        if clib.qkc_stream_read(ptrs[i % R], nbytes, sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("qkc_stream_read failed")

    gw, gk = timer.capture(rd, max(warmup, 1)), timer.capture(lambda i: rd(i + warmup), steps)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / steps
    del gw, gk
    return sec


def mfma_loop_tflops(torch, timer, clib):
    """fp16 MFMA rate of a register-only loop over every CU (TFLOP/s)."""
    sink = torch.zeros(4, device="cuda")
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4000

    def run(i):
        if clib.qkc_mfma_loop(wgs, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("qkc_mfma_loop failed")

    gw, gk = timer.capture(run, 2), timer.capture(run, 5)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / 5
    return wgs * 8 * iters * 32 * (2.0 * 16 * 16 * 32) / sec / 1e12


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


class Timer:
    """Graph-captured launches timed with HIP events on the launch stream."""

    def __init__(self, torch):
        self.t = torch

    def capture(self, fn, count):
        t = self.t
        g = t.cuda.CUDAGraph()
        s = t.cuda.Stream()
        s.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(s):
            with t.cuda.graph(g, stream=s):
                for i in range(count):
                    fn(i)
        t.cuda.current_stream().wait_stream(s)
        t.cuda.synchronize()
        return g

    def time_graph(self, g):
        t = self.t
        t.cuda.synchronize()
        st = t.cuda.current_stream()
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # seconds


def copies_for(nbytes, minimum=2):
    return max(minimum, math.ceil(COLD_BYTES / max(nbytes, 1)))


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def setup_gemv(torch, qk, synth, oracle, fmt, m, k, n, seed, wtid, xtid, d, mr=None,
               check="full", rng_seed=0):
    """Device copies of one GEMV problem plus the parity check of one launch."""
    w = synth.quant_matrix(fmt, m, k, seed=seed, tensor_id=wtid, d_range=d,
                           **({"m_range": mr} if mr else {}))
    x = synth.activations(k, 8 if n > 1 else 1, seed=seed, tensor_id=xtid)[:n]
    wd = torch.from_numpy(w).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = torch.empty((n, m), dtype=torch.float32, device="cuda")
    qk.mul_mat_vec(fmt, wd, m, k, xd, y=y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().astype(np.float64)
    if check == "none":
        return dict(w=w, x=x, wd=wd, xd=xd, y=y, ok=True, worst=0.0)
    if check == "full":
        yr, s = oracle.dot(fmt, w, m, k, x, n)
        ok = bool(np.all(np.abs(yh - yr) <= 1e-4 * s))
        worst = float(np.max(np.abs(yh - yr) / np.where(s > 0, s, 1)))
    else:
        rng = np.random.default_rng(rng_seed)
        ii = rng.integers(0, m, size=256)
        jj = rng.integers(0, n, size=256)
        yr, s = oracle.dot_entries(fmt, w, m, k, x.ravel(), k, ii, jj)
        got = yh[jj, ii]
        ok = bool(np.all(np.abs(got - yr) <= 1e-4 * s))
        worst = float(np.max(np.abs(got - yr) / np.where(s > 0, s, 1)))
    return dict(w=w, x=x, wd=wd, xd=xd, y=y, ok=ok, worst=worst)


def gemv_bytes(fmt, m, k, n):
    bs = {"q4_0": 18, "q4_1": 20, "q8_0": 34}[fmt]
    wb = m * (k // 32) * bs
    return wb, wb + 4 * n * (k + m)


def bench_gemv(torch, qk, timer, prob, fmt, m, k, n, steps, warmup, entry="qk_mul_mat_vec",
               clib=None):
    wb, algo = gemv_bytes(fmt, m, k, n)
    R = copies_for(wb)
    copies = [prob["wd"]] + [prob["wd"].clone() for _ in range(R - 1)]
    xd, y = prob["xd"], prob["y"]
    lib = qk.load()
    code = qk.FORMATS[fmt]
    ptrs = [c.data_ptr() for c in copies]
    xp, yp = xd.data_ptr(), y.data_ptr()

    call = getattr(lib, entry)

    def launch(i):
        st = call(code, ptrs[i % R], m, k, xp, n, k, yp, m, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"{entry}: {qk.status_string(st)}")

    gw = timer.capture(launch, max(warmup, 1))
    gk = timer.capture(lambda i: launch(i + warmup), steps)
    timer.time_graph(gw)
    sec = timer.time_graph(gk)
    del gw, gk
    out = dict(seconds=sec, per_launch_s=sec / steps, weight_bytes=wb, algo_bytes=algo, copies=R)
    if clib is not None:
        # the same bytes streamed by a plain read kernel, same rotation
        out["stream_read_s"] = stream_read_time(torch, timer, clib, ptrs, wb, steps, warmup)
    del copies
    return out


def cpu_baseline_gemv(oracle, prob, fmt, m, k, n, budget_s=10.0):
    wb, _ = gemv_bytes(fmt, m, k, n)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.dot(fmt, prob["w"], m, k, prob["x"], n)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= 200:
            break
    return dict(value=round(wb * passes / el / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"full {m}x{k} {fmt} matrix x {n} column(s), {passes} passes, "
                       f"{el:.1f} s, one thread")


def run_headline(torch, qk, synth, oracle, timer, name, steps, warmup, with_cpu, clib):
    cfg = synth.WORKLOADS[name]
    seed = synth.workload_seed(cfg["id"])
    fmt = cfg["fmt"]
    if "layer" in cfg or name.startswith("dequant") or name.startswith("gemm"):
        raise SystemExit(f"--workload {name}: the headline is a single GEMV; use --configs")
    n = cfg["n"] if isinstance(cfg["n"], int) else cfg["n"][0]
    m, k = cfg["m"], cfg["k"]
    prob = setup_gemv(torch, qk, synth, oracle, fmt, m, k, n, seed, 0, 100, cfg["d"],
                      cfg.get("mr"))
    if not prob["ok"]:
        raise SystemExit(f"parity check failed before timing (max err/S {prob['worst']:.3g})")
    log(f"parity ok: max |y-ref|/S = {prob['worst']:.3g}")
    r = bench_gemv(torch, qk, timer, prob, fmt, m, k, n, steps, warmup, clib=clib)
    gbps = r["weight_bytes"] * steps / r["seconds"] / 1e9
    achieved = r["algo_bytes"] / r["per_launch_s"] / 1e9
    traffic = stored_traffic(f"gemv_{fmt}_{m}x{k}_n{n}", GEMV_SOURCES)
    out = {
        "metric": "effective weight GB/s (% of HBM peak) for Q4_0/Q8_0 GEMV; batched TFLOP/s",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["seconds"] * 1e3 / steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "format": fmt, "m": m, "k": k, "n": n,
                   "cold_weight_copies": r["copies"], "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        # a plain streaming read of the same weight bytes (same cold rotation,
        # same launch pattern): the practical ceiling on this chip
        "practical_ceiling": {"stream_read_us": round(r["stream_read_s"] * 1e6, 3),
                              "stream_read_GBps": round(r["weight_bytes"] / r["stream_read_s"] / 1e9, 1),
                              "frac_of_stream_read": round(r["stream_read_s"] / r["per_launch_s"], 4)},
    }
    if with_cpu:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline_gemv(oracle, prob, fmt, m, k, n)
    return out


def run_configs(torch, qk, synth, oracle, timer, steps, warmup, clib):
    """Every workload, each parity-checked before it is timed."""
    res = {}
    # C0: dequantize Q4_0 4096x4096 -> fp32
    cfg = synth.WORKLOADS["dequant_q4_0_4096x4096_f32"]
    seed = synth.workload_seed(cfg["id"])
    m, k = cfg["m"], cfg["k"]
    w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=0, d_range=cfg["d"])
    wd = torch.from_numpy(w).cuda()
    out = qk.dequantize("q4_0", wd, m, k, "f32")
    ok = np.array_equal(out.cpu().numpy().view(np.uint32),
                        oracle.dequantize_f32("q4_0", w, m, k).view(np.uint32))
    inb, outb = w.size, m * k * 4
    R = copies_for(inb + outb)
    ins = [wd] + [wd.clone() for _ in range(R - 1)]
    outs = [out] + [torch.empty_like(out) for _ in range(R - 1)]
    lib = qk.load()

    def dq(i):
        lib.qk_dequantize(qk.QK_Q4_0, ins[i % R].data_ptr(), m, k, qk.QK_F32,
                          outs[i % R].data_ptr(), torch.cuda.current_stream().cuda_stream)

    st = max(steps // 4, 20)
    gw, gk = timer.capture(dq, warmup), timer.capture(lambda i: dq(i + warmup), st)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / st
    res["dequant_q4_0_4096x4096_f32"] = {
        "parity": "bit-exact" if ok else "FAILED", "us_per_launch": round(sec * 1e6, 3),
        "total_GBps": round((inb + outb) / sec / 1e9, 1),
        "weight_GBps": round(inb / sec / 1e9, 1),
        "pct_of_hbm_peak": round(100 * (inb + outb) / sec / 1e9 / HBM_PEAK_GBPS, 1)}
    del ins, outs, gw, gk

    # C1 and C2: single GEMVs
    for name, ns in (("gemv_q8_0_4096x4096_n1", (1,)), ("gemv_q4_1_11008x4096", (1, 2, 4, 8))):
        cfg = synth.WORKLOADS[name]
        seed = synth.workload_seed(cfg["id"])
        for n in ns:
            prob = setup_gemv(torch, qk, synth, oracle, cfg["fmt"], cfg["m"], cfg["k"], n, seed, 0,
                              100, cfg["d"], cfg.get("mr"), check="sampled", rng_seed=n)
            r = bench_gemv(torch, qk, timer, prob, cfg["fmt"], cfg["m"], cfg["k"], n, steps, warmup,
                           clib=clib)
            gbps = r["weight_bytes"] / r["per_launch_s"] / 1e9
            res[f"{name}" + ("" if len(ns) == 1 else f"_n{n}")] = {
                "parity": "ok" if prob["ok"] else "FAILED", "max_err_over_S": prob["worst"],
                "us_per_launch": round(r["per_launch_s"] * 1e6, 3),
                "weight_GBps": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
                "stream_read_us": round(r["stream_read_s"] * 1e6, 3),
                "pct_of_stream_read": round(100 * r["stream_read_s"] / r["per_launch_s"], 1)}
            del prob

    # C2 again with 8-bit activations (qk_mul_mat_vec_x8), checked against the
    # oracle's product with the same quantized activations
    cfg = synth.WORKLOADS["gemv_q4_1_11008x4096"]
    seed = synth.workload_seed(cfg["id"])
    for n in (1, 2, 4, 8):
        prob = setup_gemv(torch, qk, synth, oracle, "q4_1", cfg["m"], cfg["k"], n, seed, 0, 100,
                          cfg["d"], cfg.get("mr"), check="none")
        y8 = qk.mul_mat_vec_x8("q4_1", prob["wd"], cfg["m"], cfg["k"], prob["xd"])
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(n).choice(cfg["m"], 128, replace=False))
        rb = (cfg["k"] // 32) * 20
        wsub = np.concatenate([prob["w"][r * rb:(r + 1) * rb] for r in rows])
        yr, sr = oracle.dot_x8("q4_1", wsub, len(rows), cfg["k"], prob["x"], n)
        got = y8.cpu().numpy()[:, rows].astype(np.float64)
        ok8 = bool(np.all(np.abs(got - yr) <= 1e-4 * sr))
        r = bench_gemv(torch, qk, timer, prob, "q4_1", cfg["m"], cfg["k"], n, steps, warmup,
                       entry="qk_mul_mat_vec_x8")
        gbps = r["weight_bytes"] / r["per_launch_s"] / 1e9
        res[f"gemv_q4_1_11008x4096_x8_n{n}"] = {
            "parity": "ok" if ok8 else "FAILED", "us_per_launch": round(r["per_launch_s"] * 1e6, 3),
            "weight_GBps": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
        del prob

    # C3: the decode layer, 7 GEMVs per step (from a clean allocator: weight
    # copies carved out of the previous workloads' freed blocks measured
    # slower than fresh allocations)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    cfg = synth.WORKLOADS["gemv_q4_0_decode_layer"]
    seed = synth.workload_seed(cfg["id"])
    probs, wtot = [], 0
    for tid, (nm, m, k) in enumerate(cfg["layer"]):
        p = setup_gemv(torch, qk, synth, oracle, "q4_0", m, k, 1, seed, tid, 100 + tid, cfg["d"],
                       check="sampled", rng_seed=tid)
        p.update(m=m, k=k)
        probs.append(p)
        wtot += gemv_bytes("q4_0", m, k, 1)[0]
    R = copies_for(wtot)
    layer_copies = [[p["wd"]] + [p["wd"].clone() for _ in range(R - 1)] for p in probs]

    def layer(i):
        s = torch.cuda.current_stream().cuda_stream
        for p, cps in zip(probs, layer_copies):
            lib.qk_mul_mat_vec(qk.QK_Q4_0, cps[i % R].data_ptr(), p["m"], p["k"], p["xd"].data_ptr(),
                               1, p["k"], p["y"].data_ptr(), p["m"], s)

    st = max(steps // 7, 20)
    gw, gk = timer.capture(layer, warmup), timer.capture(lambda i: layer(i + warmup), st)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / st
    del gw, gk

    # the same layer as one grouped launch (qk_mul_mat_vec_batched)
    item_sets = [qk.make_items([(cps[r].data_ptr(), p["m"], p["k"], p["xd"].data_ptr(), p["k"],
                                 p["y"].data_ptr(), p["m"]) for p, cps in zip(probs, layer_copies)])
                 for r in range(R)]

    def grouped(i):
        lib.qk_mul_mat_vec_batched(qk.QK_Q4_0, item_sets[i % R], len(probs), 1,
                                   torch.cuda.current_stream().cuda_stream)

    grouped(0)
    torch.cuda.synchronize()
    gok = True
    for tid, p in enumerate(probs):
        rng = np.random.default_rng(200 + tid)
        ii = rng.integers(0, p["m"], 128)
        yr, sr = oracle.dot_entries("q4_0", p["w"], p["m"], p["k"], p["x"].ravel(), p["k"], ii,
                                    np.zeros_like(ii))
        got = p["y"].cpu().numpy()[0, ii].astype(np.float64)
        gok = gok and bool(np.all(np.abs(got - yr) <= 1e-4 * sr))
    gw, gk = timer.capture(grouped, warmup), timer.capture(lambda i: grouped(i + warmup), st)
    timer.time_graph(gw)
    secg = timer.time_graph(gk) / st
    # a streaming read of the layer's weight bytes as one buffer per copy
    flat = [torch.empty(wtot, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sr = stream_read_time(torch, timer, clib, [f.data_ptr() for f in flat], wtot, st, warmup)
    del flat
    res["gemv_q4_0_decode_layer"] = {
        "parity": "ok" if all(p["ok"] for p in probs) and gok else "FAILED",
        "separate_launches": {"us_per_layer": round(sec * 1e6, 3), "weight_GBps": round(wtot / sec / 1e9, 1),
                              "pct_of_hbm_peak": round(100 * wtot / sec / 1e9 / HBM_PEAK_GBPS, 1)},
        "grouped_launch": {"us_per_layer": round(secg * 1e6, 3), "weight_GBps": round(wtot / secg / 1e9, 1),
                           "pct_of_hbm_peak": round(100 * wtot / secg / 1e9 / HBM_PEAK_GBPS, 1),
                           "stream_read_us": round(sr * 1e6, 3),
                           "pct_of_stream_read": round(100 * sr / secg, 1)}}
    del probs, layer_copies, gw, gk, item_sets

    # C4: GEMM
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    cfg = synth.WORKLOADS["gemm_q4_0_14336x4096_n512"]
    seed = synth.workload_seed(cfg["id"])
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    w = synth.quant_matrix("q4_0", m, k, seed=seed, tensor_id=0, d_range=cfg["d"])
    xh = synth.activations(k, n, seed=seed, tensor_id=100, dtype=np.float16)
    wd = torch.from_numpy(w).cuda()
    xd = torch.from_numpy(xh).cuda()
    y = qk.mul_mat("q4_0", wd, m, k, xd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    ii, jj = rng.integers(0, m, 256), rng.integers(0, n, 256)
    yr, s = oracle.dot_entries("q4_0", w, m, k, xh.view(np.uint16).ravel(), k, ii, jj, x_is_f16=True)
    got = y.cpu().numpy()[jj, ii].astype(np.float64)
    ok = bool(np.all(np.abs(got - yr) <= 1e-2 * s))
    R = copies_for(w.size, minimum=4)
    wc = [wd] + [wd.clone() for _ in range(R - 1)]

    def gm(i):
        lib.qk_mul_mat(qk.QK_Q4_0, wc[i % R].data_ptr(), m, k, xd.data_ptr(), n, k, y.data_ptr(), m,
                       torch.cuda.current_stream().cuda_stream)

    st = max(steps // 20, 20)
    gw, gk = timer.capture(gm, max(warmup // 10, 2)), timer.capture(gm, st)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / st
    tf = 2.0 * m * n * k / sec / 1e12
    loop_tf = mfma_loop_tflops(torch, timer, clib)
    res["gemm_q4_0_14336x4096_n512"] = {
        "parity": "ok" if ok else "FAILED", "us_per_launch": round(sec * 1e6, 2),
        "TFLOPs": round(tf, 1), "pct_of_mfma_f16_peak": round(100 * tf / MFMA_F16_PEAK_TFLOPS, 1),
        "mfma_loop_TFLOPs": round(loop_tf, 1), "pct_of_mfma_loop": round(100 * tf / loop_tf, 1)}
    del gw, gk

    # the same weights at smaller batches (the first nb activation columns):
    # up to 128 columns there is one column tile, so 56 workgroups for 256 CUs
    batches = {}
    for nb in (16, 64, 128):
        yb = torch.empty((nb, m), dtype=torch.float32, device="cuda")

        def gmb(i, nb=nb, yb=yb):
            lib.qk_mul_mat(qk.QK_Q4_0, wc[i % R].data_ptr(), m, k, xd.data_ptr(), nb, k, yb.data_ptr(), m,
                           torch.cuda.current_stream().cuda_stream)

        gmb(0)
        torch.cuda.synchronize()
        jb = rng.integers(0, nb, 128)
        ib = rng.integers(0, m, 128)
        yr, s = oracle.dot_entries("q4_0", w, m, k, xh.view(np.uint16).ravel(), k, ib, jb, x_is_f16=True)
        okb = bool(np.all(np.abs(yb.cpu().numpy()[jb, ib].astype(np.float64) - yr) <= 1e-2 * s))
        gw, gk = timer.capture(gmb, max(warmup // 10, 2)), timer.capture(gmb, st)
        timer.time_graph(gw)
        secb = timer.time_graph(gk) / st
        batches[str(nb)] = {"parity": "ok" if okb else "FAILED", "us_per_launch": round(secb * 1e6, 2),
                            "TFLOPs": round(2.0 * m * nb * k / secb / 1e12, 1)}
        del gw, gk, yb
    res["gemm_q4_0_14336x4096_n512"]["smaller_batches"] = batches
    del wc

    log("decode layer, one GPU's share of 8-way tensor parallelism")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res["gemv_q4_0_decode_layer_tp8_share"] = run_share_layer(torch, qk, synth, oracle, timer, steps,
                                                              warmup)

    log("expert-indexed decode")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res["gemv_q4_0_moe_experts"] = run_moe(torch, qk, synth, oracle, timer, steps, warmup)
    return res


def run_share_layer(torch, qk, synth, oracle, timer, steps, warmup):
    """One GPU's share of the decode layer under 8-way tensor parallelism (row
    shards of q, k, v, gate, up; K shards of o and down): the GEMVs of one
    token as one grouped launch and as separate launches.  The all-reduce of
    the K-shard partial sums is not part of it (one GPU)."""
    cfg = synth.WORKLOADS["gemv_q4_0_decode_layer_tp8_share"]
    seed = synth.workload_seed(cfg["id"])
    lib = qk.load()
    probs, wtot = [], 0
    for tid, (nm, m, k) in enumerate(cfg["layer"]):
        p = setup_gemv(torch, qk, synth, oracle, "q4_0", m, k, 1, seed, tid, 100 + tid, cfg["d"])
        p.update(m=m, k=k)
        probs.append(p)
        wtot += gemv_bytes("q4_0", m, k, 1)[0]
    R = copies_for(wtot)
    copies = [[p["wd"]] + [p["wd"].clone() for _ in range(R - 1)] for p in probs]
    sets = [qk.make_items([(cps[r].data_ptr(), p["m"], p["k"], p["xd"].data_ptr(), p["k"],
                            p["y"].data_ptr(), p["m"]) for p, cps in zip(probs, copies)])
            for r in range(R)]

    def grouped(i):
        lib.qk_mul_mat_vec_batched(qk.QK_Q4_0, sets[i % R], len(probs), 1,
                                   torch.cuda.current_stream().cuda_stream)

    def separate(i):
        s = torch.cuda.current_stream().cuda_stream
        for p, cps in zip(probs, copies):
            lib.qk_mul_mat_vec(qk.QK_Q4_0, cps[i % R].data_ptr(), p["m"], p["k"], p["xd"].data_ptr(),
                               1, p["k"], p["y"].data_ptr(), p["m"], s)

    grouped(0)
    torch.cuda.synchronize()
    ok = all(p["ok"] for p in probs)
    for p in probs:
        yr, sr = oracle.dot("q4_0", p["w"], p["m"], p["k"], p["x"], 1)
        got = p["y"].cpu().numpy().astype(np.float64)
        ok = ok and bool(np.all(np.abs(got - yr) <= 1e-4 * sr))
    out = {"parity": "ok" if ok else "FAILED", "weight_bytes": wtot}
    st = max(steps // 4, 20)
    for name, fn in (("grouped_launch", grouped), ("separate_launches", separate)):
        gw, gk = timer.capture(fn, warmup), timer.capture(lambda i: fn(i + warmup), st)
        timer.time_graph(gw)
        sec = timer.time_graph(gk) / st
        del gw, gk
        out[name] = {"us_per_layer": round(sec * 1e6, 3), "weight_GBps": round(wtot / sec / 1e9, 1),
                     "pct_of_hbm_peak": round(100 * wtot / sec / 1e9 / HBM_PEAK_GBPS, 1)}
    return out


def run_moe(torch, qk, synth, oracle, timer, steps, warmup):
    """Expert-indexed decode: per token, the gate, up and down projections of
    8 of 128 Q4_0 experts (768 x 2048, 768 x 2048, 2048 x 768), three
    qk_mul_mat_vec_id calls; and the same with gate and up merged per expert
    (two calls).  Expert choices change every step and the stacks rotate over
    copies, so the experts a step reads are never cache-resident."""
    cfg = synth.WORKLOADS["gemv_q4_0_moe_experts"]
    seed = synth.workload_seed(cfg["id"])
    ne, nu, nt = cfg["n_experts"], cfg["n_used"], cfg["n_tokens"]
    lib = qk.load()
    stacks, ok = [], True
    for tid, (nm, m, k) in enumerate(cfg["layer"]):
        w = synth.quant_matrix("q4_0", ne * m, k, seed=seed, tensor_id=tid, d_range=cfg["d"])
        shared = nm != "down"
        # gate and up read the same hidden state; down one vector per slot
        xtid = 100 if shared else 100 + tid
        x = synth.activations(k, nt * (1 if shared else nu), seed=seed, tensor_id=xtid)
        stacks.append(dict(nm=nm, m=m, k=k, w=w, wd=torch.from_numpy(w).cuda(), x=x,
                           xd=torch.from_numpy(np.ascontiguousarray(x)).cuda(), shared=shared,
                           y=torch.empty((nt, nu, m), dtype=torch.float32, device="cuda"),
                           one=m * (k // 32) * 18))
    n_sets = 64
    ids = np.stack([synth.expert_ids(nt, nu, ne, seed=seed, tensor_id=50 + i) for i in range(n_sets)])
    ids_d = torch.from_numpy(ids).cuda()
    sel_bytes = sum(nt * nu * p["one"] for p in stacks)
    R = copies_for(sum(p["w"].size for p in stacks))
    for p in stacks:
        p["copies"] = [p["wd"]] + [p["wd"].clone() for _ in range(R - 1)]

    def call(p, wptr, idp):
        x_slot = 0 if p["shared"] else p["k"]
        x_tok = p["k"] if p["shared"] else nu * p["k"]
        return lib.qk_mul_mat_vec_id(qk.QK_Q4_0, wptr, ne, p["one"], p["m"],
                                     p["k"], idp, nu, nu, nt, p["xd"].data_ptr(), x_slot, x_tok,
                                     p["y"].data_ptr(), p["m"], nu * p["m"],
                                     torch.cuda.current_stream().cuda_stream)

    def layer(i):
        idp = ids_d[i % n_sets].data_ptr()
        for p in stacks:
            st = call(p, p["copies"][i % R].data_ptr(), idp)
            if st != 0:
                raise RuntimeError(f"qk_mul_mat_vec_id: {qk.status_string(st)}")

    layer(0)
    torch.cuda.synchronize()
    worst = 0.0
    for p in stacks:
        xs = p["x"].reshape(nt, p["k"]) if p["shared"] else p["x"].reshape(nt, nu, p["k"])
        yr, sr = oracle.dot_id("q4_0", p["w"], ne, p["one"], p["m"], p["k"], ids[0], nu, nt, xs,
                               0 if p["shared"] else p["k"], p["k"] if p["shared"] else nu * p["k"])
        got = p["y"].cpu().numpy().astype(np.float64)
        ok = ok and bool(np.all(np.abs(got - yr) <= 1e-4 * sr))
        worst = max(worst, float(np.max(np.abs(got - yr) / np.where(sr > 0, sr, 1))))
    st = max(steps // 3, 20)
    gw, gk = timer.capture(layer, warmup), timer.capture(lambda i: layer(i + warmup), st)
    timer.time_graph(gw)
    sec = timer.time_graph(gk) / st
    del gw, gk
    out = {"parity": "ok" if ok else "FAILED", "max_err_over_S": worst,
           "us_per_token": round(sec * 1e6, 3), "launches_per_token": len(stacks),
           "selected_weight_bytes": sel_bytes,
           "weight_GBps": round(sel_bytes / sec / 1e9, 1),
           "pct_of_hbm_peak": round(100 * sel_bytes / sec / 1e9 / HBM_PEAK_GBPS, 1)}

    # the same weights with gate and up merged per expert (one 1536 x 2048
    # matrix an expert: gate rows, then up rows), so one call covers both
    gate, up, down = stacks
    mg = gate["m"] + up["m"]
    layer(0)
    torch.cuda.synchronize()
    ref_gate, ref_up = gate["y"].clone(), up["y"].clone()
    gate["copies"] = up["copies"] = None
    gate["wd"] = up["wd"] = None
    torch.cuda.empty_cache()
    merged = np.concatenate([gate["w"].reshape(ne, -1), up["w"].reshape(ne, -1)], axis=1).ravel()
    md = torch.from_numpy(merged).cuda()
    mcopies = [md] + [md.clone() for _ in range(R - 1)]
    ym = torch.empty((nt, nu, mg), dtype=torch.float32, device="cuda")
    one_m = mg * (gate["k"] // 32) * 18

    def merged_layer(i):
        s = torch.cuda.current_stream().cuda_stream
        idp = ids_d[i % n_sets].data_ptr()
        st1 = lib.qk_mul_mat_vec_id(qk.QK_Q4_0, mcopies[i % R].data_ptr(), ne, one_m, mg, gate["k"],
                                    idp, nu, nu, nt, gate["xd"].data_ptr(), 0, gate["k"],
                                    ym.data_ptr(), mg, nu * mg, s)
        st2 = call(down, down["copies"][i % R].data_ptr(), idp)
        if st1 != 0 or st2 != 0:
            raise RuntimeError("qk_mul_mat_vec_id failed")

    merged_layer(0)
    torch.cuda.synchronize()
    # the merged call's rows are the separate calls' outputs, bit for bit
    same = bool(torch.equal(ym[:, :, :gate["m"]], ref_gate) and torch.equal(ym[:, :, gate["m"]:], ref_up))
    gw, gk = timer.capture(merged_layer, warmup), timer.capture(lambda i: merged_layer(i + warmup), st)
    timer.time_graph(gw)
    secm = timer.time_graph(gk) / st
    del gw, gk, mcopies
    out["merged_gate_up"] = {"parity": "bitwise equal to separate calls" if same else "FAILED",
                             "us_per_token": round(secm * 1e6, 3), "launches_per_token": 2,
                             "weight_GBps": round(sel_bytes / secm / 1e9, 1),
                             "pct_of_hbm_peak": round(100 * sel_bytes / secm / 1e9 / HBM_PEAK_GBPS, 1)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="gemv_q8_0_4096x4096_n1")
    ap.add_argument("--configs", action="store_true", help="also measure every workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import oracle
    from dequant_quantized_gemv_amd import qk, synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    qk.load()  # fails loudly if libqk.so is not built
    clib = load_ceiling()
    torch.cuda.set_device(0)
    timer = Timer(torch)
    out = run_headline(torch, qk, synth, oracle, timer, args.workload, args.steps, args.warmup,
                       not args.no_cpu, clib)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    if args.configs:
        log("measuring every workload")
        out["configs"] = run_configs(torch, qk, synth, oracle, timer, args.steps, args.warmup, clib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--print-source-hash":
        print(kernel_source_hash(GEMV_SOURCES))
        sys.exit(0)
    main()
