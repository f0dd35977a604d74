"""Build libqk.so (the gfx950 HIP kernels behind include/qk.h) in-tree.

Each source is compiled to an object of its own (in parallel, under _build/)
and the objects are linked into dequant_quantized_gemv_amd/libqk.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqk.so")
# The benchmark's helpers (practical-ceiling kernels, the native launch loop
# that times steps of qk calls): a library of their own, linked against
# libqk.so and not part of the qk C ABI.
BENCH_SOURCE = "bench_support.hip"
BENCH_LIB = os.path.join(PKG, "libqk_bench.so")
SOURCES = ["api.hip", "dequant.hip", "gemv.hip", "gemv_n1.hip", "gemv_n2.hip", "gemv_n34.hip",
           "gemv_n56.hip", "gemv_n78.hip", "gemv_id.hip", "gemv_x8_n1.hip", "gemv_x8_n24.hip",
           "gemv_x8_n58.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # every multiply and add is rounded on its own unless written as an fma
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
# Per-source flags.  gemm.hip: MFMA accumulators in VGPRs and updated in place
# (the AGPR form copies all 128 accumulators of a lane every k step).
SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _filter(stderr):
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = _filter(res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False, extra=()):
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, s.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *FLAGS, *SOURCE_FLAGS.get(s, []), *extra, *inc, "-c",
                           os.path.join(CSRC, s), "-o", obj]))
    cobj = os.path.join(OBJ, BENCH_SOURCE.replace(".hip", ".o"))
    cjob = (cobj, [HIPCC, *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, BENCH_SOURCE), "-o", cobj])
    with ThreadPoolExecutor(max_workers=len(jobs) + 1) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs + [cjob]))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs],
          "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", cobj, "-L", PKG, "-l:libqk.so",
          "-Wl,-rpath,$ORIGIN", "-o", BENCH_LIB + ".tmp"], verbose)
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
