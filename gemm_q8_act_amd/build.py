"""Build libnvq.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc.

One shared library, gfx950 code objects only.  The flags keep IEEE float
semantics (no fast-math: the Q8_0 division must be correctly rounded) and turn
off packed-fp32 instruction selection.  Each source is compiled to its own object
(in parallel, in a temporary directory), with the per-file compiler options below,
and the objects are linked into the library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libnvq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-file compiler options, by measurement.  q4_1.hip (the Q4-family kernels): without
# the scheduler's "unclustered high register pressure" rescheduling stage the integer-MFMA
# GEMM runs 7 % faster at M = 2048 (146.5 -> 136.4 us at N = K = 4096), IQ4_XS's 4 % at
# M = 512 and Q6_K's two-term GEMM 1.5 %, every other kernel of the file within 0.5 %,
# results bit-identical.  gemv_batch_f16.hip and gemv_nvfp4.hip (decode): the compiler
# raises a wavefront's priority while it issues its loads, so the weight stream starts
# sooner: the 64-layer stack at M = 8 3.0 -> 3.04 TB/s (O 7.5 -> 7.3 us, gate+up 20.8 ->
# 20.3), at M = 1 4.18 -> 4.22 TB/s (fused QKV 6.72 -> 6.63 us, O 6.53 -> 6.42); the same
# option slows the prefill GEMM 2 %.  The other files keep the default schedule.
FILE_FLAGS = {
    "q4_1.hip": ["-mllvm", "-amdgpu-disable-unclustered-high-rp-reschedule"],
    "gemv_batch_f16.hip": ["-mllvm", "-amdgpu-set-wave-priority"],
    "gemv_nvfp4.hip": ["-mllvm", "-amdgpu-set-wave-priority"],
}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(out: str = LIB_PATH, verbose: bool = False, extra_flags=(), jobs: int | None = None) -> str:
    """Compile every HIP source and the C ABI into ``out`` (always rebuilds)."""
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with tempfile.TemporaryDirectory(prefix="nvq_build_") as tmpdir:
        objs, cmds = [], []
        for src in srcs:
            name = os.path.basename(src)
            obj = os.path.join(tmpdir, name + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *FLAGS, *FILE_FLAGS.get(name, []), *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", src,
                         "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
