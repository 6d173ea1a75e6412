"""Build libmq.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m nested_int_matmul_amd.build          # or: python nested_int_matmul_amd/build.py

Compiles every source under csrc/ with hipcc and links one shared library
next to this file.  Packed fp32 VALU instructions are disabled for all device
code (-packed-fp32-ops).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmq.so")
PEAKS_LIB = os.path.join(HERE, "libmq_peaks.so")

SOURCES = ["quant_pack.hip", "gemv.hip", "gemm.hip", "gemm_panel.hip", "gemm_big.hip",
           "mixnmatch.hip", "extra.hip", "bitplane.hip", "abi.hip", "gemm_noalloc.hip"]
# measured-peak probes (a library of their own, loaded by bench.py only)
PEAKS_SOURCES = ["peaks.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm 7.x is required to build libmq)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile all sources and link libmq.so and libmq_peaks.so; returns the
    path of libmq.so."""
    _build_lib(SOURCES, LIB, verbose, extra_flags)
    _build_lib(PEAKS_SOURCES, PEAKS_LIB, verbose, extra_flags)
    return LIB


def _build_lib(sources, lib_path, verbose, extra_flags):
    cc = hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    name = os.path.basename(lib_path)
    with tempfile.TemporaryDirectory(prefix="mq_build_") as tmp:
        objs = []
        procs = []
        for src in sources:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            errors = [ln for ln in out.splitlines() if "error" in ln or "warning: " in ln and
                      "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
            if p.returncode != 0:
                failed.append((src, out))
            elif verbose and errors:
                print(out)
        if failed:
            msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
            raise RuntimeError(f"{name} build failed:\n" + msg)
        tmp_lib = os.path.join(tmp, name)
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        shutil.move(tmp_lib, lib_path + ".tmp")
        os.replace(lib_path + ".tmp", lib_path)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
