"""Build libcausalprod.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m prefix_sum_causal_amd.build

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcausalprod.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["cp_api.cpp", "cp_fwd_f32.hip", "cp_fwd_bf16.hip", "cp_fwd_f16.hip", "cp_bwd_f32.hip", "cp_bwd_bf16.hip",
           "cp_bwd_f16.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of the generated code; MFMA results
# stay in ordinary VGPRs (no copies between accumulation registers and VGPRs
# when tiles are converted and fed back as operands).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-command-line-argument"]


# The fp32 forward is compiled without the VGPR form of MFMA: with it, this
# compiler (ROCm 7.2 clang 22) crashes in its AGPR-copy rewrite on one of that
# unit's kernel instances (normalised, E = 128, M = 16).
NO_VGPR_FORM = {"cp_fwd_f32.hip"}


def _compile(src: str, build_dir: str, defines: dict) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    dflags = [f"-D{k}={v}" for k, v in sorted(defines.items())]
    flags = FLAGS
    if src in NO_VGPR_FORM:
        i = flags.index("-amdgpu-mfma-vgpr-form")
        flags = flags[:i - 1] + flags[i + 1:]
    cmd = [HIPCC, *flags, *dflags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines: dict | None = None) -> str:
    """Compile and link the library to ``out``.  ``defines`` overrides the
    tuning macros of cp_tune.hpp (e.g. {"CP_BF16_NBUF": 4})."""
    defines = dict(defines or {})
    build_dir = BUILD_DIR if not defines else os.path.join(BUILD_DIR, "_".join(f"{k}{v}" for k, v in
                                                                               sorted(defines.items())))
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(os.cpu_count() or 1, 8)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
