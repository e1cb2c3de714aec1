"""Build the HIP library libexl3.so in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled to an object with hipcc (in parallel),
then linked into ``gemm_exl3_linear_amd/libexl3.so``.  The build always runs
from scratch when called (no stale-object reuse).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libexl3.so")
ARCH = os.environ.get("EXL3_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libexl3.so)")


COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: left to its heuristics the backend
    # put the decode GEMV's matrix-core accumulators in AGPRs and copied them
    # back and forth every row step (1116 v_accvgpr moves in that kernel)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}",
]


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), *COMPILE_FLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    return src, p.returncode, p.stdout + p.stderr


CSRC_BENCH = os.path.join(HERE, "csrc_bench")
LIB_BENCH = os.path.join(HERE, "libexl3_bench.so")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Build libexl3.so (the library) and libexl3_bench.so (the benchmark's
    measurement kernels)."""
    _build_lib(CSRC, LIB, verbose, jobs)
    _build_lib(CSRC_BENCH, LIB_BENCH, verbose, jobs)
    return LIB


def _build_lib(src_dir: str, lib_path: str, verbose: bool, jobs: int | None) -> str:
    sources = sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir) if f.endswith(".hip"))
    jobs = jobs or min(len(sources), max(1, min(os.cpu_count() or 1, 16)))
    with tempfile.TemporaryDirectory(prefix="exl3build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in sources]
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_compile, sources, objs))
        failed = [(s, out) for s, rc, out in results if rc != 0]
        for s, rc, out in results:
            if verbose and out.strip():
                print(f"--- {os.path.basename(s)}\n{out}", file=sys.stderr)
        if failed:
            msg = "\n".join(f"--- {os.path.basename(s)}\n{out}" for s, out in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = lib_path + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
        os.replace(tmp_lib, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
