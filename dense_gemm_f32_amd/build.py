"""Build libmgemm.so (HIP, gfx950) in-tree.

Every translation unit under csrc/ is compiled with hipcc for gfx950 into
_build/, in parallel, then linked into dense_gemm_f32_amd/libmgemm.so.  The
benchmark's measurement aids under diag/ go into libmgemm_diag.so.  The same
csrc/ sources built with -DMGEMM_DEBUG_POISON (objects in _build/poison/) make
libmgemm_poison.so, the LDS race-check build that a GPU test runs.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
DIAG = os.path.join(PKG, "diag")
DIAG_LIB = os.path.join(PKG, "libmgemm_diag.so")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmgemm.so")
POISON_LIB = os.path.join(PKG, "libmgemm_poison.so")
POISON_FLAGS = ["-DMGEMM_DEBUG_POISON"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # compiler-formed packed fp32 arithmetic stays off (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra, objdir: str = BUILD) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), jobs: int | None = None, poison: bool = True) -> str:
    """Compile and link libmgemm.so, libmgemm_diag.so and (poison=True) the race-check
    build libmgemm_poison.so; returns the first one's path.  Always rebuilds."""
    poison_dir = os.path.join(BUILD, "poison")
    os.makedirs(poison_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    diag = sorted(glob.glob(os.path.join(DIAG, "*.hip")))
    units = [(s, list(extra_flags), BUILD) for s in srcs + diag]
    if poison:
        units += [(s, list(extra_flags) + POISON_FLAGS, poison_dir) for s in srcs]
    # the largest translation units first, so that they do not finish last
    order = sorted(range(len(units)), key=lambda i: -os.path.getsize(units[i][0]))
    jobs = jobs or min(len(units), os.cpu_count() or 4, 16)
    objs = [None] * len(units)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, *units[i]): i for i in order}
        for f in concurrent.futures.as_completed(futs):
            objs[futs[f]] = f.result()
    n, d = len(srcs), len(diag)
    _link(objs[:n], LIB)
    if diag:
        _link(objs[n:n + d], DIAG_LIB)
    if poison:
        _link(objs[n + d:], POISON_LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
