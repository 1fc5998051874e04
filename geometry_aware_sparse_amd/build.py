"""Build the PACK3D HIP library for gfx950 in-tree.

Compiles every csrc/*.hip with hipcc (one process per file, in parallel) and
links geometry_aware_sparse_amd/lib/libpack3d.so. With debug=True (script:
--debug) it builds lib/libpack3d_debug.so instead, the same sources with
PK_DEBUG_BOUNDS defined: every slot-map read is checked against the grid and
reported through the status word (include/pack3d.h). build_all() makes both.
Objects go to _build/ at the repository root.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "pack3d")
LIB = os.path.join(PKG, "lib", "libpack3d.so")
DEBUG_OBJDIR = os.path.join(ROOT, "_build", "pack3d_debug")
DEBUG_LIB = os.path.join(PKG, "lib", "libpack3d_debug.so")
DEBUG_FLAGS = ["-DPK_DEBUG_BOUNDS"]
ARCH = "gfx950"
# Per-file code generation flags.
FILE_FLAGS = {
    # Matrix accumulators in ordinary VGPRs (no AGPR split): the local
    # kernel's pipelined key reads need 155 registers, which fit three waves
    # per SIMD as one file and two as 156 VGPRs + 32 AGPRs.
    "local_tr.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU forms anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _compile(job):
    src, objdir, extra = job
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    return obj, warn


def _link(objs, lib):
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def _build(variants, verbose):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = []
    for objdir, extra, _ in variants:
        os.makedirs(objdir, exist_ok=True)
        jobs += [(src, objdir, extra) for src in srcs]
    # the slowest files first, so that they do not finish the build alone
    jobs.sort(key=lambda j: -os.path.getsize(j[0]))
    nproc = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(nproc) as ex:
        results = dict(zip(jobs, ex.map(_compile, jobs)))
    for _, w in results.values():
        if w.strip() and verbose:
            print(w, file=sys.stderr)
    for objdir, extra, lib in variants:
        _link([results[(src, objdir, extra)][0] for src in srcs], lib)


def build(verbose: bool = False, debug: bool = False) -> str:
    """Build lib/libpack3d.so, or with debug=True lib/libpack3d_debug.so."""
    v = (DEBUG_OBJDIR, tuple(DEBUG_FLAGS), DEBUG_LIB) if debug else (OBJDIR, (), LIB)
    _build([v], verbose)
    return v[2]


def build_all(verbose: bool = False):
    """Build both libraries in one pass over the sources."""
    _build([(OBJDIR, (), LIB), (DEBUG_OBJDIR, tuple(DEBUG_FLAGS), DEBUG_LIB)], verbose)
    return LIB, DEBUG_LIB


if __name__ == "__main__":
    if "--all" in sys.argv:
        print(*build_all(verbose=True))
    else:
        print(build(verbose=True, debug="--debug" in sys.argv))
